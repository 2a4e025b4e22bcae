"""The bounds-checking debug build (libultragen_debug.so, include/ultragen_debug.h)
on the small parity workloads and the edge cases: every kernel's index
checks (work items, tasks, key and query ranges, store destinations,
permutation-table values, warm-start patch indices) must pass, and the
outputs must be bit-identical to the release build's on the same inputs.

The checks record a failure in a device word instead of trapping, so a
failing case ends normally and the test reports which check fired.
"""
import numpy as np
import pytest

import workloads as WL
from tests.gpu_util import qkv_device, to_device, to_host_storage

pytestmark = pytest.mark.gpu

FORWARD = ["tiny", "tiny_masked", "small_ragged", "small_d64", "small_ragged_corr", "ragged_corr_f32",
           "small_f32_d128", "1k"]
EDGE = {
    "no_lr": ("small_ragged", dict(lr_h=0, lr_w=0)),
    "no_text_no_lr": ("small_ragged", dict(n_text=0, lr_h=0, lr_w=0)),
    "radius2": ("small_ragged", dict(radius=2)),
    "window8": ("small_ragged", dict(window=8)),
    "one_text": ("small_ragged", dict(n_text=1)),
    "batch2": ("small_ragged", dict(batch=2)),
}
BACKWARD = ["small_ragged", "small_d64", "small_ragged_corr"]
WARM = {"base": {}, "rho1": dict(rho=1, lr_h=40, lr_w=36), "rho8": dict(rho=8, lr_h=5, lr_w=5),
        "rho16": dict(rho=16, lr_h=3, lr_w=3), "bf16_c72": dict(dtype="bf16", channels=72)}


@pytest.fixture(scope="module")
def U():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import diffusion_transformer_sparse_amd as U
    yield U
    U.use_library(U.LIB_PATH)


def _forward(U, w, train=None):
    """The fused and the unfused forward path, and (bf16 workloads of
    BACKWARD, or train=True) the training layer's forward with LSE and its
    backward; returns every output as host storage."""
    import torch
    plan = U.ug_plan(U.desc_of(w))
    q, k, v = qkv_device(w)
    outs = {}
    outs["fused"] = U.ug_attn_fwd_raster(plan, *U.ug_permute_rope(plan, q, k), U.ug_permute(plan, v))
    qp, kp, vp = U.ug_permute(plan, q), U.ug_permute(plan, k), U.ug_permute(plan, v)
    U.ug_rope2d(plan, qp, kp)
    outs["unfused"] = U.ug_unpermute(plan, U.ug_attn_fwd(plan, qp, kp, vp))
    if w.dtype == "bf16" and (w.name in BACKWARD if train is None else train):
        d_o = to_device(WL.tensor_storage(w, WL.DO), w.dtype)
        train = U.TrainLayer(plan, q.device)
        o = torch.empty_like(q)
        train.forward(q, k, v, o)
        grads = [torch.empty_like(q) for _ in range(3)]
        train.backward(d_o, *grads)
        outs["train_o"], outs["lse"] = o, train.lse
        outs["dq"], outs["dk"], outs["dv"] = grads
    torch.cuda.synchronize()
    return {n: to_host_storage(t, w.dtype) if t.dtype != torch.float32 or w.dtype == "f32" else t.cpu().numpy()
            for n, t in outs.items()}


def _both(U, run):
    """run() with the release library, then with the debug library; the
    debug library's violation words after its run."""
    U.use_library(U.LIB_PATH)
    ref = run()
    U.use_library(U.DEBUG_LIB_PATH)
    U.debug_bounds(clear=True)
    got = run()
    import torch
    torch.cuda.synchronize()
    words = U.debug_bounds(clear=True)
    U.use_library(U.LIB_PATH)
    return ref, got, words


def _compare(ref, got, words):
    assert words == {"fwd": 0, "bwd": 0, "warm": 0}, words
    assert ref.keys() == got.keys()
    for name in ref:
        assert np.array_equal(ref[name], got[name]), name


@pytest.mark.parametrize("name", FORWARD)
def test_debug_build_forward_and_backward(U, name):
    w = WL.WORKLOADS[name]
    _compare(*_both(U, lambda: _forward(U, w)))


@pytest.mark.parametrize("case", list(EDGE))
def test_debug_build_edge_cases(U, case):
    base, kw = EDGE[case]
    w = WL.WORKLOADS[base].with_(**kw)
    _compare(*_both(U, lambda: _forward(U, w)))


@pytest.mark.parametrize("case", list(WARM))
def test_debug_build_warm_start(U, case):
    w = WL.WARM_WORKLOADS["warm_tiny"].with_(cfg_id=36, **WARM[case])

    def run():
        x_lr = to_device(WL.warm_storage(w, WL.WARM_LR), w.dtype)
        noise = to_device(WL.warm_storage(w, WL.WARM_NOISE), w.dtype)
        out = U.ug_warm_start(x_lr, noise, w.rho, w.alpha, w.sharpen)
        return {"x_hr": to_host_storage(out, w.dtype)}

    _compare(*_both(U, run))


def _random8():
    from tests.test_gpu_parity import RANDOM
    return dict(list(RANDOM.items())[:8])


@pytest.mark.parametrize("name", list(_random8()))
def test_debug_build_random_geometries(U, name):
    """Eight of the seeded random geometries of the parity tests, forward
    and (bf16) backward, through both builds."""
    w = _random8()[name]
    _compare(*_both(U, lambda: _forward(U, w, train=True)))


def test_debug_words_record_nothing_on_the_release_build(U):
    U.use_library(U.LIB_PATH)
    with pytest.raises(RuntimeError):
        U.debug_bounds()
