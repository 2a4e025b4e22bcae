"""GPU parity: every entry point of the C ABI (through the Python binding)
against the fp64 oracle on the same seeded inputs.

Bars: permutation bit-exact; bf16 attention max-abs <= 2e-2 and rel-L2 <=
5e-3 per segment (text / HR / LR rows) and head; fp32 1e-4 for both.
"""
import numpy as np
import pytest

import workloads as WL
from oracle import ultragen_oracle as O
from tests.gpu_util import (assert_close, qkv_device, seg_errors, to_device, to_host_f64, to_host_storage,
                            tol_of)

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "tiny_masked", "small_ragged", "small_d64", "small_ragged_f32", "small_f32_d128", "1k"]
# corresponding-LR variant (lr_mode 1): LR rows permuted window-first too
CORR = ["tiny_masked_corr", "small_ragged_corr", "ragged_corr_f32"]


@pytest.fixture(scope="module")
def U():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import diffusion_transformer_sparse_amd as U
    return U


def plan_of(U, w):
    return U.ug_plan(U.desc_of(w))


def permuted_order(w):
    """Raster row held by each row of the permuted layout, from the oracle's
    window-first orders (HR always; LR when lr_mode is 1)."""
    T, N = w.n_text, w.n_hr
    perm = O.window_first_perm(w.hr_h, w.hr_w, w.window)
    lr = O.lr_window_first_perm(O.geometry_of(w)) if w.lr_mode == 1 else np.arange(w.n_lr)
    return np.concatenate([np.arange(T), T + perm, T + N + lr]).astype(np.int64)


def expected_permuted(w, x):
    """Host gather with the oracle's window-first order (rows of all heads)."""
    return x[:, permuted_order(w)]


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("name", ["tiny", "small_ragged", "small_ragged_f32", "1k", "ragged", "4k",
                                  "small_ragged_corr", "ragged_corr_f32", "4k_corr"])
def test_permute_unpermute_bit_exact(U, name):
    import torch
    w = WL.WORKLOADS[name]
    x = WL.tensor_storage(w, WL.V)
    p = plan_of(U, w)
    xd = to_device(x, w.dtype)
    xp = U.ug_permute(p, xd)
    back = U.ug_unpermute(p, xp)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_storage(xp, w.dtype), expected_permuted(w, x))
    assert np.array_equal(to_host_storage(back, w.dtype), x)


# ------------------------------------------------------------------ RoPE

@pytest.mark.parametrize("name", ["tiny", "small_ragged", "small_d64", "small_ragged_f32", "1k"] + CORR)
def test_rope2d_matches_oracle(U, name):
    import torch
    w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    q, k, _ = qkv_device(w)
    qp, kp = U.ug_permute(p, q), U.ug_permute(p, k)
    text_before = qp[:, :w.n_text].clone()
    U.ug_rope2d(p, qp, kp)
    torch.cuda.synchronize()
    assert torch.equal(qp[:, :w.n_text], text_before)
    geo = O.geometry_of(w)
    order = permuted_order(w)
    for t, dev in ((WL.Q, qp), (WL.K, kp)):
        got = to_host_f64(dev, w.dtype)[0]
        for h in range(w.heads):
            ref = O.rotate_head(geo, WL.head_f64(w, t, h), w.rope_theta)[order]
            err = np.abs(got[:, h] - ref)
            if w.dtype == "bf16":   # fp32 math, one round to nearest bf16
                assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6), float(err.max())
            else:
                assert np.all(err <= 1e-6 * np.abs(ref) + 2e-6), float(err.max())


# ------------------------------------------------------------------ attention

def run_attn_only(U, w):
    """permute -> attention (no RoPE) -> unpermute, result [L, Hh, D] float64."""
    import torch
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    qp, kp, vp = (U.ug_permute(p, x) for x in (q, k, v))
    o = U.ug_unpermute(p, U.ug_attn_fwd(p, qp, kp, vp))
    torch.cuda.synchronize()
    return to_host_f64(o, w.dtype)[0]


def oracle_attn_only(w, h):
    geo = O.geometry_of(w)
    return O.attention_grouped(geo, WL.head_f64(w, WL.Q, h), WL.head_f64(w, WL.K, h), WL.head_f64(w, WL.V, h))


@pytest.mark.parametrize("name,qscale", [(n, 1.0) for n in SMALL + CORR] + [("small_ragged", 8.0), ("1k", 8.0),
                                                                           ("tiny_masked", 8.0),
                                                                           ("small_ragged_corr", 8.0)])
def test_attention_matches_oracle(U, name, qscale):
    w = WL.WORKLOADS[name].with_(q_scale=qscale)
    got = run_attn_only(U, w)
    for h in range(w.heads):
        assert_close(seg_errors(got[:, h], oracle_attn_only(w, h), w), tol_of(w), f"{name} x{qscale} head {h}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", SMALL + CORR)
def test_full_layer_matches_oracle(U, name, fused):
    import torch
    w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.empty_like(q)
    U.Layer(p, fused=fused)(q, k, v, out)
    torch.cuda.synchronize()
    got = to_host_f64(out, w.dtype)[0]
    geo = O.geometry_of(w)
    for h in range(w.heads):
        ref = O.forward_head(geo, *(WL.head_f64(w, t, h) for t in (WL.Q, WL.K, WL.V)), w.rope_theta)
        assert_close(seg_errors(got[:, h], ref, w), tol_of(w), f"{name} head {h}")


def test_two_images_many_heads(U):
    """Batch 2 x 8 heads on a ragged 72x88 grid: batch*heads = 16, so the
    work queues keep each head's long tiles on one XCD.  The fused layer
    against the oracle for every head of both images."""
    import torch
    w = WL.WORKLOADS["ragged_b2"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.full_like(q, float("nan"))
    U.Layer(p, fused=True)(q, k, v, out)
    torch.cuda.synchronize()
    got = to_host_f64(out, w.dtype)
    geo = O.geometry_of(w)
    for b in range(w.batch):
        for h in range(w.heads):
            ref = O.forward_head(geo, *(WL.head_f64(w, t, h, b) for t in (WL.Q, WL.K, WL.V)), w.rope_theta)
            assert_close(seg_errors(got[b][:, h], ref, w), tol_of(w), f"ragged_b2 image {b} head {h}")


def sample_rows(w, seed=0):
    rng = np.random.default_rng(seed)
    T, N, L, H, W = w.n_text, w.n_hr, w.seq_len, w.hr_h, w.hr_w
    rows = [0, T - 1, T // 2] if T else []
    pts = [(0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1), (15, 16), (16, 15), (H // 2, W // 2),
           (min(31, H - 1), min(47, W - 1)), (H - 1, W // 3)]
    rows += [T + r * W + c for r, c in pts]
    rows += list(T + rng.integers(0, N, 12))
    if w.n_lr:
        rows += [T + N, L - 1] + list(T + N + rng.integers(0, w.n_lr, 4))
    return np.unique(np.asarray(rows, np.int64))


@pytest.mark.parametrize("name,fused", [("2k", True), ("ragged", True), ("4k", True), ("4k", False),
                                        ("8k", True), ("4k_corr", True), ("4k_corr", False), ("4k_d64", True),
                                        ("4k_r2", True)])
def test_full_size_sampled_rows(U, name, fused):
    """The bench's launch configuration (fused layer) at full size; the
    oracle recomputes sampled rows one by one (text, corner/edge/interior HR
    windows, LR).  The output starts as NaN, so the final finiteness check
    shows that every row of every head was written (no work item skipped)."""
    import torch
    w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.full_like(q, float("nan"))
    U.Layer(p, fused=fused)(q, k, v, out)
    torch.cuda.synchronize()
    geo = O.geometry_of(w)
    rows = sample_rows(w)
    for h in (0, w.heads - 1):
        got = to_host_f64(out[0, rows, h], w.dtype)
        ref = O.forward_rows(geo, *(WL.head_f64(w, t, h) for t in (WL.Q, WL.K, WL.V)), w.rope_theta, rows)
        assert_close(seg_errors(got, ref, w, rows), tol_of(w), f"{name} head {h}")
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("name,heads", [("4k", (0, 11, 23)), ("8k", (7,)), ("ragged", (12,)), ("4k_corr", (5,))])
def test_full_size_whole_heads(U, name, heads):
    """The bench's launch configuration (fused layer) at full size, every
    row of the given heads (all text, HR and LR rows; the heads run on
    different XCD queues) against the oracle's whole-head forward."""
    import torch
    w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.full_like(q, float("nan"))
    U.Layer(p, fused=True)(q, k, v, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    geo = O.geometry_of(w)
    for h in heads:
        got = to_host_f64(out[0, :, h].contiguous(), w.dtype)
        ref = O.forward_head(geo, *(WL.head_f64(w, t, h) for t in (WL.Q, WL.K, WL.V)), w.rope_theta)
        assert_close(seg_errors(got, ref, w), tol_of(w), f"{name} head {h} (all {w.seq_len} rows)")


@pytest.mark.parametrize("name", ["tiny", "small_ragged", "small_d64", "small_ragged_f32", "small_f32_d128", "1k",
                                  "ragged"] + CORR)
def test_fused_entry_points_bit_exact(U, name):
    """ug_permute_rope == ug_permute + ug_rope2d and ug_attn_fwd_raster ==
    ug_attn_fwd + ug_unpermute, bit for bit."""
    import torch
    w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    qp, kp = U.ug_permute(p, q), U.ug_permute(p, k)
    U.ug_rope2d(p, qp, kp)
    qf, kf = U.ug_permute_rope(p, q, k)
    vp = U.ug_permute(p, v)
    o_sep = U.ug_unpermute(p, U.ug_attn_fwd(p, qp, kp, vp))
    o_fused = U.ug_attn_fwd_raster(p, qp, kp, vp)
    torch.cuda.synchronize()
    as_bits = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(as_bits(qf), as_bits(qp)) and torch.equal(as_bits(kf), as_bits(kp))
    assert torch.equal(as_bits(o_fused), as_bits(o_sep))


@pytest.mark.parametrize("name", ["tiny", "small_ragged", "small_d64", "small_ragged_f32", "small_f32_d128", "1k",
                                  "ragged"] + CORR
                         + ["edge:" + c for c in ("batch2", "no_lr", "no_text", "corr_batch2", "corr_lr_overhang")])
def test_permute_rope_bwd_bit_exact(U, name):
    """ug_permute_rope_bwd == ug_rope2d_bwd + ug_unpermute of dq and dk, bit
    for bit, and leaves its inputs untouched (arbitrary values stand in for
    the gradients)."""
    import torch
    if name.startswith("edge:"):
        w = WL.WORKLOADS["small_ragged_f32"].with_(dtype="bf16", cfg_id=20, **EDGE[name[5:]])
    else:
        w = WL.WORKLOADS[name]
    p = plan_of(U, w)
    gq, gk, _ = qkv_device(w)
    as_bits = (lambda t: t.view(torch.int16)) if w.dtype == "bf16" else (lambda t: t.view(torch.int32))
    gq0, gk0 = gq.clone(), gk.clone()
    dq, dk = U.ug_permute_rope_bwd(p, gq, gk)
    sq, sk = gq.clone(), gk.clone()
    U.ug_rope2d_bwd(p, sq, sk)
    rq, rk = U.ug_unpermute(p, sq), U.ug_unpermute(p, sk)
    torch.cuda.synchronize()
    assert torch.equal(as_bits(dq), as_bits(rq)) and torch.equal(as_bits(dk), as_bits(rk))
    assert torch.equal(as_bits(gq), as_bits(gq0)) and torch.equal(as_bits(gk), as_bits(gk0))


def test_attention_is_deterministic(U):
    import torch
    w = WL.WORKLOADS["1k"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    o1 = U.ug_attn_fwd(p, q, k, v)
    o2 = U.ug_attn_fwd(p, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_attention_queue_cursors_reused_and_concurrent(U):
    """The persistent attention grid takes query tiles through per-XCD queue
    cursors; each launch takes one of the plan's 64 cursor slots and leaves it
    cleared.  More launches than slots give bit-identical outputs, and
    launches with one plan on two streams at once match the serial result."""
    import torch
    w = WL.WORKLOADS["1k"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    ref = U.ug_attn_fwd(p, q, k, v)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    o = torch.empty_like(ref)
    for i in range(140):  # every slot used at least twice
        U.ug_attn_fwd(p, q, k, v, o)
        if i % 20 == 0 or i == 139:
            torch.cuda.synchronize()
            assert torch.equal(bits(o), bits(ref)), f"launch {i}"
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [torch.empty_like(ref) for _ in range(8)]
    torch.cuda.synchronize()
    for j, out in enumerate(outs):
        with torch.cuda.stream(s1 if j % 2 == 0 else s2):
            U.ug_attn_fwd(p, q, k, v, out)
    torch.cuda.synchronize()
    for j, out in enumerate(outs):
        assert torch.equal(bits(out), bits(ref)), f"concurrent launch {j}"
    # two plans (different shapes, their own cursors) at the same time
    w2 = WL.WORKLOADS["small_ragged"]
    p2 = plan_of(U, w2)
    q2, k2, v2 = qkv_device(w2)
    ref2 = U.ug_attn_fwd(p2, q2, k2, v2)
    torch.cuda.synchronize()
    o1, o2 = torch.empty_like(ref), torch.empty_like(ref2)
    for _ in range(3):
        with torch.cuda.stream(s1):
            U.ug_attn_fwd(p, q, k, v, o1)
        with torch.cuda.stream(s2):
            U.ug_attn_fwd(p2, q2, k2, v2, o2)
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(ref)) and torch.equal(bits(o2), bits(ref2))


@pytest.mark.gpu
def test_attention_cursor_slots_wrap_while_in_flight(U):
    """130 launches with one plan alternate between two streams with no
    synchronisation, so every cursor slot comes back while its previous
    launch may still run on the other stream; the launcher makes the new
    launch wait for that one, so every output matches the serial result."""
    import torch
    w = WL.WORKLOADS["small_ragged"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    ref = U.ug_attn_fwd(p, q, k, v)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(ref) for _ in range(130)]
    for j, out in enumerate(outs):
        with torch.cuda.stream(streams[j % 2]):
            U.ug_attn_fwd(p, q, k, v, out)
    torch.cuda.synchronize()
    for j, out in enumerate(outs):
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"launch {j}"


@pytest.mark.gpu
def test_attention_refuses_stream_capture(U):
    """A captured launch would take its cursor slot once, at capture time,
    and share it with every replay: the persistent launches refuse capture
    (before launching anything) with UG_ERR_UNSUPPORTED."""
    import torch
    w = WL.WORKLOADS["tiny"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    o = torch.empty_like(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(U.UgError) as err:
        with torch.cuda.graph(g):
            U.ug_attn_fwd(p, q, k, v, o)
    assert err.value.status == 2  # UG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isfinite(U.ug_attn_fwd(p, q, k, v)).all()  # the plan still works afterwards


# ------------------------------------------------------------------ edge cases

EDGE = {
    "no_text": dict(n_text=0),
    "no_lr": dict(lr_h=0, lr_w=0),
    "no_text_no_lr": dict(n_text=0, lr_h=0, lr_w=0),
    "radius0": dict(radius=0),
    "radius2": dict(radius=2),
    "window8": dict(window=8),
    "window_covers_grid": dict(window=64),
    "batch2": dict(batch=2),
    "one_text": dict(n_text=1),
    "corr_radius0": dict(lr_mode=1, radius=0),
    "corr_window8_rho3": dict(lr_mode=1, window=8, rho=3),   # windows with 0..9 anchors
    "corr_lr_overhang": dict(lr_mode=1, lr_h=14, lr_w=14),   # anchors past the window grid
    "corr_no_text": dict(lr_mode=1, n_text=0),
    "corr_batch2": dict(lr_mode=1, batch=2),
}
FUSED_EDGE = ("batch2", "no_lr", "corr_batch2", "corr_lr_overhang")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", list(EDGE))
def test_edge_cases(U, case, dtype):
    import torch
    base = WL.WORKLOADS["small_ragged_f32"].with_(dtype=dtype, cfg_id=20)
    w = base.with_(**EDGE[case])
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.empty_like(q)
    U.Layer(p, fused=(case in FUSED_EDGE))(q, k, v, out)
    torch.cuda.synchronize()
    geo = O.geometry_of(w)
    for b in range(w.batch):
        got = to_host_f64(out[b], w.dtype)
        for h in range(w.heads):
            ref = O.forward_head(geo, *(WL.head_f64(w, t, h, b) for t in (WL.Q, WL.K, WL.V)), w.rope_theta)
            assert_close(seg_errors(got[:, h], ref, w), tol_of(w), f"{case} {dtype} b{b} h{h}")


def _random_workloads(n=32):
    """Seeded small geometries in the range the edge cases cover (windows of
    8 and 16, radius 0 to 2), with random grid sizes, text rows, LR grids
    (default, explicit or none), LR mode, batch, dtype and head_dim."""
    rng = np.random.default_rng([2026, 78])
    out = {}
    for i in range(n):
        H, W = int(rng.integers(8, 73)), int(rng.integers(8, 73))
        kind = int(rng.integers(0, 3))
        lh = -(-H // 4) if kind == 0 else 0 if kind == 1 else int(rng.integers(1, -(-H // 4) + 3))
        lw = -(-W // 4) if kind == 0 else 0 if kind == 1 else int(rng.integers(1, -(-W // 4) + 3))
        dtype = "bf16" if i % 3 else "f32"
        out[f"random{i:02d}"] = WL.Workload(
            f"random{i:02d}", 200 + i, H, W, lh, lw, int(rng.choice([0, 1, 9, 40])), int(rng.integers(1, 4)),
            int(rng.choice([64, 128])), dtype, window=int(rng.choice([8, 16])), radius=int(rng.integers(0, 3)),
            batch=int(rng.integers(1, 3)), lr_mode=int(rng.integers(0, 2)))
    return out


RANDOM = _random_workloads()


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_geometries(U, name):
    """The layer (fused or not, alternately) on seeded random small
    geometries: every row of every head and image against the oracle."""
    import torch
    w = RANDOM[name]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    out = torch.full_like(q, float("nan"))
    U.Layer(p, fused=int(name[-2:]) % 2 == 0)(q, k, v, out)
    torch.cuda.synchronize()
    geo = O.geometry_of(w)
    for b in range(w.batch):
        got = to_host_f64(out[b], w.dtype)
        for h in range(w.heads):
            ref = O.forward_head(geo, *(WL.head_f64(w, t, h, b) for t in (WL.Q, WL.K, WL.V)), w.rope_theta)
            assert_close(seg_errors(got[:, h], ref, w), tol_of(w), f"{name} {w} b{b} h{h}")


def test_argument_errors_on_device(U):
    import torch
    w = WL.WORKLOADS["tiny"]
    p = plan_of(U, w)
    q, k, v = qkv_device(w)
    lib = U.lib()
    import ctypes
    vp = ctypes.c_void_p
    s = vp(torch.cuda.current_stream().cuda_stream)
    assert lib.ug_permute(p.handle, vp(q.data_ptr()), vp(q.data_ptr()), s) == 1
    assert lib.ug_permute(p.handle, vp(q.data_ptr() + 4), vp(k.data_ptr()), s) == 1
    assert lib.ug_attn_fwd(p.handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), vp(q.data_ptr()),
                           None, s) == 1
    assert lib.ug_rope2d(p.handle, vp(q.data_ptr()), vp(q.data_ptr()), s) == 1
    assert lib.ug_permute_rope(p.handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
                               s) == 1
    assert lib.ug_attn_fwd_raster(p.handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), vp(v.data_ptr()),
                                  None, s) == 1
    assert lib.ug_permute_rope_bwd(p.handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
                                   s) == 1
    assert lib.ug_permute_rope_bwd(p.handle, vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()), vp(v.data_ptr()),
                                   s) == 1
    with pytest.raises(ValueError):
        U.ug_permute(p, q[:, :10].contiguous())
