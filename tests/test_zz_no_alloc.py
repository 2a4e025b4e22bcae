"""ug_attn_bwd_noalloc (the backward with its statistics in the library's
per-GPU scratch, for callers that cannot allocate) against ug_attn_bwd with a
caller workspace: bit-identical gradients on two calls in a row, the second
on a smaller input, through the C ABI."""
import ctypes

import numpy as np
import pytest

import workloads as WL
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def U():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import diffusion_transformer_sparse_amd as U
    return U


def _case(U, name):
    import torch
    w = WL.WORKLOADS[name]
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = (to_device(WL.tensor_storage(w, t), w.dtype) for t in (WL.Q, WL.K, WL.V, WL.DO))
    o, lse = U.ug_attn_fwd_lse(p, q, k, v)
    return p, (q, k, v, o, do, lse)


def test_noalloc_backward_matches_the_workspace_backward(U):
    import torch
    bits = lambda t: t.view(torch.int16)
    for name in ("1k", "small_ragged", "small_d64"):  # the second and third calls are smaller
        p, (q, k, v, o, do, lse) = _case(U, name)
        ref = U.ug_attn_bwd(p, q, k, v, o, do, lse)
        got = [torch.full_like(q, float("nan")) for _ in range(3)]
        U.ug_attn_bwd_noalloc(p, q, k, v, o, do, lse, *got)
        torch.cuda.synchronize()
        for r, g, what in zip(ref, got, ("dq", "dk", "dv")):
            assert torch.equal(bits(g), bits(r)), (name, what)
        p.close()


def test_noalloc_refuses_a_plan_beyond_the_scratch(U):
    """64 heads at 8K need 143 MB of statistics: refused before any launch."""
    import torch
    desc = U.make_desc(512, 512, 128, 128, 512, heads=64, head_dim=128)
    p = U.ug_plan(desc)
    assert p.info["bwd_workspace_bytes"] > (64 << 20)
    bufs = [torch.empty(16, dtype=torch.uint8, device="cuda") for _ in range(9)]
    vp = [ctypes.c_void_p(b.data_ptr()) for b in bufs]
    lib = U.lib()
    st = lib.ug_attn_bwd_noalloc(p.handle, *vp, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2, U.ug_last_error()  # UG_ERR_UNSUPPORTED
    assert "scratch" in U.ug_last_error()
    p.close()
