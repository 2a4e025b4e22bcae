"""GPU parity of the warm-start kernel (UltraGen notes, 关键设计 4; reading
R12) against the fp64 oracle on the same seeded latents.

Bars: fp32 arithmetic (a dozen operations per output) keeps the fp32 path
within 1e-5 * max|ref|; the bf16 path adds one round-to-nearest of the output,
|error| <= 2^-8 |ref| + 1e-5 * max|ref|.
"""
import numpy as np
import pytest

import workloads as WL
from oracle import ultragen_oracle as O
from tests.gpu_util import to_device, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def U():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import diffusion_transformer_sparse_amd as U
    return U


def check(U, w, in_place=False):
    import torch
    x_lr = to_device(WL.warm_storage(w, WL.WARM_LR), w.dtype)
    noise = to_device(WL.warm_storage(w, WL.WARM_NOISE), w.dtype)
    out = U.ug_warm_start(x_lr, noise, w.rho, w.alpha, w.sharpen, x_hr=noise if in_place else None)
    torch.cuda.synchronize()
    got = to_host_f64(out, w.dtype)
    xl, nz = WL.warm_f64(w, WL.WARM_LR), WL.warm_f64(w, WL.WARM_NOISE)
    for b in range(w.batch):
        ref = O.warm_start(xl[b], nz[b], w.rho, w.alpha, w.sharpen)
        err = np.abs(got[b] - ref)
        scale = np.abs(ref).max()
        bound = (2.0 ** -8 * np.abs(ref) if w.dtype == "bf16" else 0.0) + 1e-5 * scale
        assert np.all(err <= bound), (w.name, b, float((err - bound).max()))


@pytest.mark.parametrize("name", ["warm_tiny", "warm_ragged", "warm_4k"])
def test_warm_start_matches_oracle(U, name):
    check(U, WL.WARM_WORKLOADS[name])


CASES = {
    "rho1": dict(rho=1, lr_h=40, lr_w=36),
    "rho2": dict(rho=2, lr_h=20, lr_w=18),
    "rho3_ragged": dict(rho=3, lr_h=14, lr_w=12),
    "lr_short": dict(lr_h=7, lr_w=5),             # HR rows/columns past the last LR sample
    "lr_long": dict(lr_h=13, lr_w=11),            # LR samples past the HR grid (unused)
    "alpha0": dict(alpha=0.0),
    "alpha1": dict(alpha=1.0),
    "no_sharpen": dict(sharpen=0.0),
    "strong_sharpen": dict(sharpen=2.0),
    "one_pixel_lr": dict(lr_h=1, lr_w=1),
    "rho8": dict(rho=8, lr_h=5, lr_w=5),           # tiles whose third LR tap lies past the staged patch
    "rho16_ragged": dict(rho=16, lr_h=3, lr_w=3),
    "bf16_c72": dict(dtype="bf16", channels=72),  # a partial block of channel vectors
    "f32_c36": dict(channels=36),
    "bf16_c16": dict(dtype="bf16", channels=16),
    "batch3": dict(batch=3),
}


@pytest.mark.parametrize("case", list(CASES))
def test_warm_start_cases(U, case):
    check(U, WL.WARM_WORKLOADS["warm_tiny"].with_(cfg_id=34, **CASES[case]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_warm_start_in_place(U, dtype):
    check(U, WL.WARM_WORKLOADS["warm_tiny"].with_(cfg_id=35, dtype=dtype, channels=16), in_place=True)
