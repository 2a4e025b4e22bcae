"""Pins of the oracle's warm start (UltraGen notes, 关键设计 4; reading R12:
bilinear upsampling with LR sample (m, n) at HR (rho*m, rho*n), unsharp-mask
sharpening with a 3x3 binomial blur, blend alpha * noise + (1 - alpha) *
reference) against closed forms and library routines.
"""
import numpy as np
import pytest
import scipy.ndimage
import torch

from oracle import ultragen_oracle as O


def test_upsampling_passes_through_the_lr_samples():
    rng = np.random.default_rng(1)
    h, w, rho = 5, 7, 4
    x = rng.standard_normal((h, w, 3))
    u = O.upsample_bilinear(x, 4 * h, 4 * w, rho)
    assert np.array_equal(u[::rho, ::rho], x)


@pytest.mark.parametrize("rho", [1, 2, 4])
def test_upsampling_reproduces_linear_fields(rho):
    h, w = 6, 5
    m, n = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    x = np.stack([3.0 * m - 2.0 * n + 0.5, -m + 0.25 * n], axis=-1)
    H, W = rho * (h - 1) + 1, rho * (w - 1) + 1
    u = O.upsample_bilinear(x, H, W, rho)
    r, c = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    ref = np.stack([3.0 * r / rho - 2.0 * c / rho + 0.5, -r / rho + 0.25 * c / rho], axis=-1)
    assert np.allclose(u, ref, atol=1e-12)


def test_upsampling_equals_torch_bilinear_align_corners():
    """On the grid whose last row and column sit on the last LR sample,
    (r/rho, c/rho) is exactly align_corners=True bilinear interpolation."""
    rng = np.random.default_rng(2)
    h, w, rho = 9, 6, 4
    x = rng.standard_normal((h, w, 4))
    H, W = rho * (h - 1) + 1, rho * (w - 1) + 1
    t = torch.from_numpy(x).permute(2, 0, 1)[None]
    ref = torch.nn.functional.interpolate(t, size=(H, W), mode="bilinear", align_corners=True)[0].permute(1, 2, 0)
    assert np.allclose(O.upsample_bilinear(x, H, W, rho), ref.numpy(), atol=1e-12)


def test_upsampling_replicates_past_the_last_sample():
    rng = np.random.default_rng(3)
    h, w, rho = 4, 4, 4
    x = rng.standard_normal((h, w, 2))
    u = O.upsample_bilinear(x, rho * h, rho * w, rho)   # rows/cols 13..15 lie past the last sample at 12
    last = rho * (h - 1)
    for r in range(last, rho * h):
        assert np.array_equal(u[r], u[last])
        assert np.array_equal(u[:, r], u[:, last])


def test_sharpen_impulse_response():
    """(1 + s) delta - s * B with B = [1 2 1]/4 x [1 2 1]/4: centre 1 + 3s/4,
    edge neighbours -s/8, corners -s/16, zero elsewhere."""
    s = 0.7
    u = np.zeros((9, 9, 1))
    u[4, 4] = 1.0
    y = O.sharpen_unsharp(u, s)[..., 0]
    ref = np.zeros((9, 9))
    ref[4, 4] = 1 + 0.75 * s
    for dy, dx in ((-1, 0), (1, 0), (0, -1), (0, 1)):
        ref[4 + dy, 4 + dx] = -s / 8
    for dy, dx in ((-1, -1), (-1, 1), (1, -1), (1, 1)):
        ref[4 + dy, 4 + dx] = -s / 16
    assert np.allclose(y, ref, atol=1e-15)


def test_sharpen_equals_nearest_edge_convolution():
    rng = np.random.default_rng(4)
    u = rng.standard_normal((11, 13, 3))
    s = 1.3
    b = np.array([1.0, 2.0, 1.0]) / 4
    kern = -s * np.outer(b, b)
    kern[1, 1] += 1 + s
    ref = np.stack([scipy.ndimage.convolve(u[..., ch], kern, mode="nearest") for ch in range(3)], axis=-1)
    assert np.allclose(O.sharpen_unsharp(u, s), ref, atol=1e-12)


def test_sharpen_keeps_constant_and_interior_linear_fields():
    H, W = 10, 12
    r, c = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    const = np.full((H, W, 2), 3.25)
    assert np.allclose(O.sharpen_unsharp(const, 2.0), const, atol=1e-14)
    lin = (0.5 * r - 1.5 * c)[..., None]
    assert np.allclose(O.sharpen_unsharp(lin, 2.0)[1:-1, 1:-1], lin[1:-1, 1:-1], atol=1e-12)


def test_blend_endpoints_and_linearity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 5, 8))
    noise = rng.standard_normal((16, 20, 8))
    ref = O.sharpen_unsharp(O.upsample_bilinear(x, 16, 20, 4), 0.5)
    assert np.array_equal(O.warm_start(x, noise, 4, 1.0, 0.5), noise)
    assert np.allclose(O.warm_start(x, noise, 4, 0.0, 0.5), ref, atol=1e-15)
    a = 0.3
    assert np.allclose(O.warm_start(x, noise, 4, a, 0.5), a * noise + (1 - a) * ref, atol=1e-15)
