"""Pins of the oracle's backward (gradients of the joint attention with RoPE,
UltraGen notes, 关键设计 3 and the training section) against facts that do not
come from the oracle's own formulas: central finite differences of the pinned
forward, torch.autograd (float64, CPU) of an independently written dense
formulation with complex-number RoPE, closed forms at K = 0, and conservation
laws of the softmax gradient.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ultragen_oracle as O

THETA = 1e4

# masked geometries: 3x3 windows (corner windows miss the far corner), LR on
GEOS = {
    "lr_all": O.geometry(6, 6, 2, 2, 1, 2),                 # HR 6x6, l 2, LR 3x3 (rho 2), 2 text
    "lr_corr": O.geometry(6, 6, 2, 2, 1, 2, lr_mode=1),
    "overhang": O.geometry(6, 6, 1, 2, 1, 2, 4, 4, lr_mode=1),  # LR 4x4 past the grid
    "no_text_r0": O.geometry(6, 4, 0, 2, 0, 2),
}


def rand(geo, D, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((geo.seq_len, D)) for _ in range(4)]


def loss(geo, q, k, v, do):
    return float((O.forward_head(geo, q, k, v, THETA, "dense") * do).sum())


@pytest.mark.parametrize("name", list(GEOS))
def test_backward_matches_central_differences(name):
    """<grad, d> equals (f(x + eps d) - f(x - eps d)) / (2 eps) for a random
    direction d in each of q, k, v, with f = sum(O * dO)."""
    geo = GEOS[name]
    q, k, v, do = rand(geo, 8, 5)
    grads = O.backward_head(geo, q, k, v, do, THETA)
    rng = np.random.default_rng(9)
    eps = 1e-5
    for which in range(3):
        d = rng.standard_normal(q.shape)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p = [a + eps * d if n == which else a for n, a in enumerate(args_p)]
        args_m = [a - eps * d if n == which else a for n, a in enumerate(args_m)]
        fd = (loss(geo, *args_p, do) - loss(geo, *args_m, do)) / (2 * eps)
        an = float((grads[which] * d).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def _torch_layer(geo, q, k, v):
    """Dense masked attention with RoPE written independently of the oracle:
    each (2k, 2k+1) pair of a half is a complex number multiplied by
    exp(i * pos * theta^(-2k/(D/2)))."""
    L, D = q.shape
    _, pr, pc, _, _ = O.token_coords(geo)
    half = D // 2
    omega = THETA ** (-torch.arange(D // 4, dtype=torch.float64) * 2.0 / half)

    def rot(x):
        parts = []
        for h, pos in enumerate((pr, pc)):
            z = torch.view_as_complex(x[:, h * half:(h + 1) * half].reshape(L, D // 4, 2).contiguous())
            ang = torch.from_numpy(pos.astype(np.float64))[:, None] * omega[None, :]
            parts.append(torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)).reshape(L, half))
        return torch.cat(parts, dim=1)

    mask = torch.from_numpy(O.allowed_dense(geo))
    s = rot(q) @ rot(k).T / math.sqrt(D)
    s = s.masked_fill(~mask, float("-inf"))
    return torch.softmax(s, dim=1) @ v


@pytest.mark.parametrize("name", list(GEOS))
def test_backward_matches_autograd_of_independent_formulation(name):
    geo = GEOS[name]
    q, k, v, do = rand(geo, 16, 11)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = _torch_layer(geo, tq, tk, tv)
    assert np.allclose(out.detach().numpy(), O.forward_head(geo, q, k, v, THETA), atol=1e-12)
    out.backward(torch.from_numpy(do))
    dq, dk, dv = O.backward_head(geo, q, k, v, do, THETA)
    for ref, got in ((tq.grad, dq), (tk.grad, dk), (tv.grad, dv)):
        assert np.allclose(got, ref.numpy(), atol=1e-11, rtol=1e-10)


@pytest.mark.parametrize("name", list(GEOS))
def test_backward_closed_form_at_zero_keys(name):
    """K = 0: every allowed logit is 0, so P_ij = 1/n_i, LSE_i = log n_i,
    dQ = 0 and dV_j = sum over the queries i that see j of dO_i / n_i."""
    geo = GEOS[name]
    q, _, v, do = rand(geo, 8, 3)
    k = np.zeros_like(q)
    allowed = O.allowed_dense(geo)
    n = allowed.sum(axis=1)
    dqr, dkr, dv = O.attention_backward_grouped(geo, q, k, v, do)
    assert np.abs(dqr).max() == 0.0
    assert np.allclose(dv, (allowed / n[:, None]).T @ do, atol=1e-13)
    assert np.allclose(O.lse_grouped(geo, q, k), np.log(n), atol=1e-13)


@pytest.mark.parametrize("name", list(GEOS))
def test_backward_conservation_laws(name):
    """Each probability row sums to 1, so sum_j dV_j = sum_i dO_i; each row of
    dS sums to 0, so sum_j dKr_j = 0 (a transposed dS breaks this)."""
    geo = GEOS[name]
    q, k, v, do = rand(geo, 8, 4)
    _, dkr, dv = O.attention_backward_grouped(geo, q, k, v, do)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    assert np.abs(dkr.sum(axis=0)).max() < 1e-12


def test_lse_matches_logsumexp_of_masked_logits():
    geo = GEOS["lr_corr"]
    q, k, _, _ = rand(geo, 8, 6)
    s = q @ k.T / math.sqrt(8)
    s = np.where(O.allowed_dense(geo), s, -np.inf)
    ref = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
    assert np.allclose(O.lse_grouped(geo, q, k), ref, atol=1e-13)


@pytest.mark.parametrize("name", list(GEOS))
def test_allowed_queries_are_mask_columns(name):
    geo = GEOS[name]
    dense = O.allowed_dense(geo)
    coords = O.token_coords(geo)
    for j in range(geo.seq_len):
        assert np.array_equal(O.allowed_queries_of(geo, coords, j), np.nonzero(dense[:, j])[0])


def test_rope_transpose_is_adjoint_and_inverse():
    rng = np.random.default_rng(2)
    x, y = rng.standard_normal((2, 50, 16))
    pr, pc = rng.integers(0, 300, 50), rng.integers(0, 300, 50)
    rx = O.rope_rotate(x, pr, pc, THETA)
    assert np.allclose(O.rope_rotate_transpose(rx, pr, pc, THETA), x, atol=1e-13)
    assert abs((rx * y).sum() - (x * O.rope_rotate_transpose(y, pr, pc, THETA)).sum()) < 1e-11


@pytest.mark.parametrize("name", ["lr_all", "overhang"])
def test_sampled_rows_agree_with_full_backward(name):
    geo = GEOS[name]
    q, k, v, do = rand(geo, 8, 8)
    dq, dk, dv = O.backward_head(geo, q, k, v, do, THETA)
    rows = np.array([0, 1, 5, 20, geo.seq_len - 1])
    assert np.allclose(O.backward_query_rows(geo, q, k, v, do, THETA, rows), dq[rows], atol=1e-12)
    dk_s, dv_s = O.backward_key_rows(geo, q, k, v, do, THETA, rows)
    assert np.allclose(dk_s, dk[rows], atol=1e-12) and np.allclose(dv_s, dv[rows], atol=1e-12)
