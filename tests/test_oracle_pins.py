"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties one oracle function to something other than itself: a
hand-worked fixture under tests/golden/, a closed form, or a special case that
reduces to a library routine (torch's scaled_dot_product_attention on the CPU).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ultragen_oracle as O
from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- permutation

@pytest.mark.parametrize("name", ["window_first_4x4_l2.json", "window_first_3x5_l2.json"])
def test_window_first_perm_hand_worked(name):
    g = golden(name)
    perm = O.window_first_perm(g["hr_h"], g["hr_w"], g["window"])
    assert perm.tolist() == g["perm"]
    assert O.window_offsets(g["hr_h"], g["hr_w"], g["window"]).tolist() == g["win_off"]
    if "inverse" in g:
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size)
        assert inv.tolist() == g["inverse"]


@pytest.mark.parametrize("H,W,l", [(64, 64, 16), (32, 48, 16), (256, 256, 16), (12, 8, 4)])
def test_window_first_square_closed_form(H, W, l):
    """Divisible grids: window-first index j = ((wy*gx + wx)*l + ry)*l + rx."""
    perm = O.window_first_perm(H, W, l)
    gx = W // l
    r, c = np.divmod(perm, W)
    j = ((r // l * gx + c // l) * l + r % l) * l + c % l
    assert np.array_equal(j, np.arange(H * W))


@pytest.mark.parametrize("H,W,l", [(250, 380, 16), (37, 45, 16), (3, 5, 2), (17, 1, 16)])
def test_window_first_is_bijection_and_contiguous(H, W, l):
    perm = O.window_first_perm(H, W, l)
    assert np.array_equal(np.sort(perm), np.arange(H * W))
    off = O.window_offsets(H, W, l)
    assert off[-1] == H * W
    gx = -(-W // l)
    r, c = np.divmod(perm, W)
    win = r // l * gx + c // l
    # each window's tokens form the block [off[w], off[w+1])
    for w in range(off.size - 1):
        assert np.all(win[off[w]:off[w + 1]] == w)


# ---------------------------------------------------------------- neighbours

def test_neighbours_hand_worked():
    g = golden("neighbours_3x3_r1.json")
    flat, off = O.neighbour_windows(g["hr_h"], g["hr_w"], g["window"], g["radius"])
    got = [flat[off[i]:off[i + 1]].tolist() for i in range(off.size - 1)]
    assert got == g["neighbours"]


def test_neighbour_counts_closed_form():
    pins = golden("pair_counts.json")["neighbour_entries"]
    for name, expect in pins.items():
        w = WORKLOADS[name]
        flat, off = O.neighbour_windows(w.hr_h, w.hr_w, w.window, w.radius)
        gy, gx = -(-w.hr_h // w.window), -(-w.hr_w // w.window)
        assert flat.size == expect == (3 * gy - 2) * (3 * gx - 2)
        cnt = np.diff(off)
        # corners 4, edges 6, interior 9
        grid = cnt.reshape(gy, gx)
        assert grid[0, 0] == grid[-1, -1] == grid[0, -1] == grid[-1, 0] == 4
        if gx > 2:
            assert grid[0, 1] == 6
        if gy > 2 and gx > 2:
            assert grid[1, 1] == 9
        # symmetry
        pairs = {(i, j) for i in range(off.size - 1) for j in flat[off[i]:off[i + 1]]}
        assert all((j, i) in pairs for (i, j) in pairs)


# ---------------------------------------------------------------- mask

def test_mask_hand_worked():
    g = golden("mask_4x4_l2_t2_lr2x2.json")
    geo = O.geometry(g["hr_h"], g["hr_w"], g["n_text"], g["window"], g["radius"], g["rho"],
                     g["lr_h"], g["lr_w"])
    dense = O.allowed_dense(geo)
    coords = O.token_coords(geo)
    for row, keys in g["allowed"].items():
        assert np.nonzero(dense[int(row)])[0].tolist() == keys
        assert O.allowed_keys_of(geo, coords, int(row)).tolist() == keys


def test_one_hot_v_reads_probability_rows():
    """With V = identity (D >= L) the output rows are the softmax rows: they
    sum to one and are zero exactly off the hand-worked allowed sets."""
    g = golden("mask_4x4_l2_t2_lr2x2.json")
    geo = O.geometry(g["hr_h"], g["hr_w"], g["n_text"], g["window"], g["radius"], g["rho"],
                     g["lr_h"], g["lr_w"])
    L, D = geo.seq_len, 24
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    v = np.zeros((L, D))
    v[np.arange(L), np.arange(L)] = 1.0
    for mode in ("dense", "grouped"):
        out = O.forward_head(geo, q, k, v, 10000.0, mode)
        assert np.allclose(out.sum(axis=1), 1.0, atol=1e-14)
        for row, keys in g["allowed"].items():
            nz = np.nonzero(out[int(row), :L] > 0)[0].tolist()
            assert nz == keys


def test_zero_keys_give_window_means():
    """K = 0 makes every allowed weight equal, so o_i is the mean of V over the
    allowed keys.  4x4 HR, 2x2 windows, radius 0, no text, no LR, V_j = j:
    token 0 -> 2.5, token 2 -> 4.5, token 10 -> 12.5; radius 1 -> 7.5."""
    geo = O.geometry(4, 4, 0, window=2, radius=0, rho=4, lr_h=0, lr_w=0)
    geo = O.Geometry(4, 4, 0, 0, 0, 2, 0, 4)
    L, D = 16, 8
    q = np.random.default_rng(1).standard_normal((L, D))
    k = np.zeros((L, D))
    v = np.repeat(np.arange(L, dtype=np.float64)[:, None], D, axis=1)
    out = O.forward_head(geo, q, k, v, 10000.0)
    assert out[0, 0] == pytest.approx(2.5, abs=1e-14)
    assert out[2, 0] == pytest.approx(4.5, abs=1e-14)
    assert out[10, 0] == pytest.approx(12.5, abs=1e-14)
    geo1 = O.Geometry(4, 4, 0, 0, 0, 2, 1, 4)
    out1 = O.forward_head(geo1, q, k, v, 10000.0)
    assert np.allclose(out1, 7.5, atol=1e-13)


def test_constant_v_gives_constant_output():
    w = WORKLOADS["tiny_masked"]
    geo = O.geometry_of(w)
    rng = np.random.default_rng(3)
    L, D = geo.seq_len, 64
    q, k = rng.standard_normal((L, D)) * 4, rng.standard_normal((L, D)) * 4
    out = O.forward_head(geo, q, k, np.ones((L, D)), 10000.0)
    assert np.max(np.abs(out - 1.0)) < 1e-13


# ---------------------------------------------------------------- pair counts

def test_pair_counts_closed_form():
    pins = golden("pair_counts.json")
    for name, expect in pins["counts"].items():
        assert O.pair_count(O.geometry_of(WORKLOADS[name])) == expect, name


def test_pair_count_matches_dense_mask():
    for name in ("tiny", "tiny_masked", "small_ragged"):
        geo = O.geometry_of(WORKLOADS[name])
        assert O.pair_count(geo) == int(O.allowed_dense(geo).sum())


def test_complexity_law_of_local_windows():
    """Own-window-only HR attention at 4K is N*l^2 pairs, 256x fewer than
    dense (UltraGen notes, 关键设计 1); a 64-token window (1024 px) costs 16x
    the 16-token one (ablation table)."""
    pins = golden("pair_counts.json")
    g16 = O.Geometry(256, 256, 0, 0, 0, 16, 0, 4)
    g64 = O.Geometry(256, 256, 0, 0, 0, 64, 0, 4)
    p16, p64 = O.pair_count(g16), O.pair_count(g64)
    assert p16 == pins["own_window_4k_hr_only"] == 65536 * 16 ** 2
    assert 65536 ** 2 // p16 == 256
    assert p64 == pins["own_window_4k_l64_hr_only"] == 16 * p16


# ---------------------------------------------------------------- RoPE

def test_rope_hand_worked():
    for case in golden("rope_worked.json")["cases"]:
        x = np.asarray(case["x"], np.float64)[None, :]
        if "lr_index" in case:
            # LR token (m, n) sits at (rho m, rho n): check through token_coords
            geo = O.geometry(4, 8, 0, window=4, radius=0, rho=case["rho"], lr_h=1, lr_w=2)
            kind, pr, pc, _, _ = O.token_coords(geo)
            m, n = case["lr_index"]
            row = geo.n_hr + m * geo.lr_w + n
            assert kind[row] == O.LR and [pr[row], pc[row]] == case["pos"]
        out = O.rope_rotate(x, np.array([case["pos"][0]]), np.array([case["pos"][1]]), case["theta"])
        assert np.allclose(out[0], case["out"], atol=5e-8)


def test_rope_invariants():
    rng = np.random.default_rng(11)
    D, n = 64, 50
    x = rng.standard_normal((n, D))
    pr, pc = rng.integers(0, 512, n), rng.integers(0, 512, n)
    # position (0,0) is the identity; rotation preserves norms
    assert np.array_equal(O.rope_rotate(x, np.zeros(n, int), np.zeros(n, int), 1e4), x)
    y = O.rope_rotate(x, pr, pc, 1e4)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    # q.k depends only on the position difference
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    a = O.rope_rotate(q, np.array([7]), np.array([3]), 1e4) @ O.rope_rotate(k, np.array([2]), np.array([9]), 1e4).T
    b = O.rope_rotate(q, np.array([107]), np.array([203]), 1e4) @ O.rope_rotate(k, np.array([102]), np.array([209]), 1e4).T
    assert a[0, 0] == pytest.approx(b[0, 0], rel=1e-11)
    # the rotation is a rotation of each pair: (a,b) -> angle shift; rotating
    # by p then by -p is the identity
    back = O.rope_rotate(y, -pr, -pc, 1e4)
    assert np.allclose(back, x, atol=1e-12)


def test_lr_positions_scaled_by_rho():
    geo = O.geometry_of(WORKLOADS["ragged"])
    kind, pr, pc, _, _ = O.token_coords(geo)
    T, N = geo.n_text, geo.n_hr
    m, n = np.divmod(np.arange(geo.n_lr), geo.lr_w)
    assert np.array_equal(pr[T + N:], 4 * m) and np.array_equal(pc[T + N:], 4 * n)
    assert pr[T + N:].max() <= geo.hr_h - 1 and pc[T + N:].max() <= geo.hr_w - 1
    assert np.all(pr[:T] == 0) and np.all(pc[:T] == 0)


# ---------------------------------------------------------------- attention vs library

def _sdpa(q, k, v, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)[0, 0].numpy()


def test_window_covering_grid_is_dense_attention():
    """l >= max(H, W), no text, no LR: the method is textbook attention on the
    rotated Q and K (torch SDPA, float64, CPU)."""
    geo = O.Geometry(12, 10, 0, 0, 0, 16, 1, 4)
    rng = np.random.default_rng(21)
    L, D = geo.seq_len, 32
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    out = O.forward_head(geo, q, k, v, 10000.0)
    qr, kr = O.rotate_head(geo, q, 1e4), O.rotate_head(geo, k, 1e4)
    assert np.allclose(out, _sdpa(qr, kr, v), atol=1e-12)
    # radius covering the window grid gives the same
    geo2 = O.Geometry(12, 10, 0, 0, 0, 4, 3, 4)
    assert np.allclose(O.forward_head(geo2, q, k, v, 1e4), out, atol=1e-12)


def test_composite_matches_library_with_hand_checked_mask():
    w = WORKLOADS["tiny_masked"]
    geo = O.geometry_of(w)
    rng = np.random.default_rng(22)
    L, D = geo.seq_len, 64
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    qr, kr = O.rotate_head(geo, q, 1e4), O.rotate_head(geo, k, 1e4)
    ref = _sdpa(qr, kr, v, O.allowed_dense(geo))
    for mode in ("dense", "grouped"):
        assert np.allclose(O.forward_head(geo, q, k, v, 1e4, mode), ref, atol=1e-12)
    rows = np.array([0, 7, 16, 17, 300, 1000, L - 144, L - 1])
    assert np.allclose(O.forward_rows(geo, q, k, v, 1e4, rows), ref[rows], atol=1e-12)


def test_mask_structure_on_tiny_masked():
    """Spot-check of the composite mask on a 3x3 window grid: HR rows of the
    centre window see all 2304 HR tokens, corner windows only 4 windows."""
    geo = O.geometry_of(WORKLOADS["tiny_masked"])
    dense = O.allowed_dense(geo)
    T, N, Nl = geo.n_text, geo.n_hr, geo.n_lr
    counts = dense.sum(axis=1)
    assert np.all(counts[:T] == T + N)
    assert np.all(counts[T + N:] == Nl + T)
    centre = T + 24 * 48 + 24      # raster (24, 24) -> window (1, 1)
    corner = T + 0
    assert counts[centre] == T + Nl + 9 * 256
    assert counts[corner] == T + Nl + 4 * 256


# ---------------------------------------------------------------- corresponding-LR variant

@pytest.mark.parametrize("fixture", ["corresponding_lr_8x8_l4_rho2.json", "corresponding_lr_overhang_4x4_l2_rho2.json"])
def test_corresponding_lr_hand_worked(fixture):
    g = golden(fixture)
    geo = O.geometry(g["hr_h"], g["hr_w"], g["n_text"], g["window"], g["radius"], g["rho"], g["lr_h"], g["lr_w"],
                     g["lr_mode"])
    assert O.lr_window_first_perm(geo).tolist() == g["lr_perm"]
    assert O.lr_window_offsets(geo).tolist() == g["lr_win_off"]
    dense = O.allowed_dense(geo)
    coords = O.token_coords(geo)
    for row, keys in g["allowed"].items():
        assert np.nonzero(dense[int(row)])[0].tolist() == keys
        assert O.allowed_keys_of(geo, coords, int(row)).tolist() == keys
    assert O.pair_count(geo) == int(dense.sum())
    if "pairs" in g:
        assert O.pair_count(geo) == g["pairs"]


def test_corresponding_lr_closed_form_4k():
    pins = golden("pair_counts.json")["corresponding_lr_4k"]
    w = WORKLOADS["4k"]
    g1 = O.geometry(w.hr_h, w.hr_w, w.n_text, w.window, w.radius, w.rho, w.lr_h, w.lr_w, 1)
    g0 = O.geometry(w.hr_h, w.hr_w, w.n_text, w.window, w.radius, w.rho, w.lr_h, w.lr_w, 0)
    assert O.pair_count(g1) == pins["total"]
    assert O.pair_count(g0) - O.pair_count(g1) == w.n_hr * w.n_lr - pins["hr_to_lr"]
    off = O.lr_window_offsets(g1)
    assert np.all(np.diff(off)[:-1] == 16) and off[-1] == off[-2] == w.n_lr


@pytest.mark.parametrize("H,W,lh,lw,l,rho,r", [(48, 40, 12, 10, 16, 4, 1), (37, 45, 10, 12, 16, 4, 1),
                                              (30, 30, 11, 11, 8, 3, 0), (20, 28, 8, 9, 8, 4, 2),
                                              (30, 30, 20, 3, 8, 2, 2)])
def test_corresponding_lr_dense_vs_grouped_and_library(H, W, lh, lw, l, rho, r):
    """Both oracle modes agree and match torch SDPA given the variant's mask;
    the LR window-first order is a bijection grouping LR tokens by window."""
    geo = O.geometry(H, W, 7, l, r, rho, lh, lw, 1)
    rng = np.random.default_rng(31)
    L, D = geo.seq_len, 32
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    dense = O.forward_head(geo, q, k, v, 1e4, "dense")
    grouped = O.forward_head(geo, q, k, v, 1e4, "grouped")
    qr, kr = O.rotate_head(geo, q, 1e4), O.rotate_head(geo, k, 1e4)
    assert np.allclose(dense, grouped, atol=1e-12)
    assert np.allclose(dense, _sdpa(qr, kr, v, O.allowed_dense(geo)), atol=1e-12)
    perm = O.lr_window_first_perm(geo)
    assert np.array_equal(np.sort(perm), np.arange(geo.n_lr))
    off = O.lr_window_offsets(geo)
    _, _, _, wy, wx = O.token_coords(geo)
    gy, gx = geo.grid
    lw_ = (wy * gx + wx)[geo.n_text + geo.n_hr:][perm]
    for wdx in range(gy * gx):
        assert np.all(lw_[off[wdx]:off[wdx + 1]] == wdx)
