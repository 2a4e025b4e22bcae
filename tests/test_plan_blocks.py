"""Bit-exact pins of the block lists the attention kernels walk (the query
tiles with their key ranges, and the backward's key tiles with their query
ranges and per-key range masks) against the oracle's composite mask, which
is written out from 2D coordinates (UltraGen notes, 关键设计 1-2: windows,
adjacent windows, text and LR anchors).

The lists are expanded as they are: the union of a query row's key ranges
is compared with oracle.allowed_keys_of, and the union of a key row's
(masked) query ranges with oracle.allowed_queries_of, for every row.  Permuted
rows are mapped to raster rows with the oracle's own window-first orders.
Both oracle functions depend on a row only through its coordinates class
(kind, window): every row is checked, the oracle set is computed once per
class.  Besides the evaluation workloads and hand-picked radius 2 and 4
cases, 96 seeded random small geometries (windows of 2 to 16, radius 0 to
3, rho 1 to 5, default, explicit or no LR grid, both LR modes) are checked
the same way."""
import numpy as np
import pytest

import diffusion_transformer_sparse_amd as U
from oracle import ultragen_oracle as O
from workloads import WORKLOADS

# (name, descriptor arguments): the evaluation workloads plus radius 2 and 4
EXTRA = {
    "radius2_ragged": dict(hr_h=72, hr_w=88, lr_h=18, lr_w=22, n_text=24, radius=2),
    "radius4": dict(hr_h=160, hr_w=160, lr_h=40, lr_w=40, n_text=32, radius=4),
    "radius4_corr": dict(hr_h=160, hr_w=144, lr_h=40, lr_w=36, n_text=16, radius=4, lr_mode=1),
    "radius2_corr_ragged": dict(hr_h=100, hr_w=70, lr_h=25, lr_w=18, n_text=8, radius=2, lr_mode=1),
    "no_text_no_lr": dict(hr_h=48, hr_w=40, lr_h=0, lr_w=0, n_text=0, radius=1),
}



def _random_cases(n=96):
    """Seeded small geometries beyond the hand-picked ones: odd grids, windows
    of 2 to 16, radius 0 to 3, text 0 to 37 rows, rho 1 to 5, the default,
    an explicit (possibly overhanging or short) or no LR grid, both LR modes."""
    rng = np.random.default_rng([2026, 77])
    out = {}
    for i in range(n):
        H, W = int(rng.integers(1, 71)), int(rng.integers(1, 71))
        rho = int(rng.integers(1, 6))
        kind = int(rng.integers(0, 3))
        if kind == 0:
            lh = lw = None
        elif kind == 1:
            lh = lw = 0
        else:
            lh = int(rng.integers(1, -(-H // rho) + 4))
            lw = int(rng.integers(1, -(-W // rho) + 4))
        out[f"random{i:02d}"] = dict(hr_h=H, hr_w=W, lr_h=lh, lr_w=lw, n_text=int(rng.choice([0, 1, 5, 37])),
                                     radius=int(rng.integers(0, 4)), window=int(rng.choice([2, 4, 8, 16])), rho=rho,
                                     lr_mode=int(rng.integers(0, 2)))
    return out


EXTRA.update(_random_cases())
RANDOM = [k for k in EXTRA if k.startswith("random")]
NAMES = ["tiny", "tiny_masked", "small_ragged", "small_ragged_corr", "tiny_masked_corr", "ragged_corr_f32", "1k",
         "2k", "4k", "4k_corr", "4k_r2", "ragged"] + list(EXTRA)


def _case(name):
    if name in WORKLOADS:
        w = WORKLOADS[name]
        return U.desc_of(w, host_only=True), O.geometry_of(w)
    a = dict(EXTRA[name])
    lr_mode = a.pop("lr_mode", 0)
    window, rho = a.get("window", 16), a.get("rho", 4)
    desc = U.make_desc(a["hr_h"], a["hr_w"], a["lr_h"], a["lr_w"], a["n_text"], heads=2, head_dim=128,
                       dtype="bf16", window=window, radius=a["radius"], rho=rho, host_only=True, lr_mode=lr_mode)
    geo = O.geometry(a["hr_h"], a["hr_w"], a["n_text"], window=window, radius=a["radius"], rho=rho, lr_h=a["lr_h"],
                     lr_w=a["lr_w"], lr_mode=lr_mode)
    return desc, geo


def _raster_of_permuted(geo):
    """raster row of each permuted row, from the oracle's window-first orders"""
    T, N = geo.n_text, geo.n_hr
    hr = O.window_first_perm(geo.hr_h, geo.hr_w, geo.window)
    lr = O.lr_window_first_perm(geo) if geo.lr_mode == 1 else np.arange(geo.n_lr)
    return np.concatenate([np.arange(T), T + hr, T + N + lr]).astype(np.int64)


class _OracleSets:
    """Boolean raster masks of the oracle's allowed keys / queries, one per
    coordinates class (kind, window)."""

    def __init__(self, geo):
        self.geo = geo
        self.coords = O.token_coords(geo)
        kind, _, _, wy, wx = self.coords
        self.cls = np.stack([kind, wy, wx], 1)
        self.keys, self.queries = {}, {}

    def _mask(self, cache, fn, row):
        c = tuple(self.cls[row])
        if c not in cache:
            m = np.zeros(self.geo.seq_len, bool)
            m[fn(self.geo, self.coords, int(row))] = True
            cache[c] = m
        return cache[c]

    def keys_of(self, row):
        return self._mask(self.keys, O.allowed_keys_of, row)

    def queries_of(self, row):
        return self._mask(self.queries, O.allowed_queries_of, row)


def _union(ranges, sel, L, to_raster):
    """raster boolean mask of the union of ranges[sel]; ranges must be disjoint"""
    m = np.zeros(L, bool)
    n = 0
    for k0, k1 in ranges[sel]:
        assert 0 <= k0 < k1 <= L, (k0, k1, L)
        m[k0:k1] = True
        n += k1 - k0
    assert m.sum() == n, "ranges overlap"
    out = np.zeros(L, bool)
    out[to_raster[m]] = True
    return out


@pytest.mark.parametrize("name", NAMES)
def test_query_tiles_expand_to_the_oracle_mask(name):
    desc, geo = _case(name)
    p = U.ug_plan(desc)
    b = U.ug_plan_export_blocks(p)
    L = geo.seq_len
    to_raster = _raster_of_permuted(geo)
    sets = _OracleSets(geo)
    covered = np.zeros(L, np.int64)
    pairs = 0
    for tile in b["q_tiles"]:
        q0, q1, r0, r1 = (int(x) for x in tile)
        assert 0 <= q0 < q1 <= L and q1 - q0 <= 256 and r0 < r1
        covered[q0:q1] += 1
        keys = _union(b["k_ranges"], slice(r0, r1), L, to_raster)
        for row in to_raster[q0:q1]:
            assert np.array_equal(keys, sets.keys_of(row)), (name, int(row))
        pairs += (q1 - q0) * int(keys.sum())
    assert np.all(covered == 1), "query tiles must partition the rows"
    assert pairs == O.pair_count(geo) == p.info["pairs_per_head"]


@pytest.mark.parametrize("name", NAMES)
def test_key_tiles_expand_to_the_oracle_mask(name):
    desc, geo = _case(name)
    p = U.ug_plan(desc)
    b = U.ug_plan_export_blocks(p)
    L = geo.seq_len
    to_raster = _raster_of_permuted(geo)
    sets = _OracleSets(geo)
    covered = np.zeros(L, np.int64)
    pairs = 0
    masked_tiles = 0
    for u, tile in enumerate(b["k_tiles"]):
        k0, k1, r0, r1 = (int(x) for x in tile)
        assert 0 <= k0 < k1 <= L and k1 - k0 <= 256 and r0 < r1
        covered[k0:k1] += 1
        off = int(b["mask_off"][u])
        if off < 0:
            queries = _union(b["q_ranges"], slice(r0, r1), L, to_raster)
            for row in to_raster[k0:k1]:
                assert np.array_equal(queries, sets.queries_of(row)), (name, int(row))
            pairs += (k1 - k0) * int(queries.sum())
            continue
        masked_tiles += 1
        assert r1 - r0 <= 64
        for j in range(k1 - k0):
            bits = int(b["masks"][off + j])
            assert bits >> (r1 - r0) == 0, "mask bits past the tile's ranges"
            sel = np.array([r0 + r for r in range(r1 - r0) if (bits >> r) & 1], np.int64)
            queries = _union(b["q_ranges"], sel, L, to_raster) if sel.size else np.zeros(L, bool)
            row = to_raster[k0 + j]
            assert np.array_equal(queries, sets.queries_of(row)), (name, int(row))
            pairs += int(queries.sum())
    assert np.all(covered == 1), "key tiles must partition the rows"
    assert pairs == O.pair_count(geo)
    if geo.lr_mode == 1 and geo.n_lr:
        assert masked_tiles > 0  # the grouped LR key tiles carry masks


def _first_mismatch(blocks, geo):
    """first query row whose expanded key set differs from the oracle's, or None"""
    L = geo.seq_len
    to_raster = _raster_of_permuted(geo)
    sets = _OracleSets(geo)
    for tile in blocks["q_tiles"]:
        q0, q1, r0, r1 = (int(x) for x in tile)
        keys = _union(blocks["k_ranges"], slice(r0, r1), L, to_raster)
        for row in to_raster[q0:q1]:
            if not np.array_equal(keys, sets.keys_of(row)):
                return int(row)
    return None


@pytest.mark.parametrize("name", ["tiny_masked", "small_ragged", "1k"])
def test_expansion_catches_a_shifted_range(name):
    """A range moved by one row keeps its length (and every pair count) but
    must fail the expansion check."""
    desc, geo = _case(name)
    b = U.ug_plan_export_blocks(U.ug_plan(desc))
    assert _first_mismatch(b, geo) is None
    # shift an HR window range of some tile down by one row, inside [0, L)
    T, N = geo.n_text, geo.n_hr
    r = next(i for i, (k0, k1) in enumerate(b["k_ranges"]) if T < k0 and k1 < T + N)
    bad = {k: v.copy() for k, v in b.items()}
    bad["k_ranges"][r] -= 1
    assert _first_mismatch(bad, geo) is not None
