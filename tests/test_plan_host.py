"""Host-side tests of the C-ABI library (no GPU): symbol exports, descriptor
validation, and bit-exact plan tables against the oracle's coordinate-derived
window-first order, window offsets and neighbourhoods."""
import ctypes
import os
import re

import numpy as np
import pytest

import diffusion_transformer_sparse_amd as U
from oracle import ultragen_oracle as O
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "ultragen.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(ug_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(U.EXPORTED), names
    lib = ctypes.CDLL(U.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_debug_library_exports_its_symbols():
    """The bounds-checking build exports the calls include/ultragen_debug.h
    declares, besides every release entry point; the release build does not."""
    with open(os.path.join(ROOT, "include", "ultragen_debug.h")) as f:
        names = sorted(set(re.findall(r"^\s*ug_status\s+(ug_\w+)\s*\(", f.read(), re.M)))
    assert set(names) == set(U.DEBUG_EXPORTED), names
    if not os.path.exists(U.DEBUG_LIB_PATH):
        pytest.skip("libultragen_debug.so is not built")
    dbg = ctypes.CDLL(U.DEBUG_LIB_PATH)
    for n in names + header_functions():
        assert hasattr(dbg, n), n
    rel = ctypes.CDLL(U.LIB_PATH)
    for n in names:
        assert not hasattr(rel, n), n


def test_status_strings():
    assert U.ug_status_str(0) == "UG_OK"
    assert U.ug_status_str(1) == "UG_ERR_INVALID_ARGUMENT"
    assert U.ug_status_str(4) == "UG_ERR_HIP"


def _host_plan(w):
    return U.ug_plan(U.desc_of(w, host_only=True))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_plan_tables_bit_exact(name):
    w = WORKLOADS[name]
    p = _host_plan(w)
    t = U.ug_plan_export(p)
    assert np.array_equal(t["perm"], O.window_first_perm(w.hr_h, w.hr_w, w.window))
    assert np.array_equal(t["win_off"], O.window_offsets(w.hr_h, w.hr_w, w.window))
    nbr, off = O.neighbour_windows(w.hr_h, w.hr_w, w.window, w.radius)
    assert np.array_equal(t["nbr"], nbr) and np.array_equal(t["nbr_off"], off)
    geo = O.geometry_of(w)
    info = p.info
    assert info["pairs_per_head"] == O.pair_count(geo)
    assert info["seq_len"] == geo.seq_len and info["n_lr"] == geo.n_lr
    assert info["eff_flops"] == 4.0 * w.head_dim * info["pairs_per_head"] * w.heads * w.batch
    lr = U.ug_plan_export_lr(p)
    if w.lr_mode == 1:
        assert np.array_equal(lr["lr_perm"], O.lr_window_first_perm(geo))
        assert np.array_equal(lr["lr_win_off"], O.lr_window_offsets(geo))
    else:
        assert np.array_equal(lr["lr_perm"], np.arange(w.n_lr))
    p.close()


@pytest.mark.parametrize("H,W,l,r,T,lh,lw,rho", [(3, 5, 2, 1, 2, 1, 2, 2), (17, 33, 16, 1, 0, 5, 9, 4),
                                                  (64, 48, 32, 1, 5, 16, 12, 4), (20, 20, 64, 0, 3, 5, 5, 4),
                                                  (33, 65, 16, 0, 0, 9, 17, 4), (8, 8, 4, 1, 1, 4, 4, 2),
                                                  (30, 30, 8, 2, 4, 20, 3, 2), (16, 16, 16, 1, 2, 1, 1, 1)])
def test_corresponding_lr_tables(H, W, l, r, T, lh, lw, rho):
    """lr_mode 1: LR window-first order, LR window offsets and the exact pair
    count (hence the key ranges) agree with the oracle, also where LR
    anchors overhang the window grid."""
    d = U.make_desc(H, W, lh, lw, T, 2, 64, "f32", window=l, radius=r, rho=rho, host_only=True, lr_mode=1)
    p = U.ug_plan(d)
    geo = O.Geometry(H, W, lh, lw, T, l, r, rho, lr_mode=1)
    lr = U.ug_plan_export_lr(p)
    assert np.array_equal(lr["lr_perm"], O.lr_window_first_perm(geo))
    assert np.array_equal(lr["lr_win_off"], O.lr_window_offsets(geo))
    assert p.info["pairs_per_head"] == O.pair_count(geo) == int(O.allowed_dense(geo).sum())


@pytest.mark.parametrize("H,W,l,r,rho", [(160, 160, 16, 4, 4), (96, 80, 8, 4, 2), (160, 160, 16, 3, 4),
                                         (72, 72, 8, 5, 4)])
def test_corresponding_lr_key_tiles_at_large_radius(H, W, l, r, rho):
    """lr_mode 1 key-major view where one window's neighbourhood alone exceeds
    the 64 query ranges a key tile may hold (interior windows at radius >= 4):
    those windows get plain key tiles, the rest grouped, masked ones.  The
    plan checks internally that the masked transpose counts the forward's
    pairs; the count itself must equal the oracle's."""
    lh, lw = -(-H // rho), -(-W // rho)
    d = U.make_desc(H, W, lh, lw, 5, 2, 64, "f32", window=l, radius=r, rho=rho, host_only=True, lr_mode=1)
    p = U.ug_plan(d)
    assert p.info["pairs_per_head"] == O.pair_count(O.Geometry(H, W, lh, lw, 5, l, r, rho, lr_mode=1))
    p.close()


@pytest.mark.parametrize("H,W,l,r,T,lh,lw", [(3, 5, 2, 1, 2, 1, 2), (17, 33, 16, 1, 0, 5, 9), (40, 40, 8, 2, 7, 0, 0),
                                              (64, 48, 32, 1, 5, 16, 12), (20, 20, 64, 0, 3, 5, 5),
                                              (33, 65, 16, 0, 0, 9, 17)])
def test_plan_odd_geometries(H, W, l, r, T, lh, lw):
    d = U.make_desc(H, W, lh, lw, T, 2, 64, "f32", window=l, radius=r, host_only=True)
    p = U.ug_plan(d)
    t = U.ug_plan_export(p)
    assert np.array_equal(t["perm"], O.window_first_perm(H, W, l))
    assert np.array_equal(t["win_off"], O.window_offsets(H, W, l))
    nbr, off = O.neighbour_windows(H, W, l, r)
    assert np.array_equal(t["nbr"], nbr) and np.array_equal(t["nbr_off"], off)
    geo = O.Geometry(H, W, lh, lw, T, l, r, 4)
    assert p.info["pairs_per_head"] == O.pair_count(geo) == int(O.allowed_dense(geo).sum())


def test_rope_table_rows_cover_scaled_lr_positions():
    w = WORKLOADS["ragged"]
    p = _host_plan(w)
    assert p.info["rope_positions"] == max(w.hr_h, w.hr_w, 4 * (w.lr_h - 1) + 1, 4 * (w.lr_w - 1) + 1)
    w2 = w.with_(lr_h=80, lr_w=120)   # LR grid reaching past the HR grid
    p2 = _host_plan(w2)
    assert p2.info["rope_positions"] == 4 * 119 + 1


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, U.UgError), ("heads", 0, U.UgError), ("head_dim", 6, U.UgError), ("hr_h", 0, U.UgError),
    ("lr_w", -1, U.UgError), ("n_text", -3, U.UgError), ("window", 0, U.UgError), ("radius", -1, U.UgError),
    ("rho", 0, U.UgError), ("dtype", 7, U.UgError), ("flags", 8, U.UgError), ("rope_theta", -1.0, U.UgError),
    ("lr_mode", 2, U.UgError), ("lr_mode", -1, U.UgError)])
def test_descriptor_validation(field, value, status):
    d = U.desc_of(WORKLOADS["tiny"], host_only=True)
    setattr(d, field, value)
    with pytest.raises(status) as e:
        U.ug_plan(d)
    assert e.value.status == 1  # UG_ERR_INVALID_ARGUMENT
    assert "ug_plan" in U.ug_last_error()


@pytest.mark.parametrize("H,W,rho", [(32, 32, 4), (37, 45, 4), (250, 380, 4), (40, 36, 3), (17, 5, 1)])
def test_zero_lr_grid_is_the_scaled_grid(H, W, rho):
    """A 0 x 0 LR grid is the one the coordinate scaling implies (one LR
    token per rho x rho block, ceil division); UG_PLAN_NO_LR gives none.
    (UltraGen notes, 关键设计 2: LR positions scaled by rho.)"""
    dflt = U.ug_plan(U.make_desc(H, W, None, None, 8, 2, 64, "f32", rho=rho, host_only=True))
    assert dflt.info["n_lr"] == -(-H // rho) * -(-W // rho)
    explicit = U.ug_plan(U.make_desc(H, W, -(-H // rho), -(-W // rho), 8, 2, 64, "f32", rho=rho, host_only=True))
    a, b = U.ug_plan_export_blocks(dflt), U.ug_plan_export_blocks(explicit)
    assert a.keys() == b.keys() and all(np.array_equal(a[k], b[k]) for k in a)
    assert dflt.info["seq_len"] == explicit.info["seq_len"]
    none = U.ug_plan(U.make_desc(H, W, 0, 0, 8, 2, 64, "f32", rho=rho, host_only=True))
    assert none.info["n_lr"] == 0 and none.info["seq_len"] == 8 + H * W


def test_lr_grid_flag_errors():
    d = U.make_desc(16, 16, 4, 4, 0, 2, 64, "f32", host_only=True)
    d.flags |= U.UG_PLAN_NO_LR
    with pytest.raises(U.UgError):
        U.ug_plan(d)
    d = U.make_desc(16, 16, 4, 4, 0, 2, 64, "f32", host_only=True)
    d.lr_h = 0
    with pytest.raises(U.UgError):
        U.ug_plan(d)


def test_host_only_plan_rejects_device_calls():
    p = _host_plan(WORKLOADS["tiny"])
    lib = U.lib()
    st = lib.ug_permute(p.handle, ctypes.c_void_p(16), ctypes.c_void_p(4096), None)
    assert st == 1 and "host-only" in U.ug_last_error()
    st = lib.ug_attn_fwd(p.handle, *(ctypes.c_void_p(16 * (i + 1)) for i in range(4)), None, None)
    assert st == 1
    st = lib.ug_permute(None, ctypes.c_void_p(16), ctypes.c_void_p(4096), None)
    assert st == 1 and "NULL" in U.ug_last_error()


def test_null_arguments():
    lib = U.lib()
    assert lib.ug_plan(None, None) == 1
    assert lib.ug_plan_info(None, None) == 1
    assert lib.ug_plan_free(None) == 0


@pytest.mark.parametrize("name", ["tiny", "tiny_masked", "small_ragged", "small_ragged_corr", "1k", "4k", "ragged",
                                  "4k_corr"])
def test_work_queues_cover_every_item_once(name):
    """The per-XCD work queues (item k*8 + x is the k-th of XCD x's queue) hold
    every (task, batch*head) pair exactly once, each queue's items before its
    padding: the persistent grids take a cursor on padding to mean that queue
    is empty, so a real item after padding would never run."""
    w = WORKLOADS[name]
    p = _host_plan(w)
    info = p.info
    bh = w.batch * w.heads
    q = U.ug_plan_export_queues(p)
    for items, n_tasks in ((q["attn"], info["attn_tasks"]), (q["bwd"], info["bwd_key_tasks"])):
        assert len(items) % 8 == 0
        per_xcd = items.reshape(-1, 8, 2)
        for x in range(8):
            real = per_xcd[:, x, 0] >= 0
            n_real = int(real.sum())
            assert real[:n_real].all() and not real[n_real:].any(), f"padding inside XCD {x}'s queue"
        r = items[items[:, 0] >= 0].astype(np.int64)
        assert r[:, 0].max() < n_tasks and r[:, 1].min() >= 0 and r[:, 1].max() < bh
        keys = r[:, 0] * bh + r[:, 1]
        assert len(np.unique(keys)) == len(keys) == n_tasks * bh


def test_work_queue_order_4k():
    """The attention's work order at 4K (performance choices, pinned so they
    do not drift): each queue starts with long items (the text query tiles),
    a head's long items all sit on one XCD, the window tiles follow in
    Z-order of their window, and each queue ends with its short items (the
    LR query tiles)."""
    w = WORKLOADS["4k"]
    p = _host_plan(w)
    T, N = w.n_text, w.n_hr
    ex = U.ug_plan_export(p)
    gx = w.hr_w // w.window
    q = U.ug_plan_export_queues(p)["attn"].reshape(-1, 8, 2)
    # task ids: text tiles, then LR tiles, then one per window (4K: whole 256-token windows)
    n_text_tiles, n_lr_tiles = -(-T // 256), -(-w.n_lr // 256)
    kind = lambda t: "text" if t < n_text_tiles else "lr" if t < n_text_tiles + n_lr_tiles else "win"
    xcd_of_text_head = {}
    for x in range(8):
        items = [(int(t), int(bh)) for t, bh in q[:, x] if t >= 0]
        kinds = [kind(t) for t, _ in items]
        n_long = kinds.count("text")
        assert kinds[:n_long] == ["text"] * n_long, f"XCD {x}: long items first"
        n_lr = kinds.count("lr")
        assert kinds[len(kinds) - n_lr:] == ["lr"] * n_lr, f"XCD {x}: short items last"
        for t, bh in items[:n_long]:
            assert xcd_of_text_head.setdefault(bh, x) == x, f"head {bh}'s long items on two XCDs"
        # window tiles of one head follow in increasing Z-order of their window
        def morton(wi):
            y, xx, m = wi // gx, wi % gx, 0
            for b in range(8):
                m |= ((y >> b) & 1) << (2 * b + 1) | ((xx >> b) & 1) << (2 * b)
            return m
        last = {}
        for t, bh in items:
            if kind(t) == "win":
                z = morton(t - n_text_tiles - n_lr_tiles)
                assert z > last.get(bh, -1), f"XCD {x}: head {bh} windows out of Z-order"
                last[bh] = z
    assert len(xcd_of_text_head) == w.batch * w.heads


@pytest.mark.parametrize("field,value", [("batch", 0), ("hr_h", 0), ("lr_w", 0), ("rho", 0), ("channels", 12),
                                         ("channels", 0), ("dtype", 5), ("alpha", 1.5), ("alpha", -0.1),
                                         ("alpha", float("nan")), ("sharpen", -1.0), ("sharpen", float("inf"))])
def test_warm_start_descriptor_validation(field, value):
    """Invalid warm-start descriptors are rejected before any HIP call."""
    d = U.UgWarmDesc(batch=1, hr_h=16, hr_w=16, lr_h=4, lr_w=4, channels=16, rho=4, dtype=U.UG_BF16, alpha=0.5,
                     sharpen=0.5)
    setattr(d, field, value)
    st = U.lib().ug_warm_start(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(4096),
                               ctypes.c_void_p(1 << 20), None)
    assert st == 1 and "ug_warm_start" in U.ug_last_error()


def test_warm_start_rejects_overlap_and_null():
    d = U.UgWarmDesc(batch=1, hr_h=16, hr_w=16, lr_h=4, lr_w=4, channels=16, rho=4, dtype=U.UG_BF16, alpha=0.5,
                     sharpen=0.5)
    lib = U.lib()
    assert lib.ug_warm_start(None, None, None, None, None) == 1
    assert lib.ug_warm_start(ctypes.byref(d), None, ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20), None) == 1
    # x_hr starting inside noise (partial overlap)
    assert lib.ug_warm_start(ctypes.byref(d), ctypes.c_void_p(16), ctypes.c_void_p(1 << 20),
                             ctypes.c_void_p((1 << 20) + 256), None) == 1
    # x_hr overlapping x_lr
    assert lib.ug_warm_start(ctypes.byref(d), ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24),
                             ctypes.c_void_p((1 << 20) - 4096), None) == 1
