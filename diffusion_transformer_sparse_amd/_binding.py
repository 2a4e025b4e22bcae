"""ctypes binding of libultragen.so (the C ABI in include/ultragen.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current HIP stream.  The
library must be built (``python -m diffusion_transformer_sparse_amd.build``);
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_int32, c_int64, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libultragen.so")
# the same sources built with index checks that record violations in a device
# word (UG_BOUNDS_CHECK); see use_library and debug_bounds
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libultragen_debug.so")

UG_OK, UG_ERR_INVALID_ARGUMENT, UG_ERR_UNSUPPORTED, UG_ERR_OUT_OF_MEMORY, UG_ERR_HIP, UG_ERR_INTERNAL = range(6)
UG_F32, UG_BF16 = 0, 1
UG_PLAN_HOST_ONLY = 1
UG_PLAN_NO_LR = 2

EXPORTED = ("ug_plan", "ug_plan_free", "ug_plan_info", "ug_plan_export", "ug_plan_export_lr", "ug_plan_export_queues",
            "ug_plan_export_blocks", "ug_permute",
            "ug_unpermute",
            "ug_rope2d", "ug_attn_fwd", "ug_permute_rope", "ug_attn_fwd_raster", "ug_attn_fwd_lse", "ug_attn_bwd",
            "ug_attn_bwd_noalloc",
            "ug_rope2d_bwd", "ug_permute_rope_bwd", "ug_warm_start", "ug_status_str", "ug_last_error")


class UgDesc(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("heads", c_int32), ("head_dim", c_int32), ("hr_h", c_int32),
                ("hr_w", c_int32), ("lr_h", c_int32), ("lr_w", c_int32), ("n_text", c_int32),
                ("window", c_int32), ("radius", c_int32), ("rho", c_int32), ("dtype", c_int32),
                ("flags", c_int32), ("lr_mode", c_int32), ("rope_theta", c_double)]


class UgWarmDesc(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("hr_h", c_int32), ("hr_w", c_int32), ("lr_h", c_int32), ("lr_w", c_int32),
                ("channels", c_int32), ("rho", c_int32), ("dtype", c_int32), ("alpha", ctypes.c_float),
                ("sharpen", ctypes.c_float)]


class UgInfo(ctypes.Structure):
    _fields_ = [("seq_len", c_int64), ("n_hr", c_int64), ("n_lr", c_int64), ("n_text", c_int64),
                ("grid_y", c_int32), ("grid_x", c_int32), ("n_windows", c_int32), ("max_neighbours", c_int32),
                ("n_neighbour_entries", c_int64), ("pairs_per_head", c_int64), ("eff_flops", c_double),
                ("workspace_bytes", c_int64), ("attn_tasks", c_int64), ("attn_blocks", c_int64),
                ("attn_key_tiles", c_int64), ("rope_positions", c_int64), ("bwd_workspace_bytes", c_int64),
                ("bwd_key_tasks", c_int64), ("bwd_blocks", c_int64), ("attn_ranges", c_int64),
                ("bwd_key_ranges", c_int64), ("bwd_mask_words", c_int64)]


class UgError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {status_name(status)}: {msg}")
        self.status = status


_lib = None


_libs = {}


def use_library(path: str = LIB_PATH):
    """Make every entry point of this module call the library at `path`
    (LIB_PATH, or DEBUG_LIB_PATH for the bounds-checking build).  Plans are
    tied to the library that built them."""
    global _lib
    _lib = _load(path)
    return _lib


def lib():
    """Load libultragen.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def _load(path):
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m diffusion_transformer_sparse_amd.build` (no fallback exists)")
        L = ctypes.CDLL(path)
        L.ug_plan.argtypes = [POINTER(UgDesc), POINTER(c_void_p)]
        L.ug_plan_free.argtypes = [c_void_p]
        L.ug_plan_info.argtypes = [c_void_p, POINTER(UgInfo)]
        L.ug_plan_export.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.ug_plan_export_lr.argtypes = [c_void_p, c_void_p, c_void_p]
        L.ug_plan_export_queues.argtypes = [c_void_p, c_void_p, c_void_p]
        L.ug_plan_export_blocks.argtypes = [c_void_p] * 7
        L.ug_permute.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.ug_unpermute.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.ug_rope2d.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p]
        L.ug_attn_fwd.argtypes = [c_void_p] * 7
        L.ug_attn_fwd_raster.argtypes = [c_void_p] * 7
        L.ug_permute_rope.argtypes = [c_void_p] * 6
        L.ug_attn_fwd_lse.argtypes = [c_void_p] * 8
        L.ug_attn_bwd.argtypes = [c_void_p] * 12
        L.ug_attn_bwd_noalloc.argtypes = [c_void_p] * 11
        L.ug_rope2d_bwd.argtypes = [c_void_p] * 4
        L.ug_permute_rope_bwd.argtypes = [c_void_p] * 6
        L.ug_warm_start.argtypes = [POINTER(UgWarmDesc), c_void_p, c_void_p, c_void_p, c_void_p]
        L.ug_status_str.argtypes = [c_int32]
        L.ug_status_str.restype = c_char_p
        L.ug_last_error.argtypes = []
        L.ug_last_error.restype = c_char_p
        for name in ("ug_plan", "ug_plan_free", "ug_plan_info", "ug_plan_export", "ug_plan_export_lr",
                     "ug_plan_export_queues", "ug_plan_export_blocks", "ug_permute",
                     "ug_unpermute",
                     "ug_rope2d", "ug_attn_fwd", "ug_permute_rope", "ug_attn_fwd_raster", "ug_attn_fwd_lse",
                     "ug_attn_bwd", "ug_attn_bwd_noalloc", "ug_rope2d_bwd", "ug_permute_rope_bwd", "ug_warm_start"):
            getattr(L, name).restype = c_int32
        for name in DEBUG_EXPORTED:
            if hasattr(L, name):
                getattr(L, name).argtypes = [c_void_p, c_int32]
                getattr(L, name).restype = c_int32
        _libs[path] = L
    return _libs[path]


DEBUG_EXPORTED = ("ug_debug_bounds_fwd", "ug_debug_bounds_bwd", "ug_debug_bounds_warm")


def debug_bounds(clear: bool = True) -> dict:
    """Violation words of the debug build's kernels (forward and layout,
    backward, warm start), each cleared after reading if `clear`; raises on the
    release build, which has no such words."""
    L = lib()
    out = {}
    for name in DEBUG_EXPORTED:
        if not hasattr(L, name):
            raise RuntimeError("debug_bounds needs the debug build (use_library(DEBUG_LIB_PATH))")
        w = ctypes.c_uint32(0)
        _check(name, getattr(L, name)(ctypes.byref(w), int(clear)))
        out[name[len("ug_debug_bounds_"):]] = w.value
    return out


def status_name(s: int) -> str:
    return lib().ug_status_str(int(s)).decode()


def ug_status_str(s: int) -> str:
    return status_name(s)


def ug_last_error() -> str:
    return lib().ug_last_error().decode()


def _check(fn, status):
    if status != UG_OK:
        raise UgError(fn, status, ug_last_error())


def make_desc(hr_h, hr_w, lr_h, lr_w, n_text, heads, head_dim, dtype="bf16", window=16, radius=1, rho=4,
              rope_theta=10000.0, batch=1, host_only=False, lr_mode=0) -> UgDesc:
    """lr_h = lr_w = 0: no LR tokens (flag UG_PLAN_NO_LR); None, None: the
    grid the coordinate scaling implies, ceil(hr_h/rho) x ceil(hr_w/rho)
    (the C-ABI's 0 x 0)."""
    flags = UG_PLAN_HOST_ONLY if host_only else 0
    if lr_h is None and lr_w is None:
        lr_h = lr_w = 0
    elif lr_h == 0 and lr_w == 0:
        flags |= UG_PLAN_NO_LR
    return UgDesc(batch=batch, heads=heads, head_dim=head_dim, hr_h=hr_h, hr_w=hr_w, lr_h=lr_h, lr_w=lr_w,
                  n_text=n_text, window=window, radius=radius, rho=rho,
                  dtype=UG_BF16 if dtype in ("bf16", UG_BF16) else UG_F32,
                  flags=flags, lr_mode=lr_mode, rope_theta=rope_theta)


def desc_of(w, host_only=False) -> UgDesc:
    """Descriptor of a workloads.Workload (duck-typed)."""
    return make_desc(w.hr_h, w.hr_w, w.lr_h, w.lr_w, w.n_text, w.heads, w.head_dim, w.dtype, w.window,
                     w.radius, w.rho, w.rope_theta, w.batch, host_only, getattr(w, "lr_mode", 0))


class Plan:
    """Owning handle of a ug_plan_t."""

    def __init__(self, desc: UgDesc):
        h = c_void_p()
        self.lib = lib()  # the library that built the plan frees it
        _check("ug_plan", self.lib.ug_plan(byref(desc), byref(h)))
        self.handle = h
        self.desc = desc
        self.info = ug_plan_info(self)

    def close(self):
        if self.handle:
            self.lib.ug_plan_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    @property
    def shape(self):
        d = self.desc
        return (d.batch, self.info["seq_len"], d.heads, d.head_dim)


def ug_plan(desc: UgDesc) -> Plan:
    return Plan(desc)


def ug_plan_free(plan: Plan) -> None:
    plan.close()


def ug_plan_info(plan: Plan) -> dict:
    info = UgInfo()
    _check("ug_plan_info", lib().ug_plan_info(plan.handle, byref(info)))
    return {name: getattr(info, name) for name, _ in UgInfo._fields_}


def ug_plan_export(plan: Plan) -> dict:
    info = plan.info
    perm = np.empty(info["n_hr"], np.int32)
    win_off = np.empty(info["n_windows"] + 1, np.int32)
    nbr = np.empty(max(1, info["n_neighbour_entries"]), np.int32)
    nbr_off = np.empty(info["n_windows"] + 1, np.int32)
    _check("ug_plan_export", lib().ug_plan_export(plan.handle, perm.ctypes.data, win_off.ctypes.data,
                                                  nbr.ctypes.data, nbr_off.ctypes.data))
    return {"perm": perm, "win_off": win_off, "nbr": nbr[:info["n_neighbour_entries"]], "nbr_off": nbr_off}


def ug_plan_export_queues(plan: Plan) -> dict:
    """Per-XCD work queues as [n, 2] (task, batch*head) arrays; task -1 = padding."""
    info = plan.info
    attn = np.empty((max(1, info["attn_blocks"]), 2), np.int32)
    bwd = np.empty((max(1, info["bwd_blocks"]), 2), np.int32)
    _check("ug_plan_export_queues", lib().ug_plan_export_queues(plan.handle, attn.ctypes.data, bwd.ctypes.data))
    return {"attn": attn[:info["attn_blocks"]], "bwd": bwd[:info["bwd_blocks"]]}


def ug_plan_export_lr(plan: Plan) -> dict:
    info = plan.info
    lr_perm = np.empty(max(1, info["n_lr"]), np.int32)
    lr_win_off = np.empty(info["n_windows"] + 2, np.int32)
    _check("ug_plan_export_lr", lib().ug_plan_export_lr(plan.handle, lr_perm.ctypes.data, lr_win_off.ctypes.data))
    return {"lr_perm": lr_perm[:info["n_lr"]], "lr_win_off": lr_win_off}


def ug_plan_export_blocks(plan: Plan) -> dict:
    """The block lists the attention kernels walk: query tiles [n, 4] (q0, q1,
    r0, r1) with key ranges [m, 2] (k0, k1), and the backward's key tiles with
    their query ranges and per-key 64-bit range masks (mask_off -1: unmasked)."""
    info = plan.info
    q_tiles = np.empty((max(1, info["attn_tasks"]), 4), np.int32)
    k_ranges = np.empty((max(1, info["attn_ranges"]), 2), np.int32)
    k_tiles = np.empty((max(1, info["bwd_key_tasks"]), 4), np.int32)
    q_ranges = np.empty((max(1, info["bwd_key_ranges"]), 2), np.int32)
    mask_off = np.empty(max(1, info["bwd_key_tasks"]), np.int32)
    masks = np.empty(max(1, info["bwd_mask_words"]), np.uint64)
    _check("ug_plan_export_blocks", lib().ug_plan_export_blocks(
        plan.handle, q_tiles.ctypes.data, k_ranges.ctypes.data, k_tiles.ctypes.data, q_ranges.ctypes.data,
        mask_off.ctypes.data, masks.ctypes.data))
    return {"q_tiles": q_tiles[:info["attn_tasks"]], "k_ranges": k_ranges[:info["attn_ranges"]],
            "k_tiles": k_tiles[:info["bwd_key_tasks"]], "q_ranges": q_ranges[:info["bwd_key_ranges"]],
            "mask_off": mask_off[:info["bwd_key_tasks"]], "masks": masks[:info["bwd_mask_words"]]}


# ---------------------------------------------------------------- device calls

def _torch():
    import torch
    return torch


def _stream_ptr(t):
    torch = _torch()
    return c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check_tensor(plan: Plan, t, name):
    torch = _torch()
    want = torch.bfloat16 if plan.desc.dtype == UG_BF16 else torch.float32
    if not t.is_cuda or t.dtype != want or not t.is_contiguous() or tuple(t.shape) != plan.shape:
        raise ValueError(f"{name}: expected a contiguous {want} CUDA tensor of shape {plan.shape}, "
                         f"got {tuple(t.shape)} {t.dtype} on {t.device} contiguous={t.is_contiguous()}")


def ug_permute(plan: Plan, x_raster, x_perm=None):
    _check_tensor(plan, x_raster, "x_raster")
    if x_perm is None:
        x_perm = _torch().empty_like(x_raster)
    _check_tensor(plan, x_perm, "x_perm")
    _check("ug_permute", lib().ug_permute(plan.handle, c_void_p(x_raster.data_ptr()), c_void_p(x_perm.data_ptr()),
                                          _stream_ptr(x_raster)))
    return x_perm


def ug_unpermute(plan: Plan, x_perm, x_raster=None):
    _check_tensor(plan, x_perm, "x_perm")
    if x_raster is None:
        x_raster = _torch().empty_like(x_perm)
    _check_tensor(plan, x_raster, "x_raster")
    _check("ug_unpermute", lib().ug_unpermute(plan.handle, c_void_p(x_perm.data_ptr()),
                                              c_void_p(x_raster.data_ptr()), _stream_ptr(x_perm)))
    return x_raster


def ug_rope2d(plan: Plan, q_perm, k_perm):
    _check_tensor(plan, q_perm, "q_perm")
    _check_tensor(plan, k_perm, "k_perm")
    _check("ug_rope2d", lib().ug_rope2d(plan.handle, c_void_p(q_perm.data_ptr()), c_void_p(k_perm.data_ptr()),
                                        _stream_ptr(q_perm)))
    return q_perm, k_perm


def ug_attn_fwd(plan: Plan, q, k, v, o=None, workspace=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(plan, t, n)
    if o is None:
        o = _torch().empty_like(q)
    _check_tensor(plan, o, "o")
    ws = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p()
    _check("ug_attn_fwd", lib().ug_attn_fwd(plan.handle, c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                            c_void_p(v.data_ptr()), c_void_p(o.data_ptr()), ws, _stream_ptr(q)))
    return o


def ug_permute_rope(plan: Plan, q_raster, k_raster, q_perm=None, k_perm=None):
    _check_tensor(plan, q_raster, "q_raster")
    _check_tensor(plan, k_raster, "k_raster")
    if q_perm is None:
        q_perm = _torch().empty_like(q_raster)
    if k_perm is None:
        k_perm = _torch().empty_like(k_raster)
    _check_tensor(plan, q_perm, "q_perm")
    _check_tensor(plan, k_perm, "k_perm")
    _check("ug_permute_rope", lib().ug_permute_rope(plan.handle, c_void_p(q_raster.data_ptr()),
                                                    c_void_p(k_raster.data_ptr()), c_void_p(q_perm.data_ptr()),
                                                    c_void_p(k_perm.data_ptr()), _stream_ptr(q_raster)))
    return q_perm, k_perm


def ug_attn_fwd_raster(plan: Plan, q, k, v, o_raster=None, workspace=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(plan, t, n)
    if o_raster is None:
        o_raster = _torch().empty_like(q)
    _check_tensor(plan, o_raster, "o_raster")
    ws = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p()
    _check("ug_attn_fwd_raster", lib().ug_attn_fwd_raster(plan.handle, c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                                          c_void_p(v.data_ptr()), c_void_p(o_raster.data_ptr()), ws,
                                                          _stream_ptr(q)))
    return o_raster


def _lse_shape(plan: Plan):
    return (plan.desc.batch, plan.desc.heads, plan.info["seq_len"])


def ug_attn_fwd_lse(plan: Plan, q, k, v, o=None, lse=None, workspace=None):
    """ug_attn_fwd that also returns the natural-log LSE of every row,
    float32 [B, Hh, L] in the permuted row order."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(plan, t, n)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(_lse_shape(plan), dtype=torch.float32, device=q.device)
    _check_tensor(plan, o, "o")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != _lse_shape(plan):
        raise ValueError(f"lse: expected a contiguous float32 tensor of shape {_lse_shape(plan)}")
    ws = c_void_p(workspace.data_ptr()) if workspace is not None else c_void_p()
    _check("ug_attn_fwd_lse", lib().ug_attn_fwd_lse(plan.handle, c_void_p(q.data_ptr()), c_void_p(k.data_ptr()),
                                                    c_void_p(v.data_ptr()), c_void_p(o.data_ptr()),
                                                    c_void_p(lse.data_ptr()), ws, _stream_ptr(q)))
    return o, lse


def bwd_workspace(plan: Plan, device="cuda"):
    torch = _torch()
    return torch.empty(plan.info["bwd_workspace_bytes"], dtype=torch.uint8, device=device)


def ug_attn_bwd(plan: Plan, q, k, v, o, d_o, lse, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of the attention in the permuted layout (dq, dk
    with respect to the rotated q, k), given dO, O and the forward's LSE."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o")):
        _check_tensor(plan, t, n)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(plan, t, n)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != _lse_shape(plan):
        raise ValueError(f"lse: expected a contiguous float32 tensor of shape {_lse_shape(plan)}")
    if workspace is None:
        workspace = bwd_workspace(plan, q.device)
    vp = lambda t: c_void_p(t.data_ptr())
    _check("ug_attn_bwd", lib().ug_attn_bwd(plan.handle, vp(q), vp(k), vp(v), vp(o), vp(d_o), vp(lse), vp(dq), vp(dk),
                                            vp(dv), vp(workspace), _stream_ptr(q)))
    return dq, dk, dv


def ug_attn_bwd_noalloc(plan: Plan, q, k, v, o, d_o, lse, dq, dk, dv):
    """ug_attn_bwd with the statistics in the library's per-GPU scratch: the
    caller passes inputs and outputs only, nothing is allocated."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(plan, t, n)
    vp = lambda t: c_void_p(t.data_ptr())
    _check("ug_attn_bwd_noalloc", lib().ug_attn_bwd_noalloc(plan.handle, vp(q), vp(k), vp(v), vp(o), vp(d_o),
                                                            vp(lse), vp(dq), vp(dk), vp(dv), _stream_ptr(q)))
    return dq, dk, dv


def ug_rope2d_bwd(plan: Plan, dq_perm, dk_perm):
    """In place: the transpose of ug_rope2d's rotation (gradients with
    respect to the rotated Q, K become gradients with respect to Q, K)."""
    _check_tensor(plan, dq_perm, "dq_perm")
    _check_tensor(plan, dk_perm, "dk_perm")
    _check("ug_rope2d_bwd", lib().ug_rope2d_bwd(plan.handle, c_void_p(dq_perm.data_ptr()),
                                                c_void_p(dk_perm.data_ptr()), _stream_ptr(dq_perm)))
    return dq_perm, dk_perm


def ug_permute_rope_bwd(plan: Plan, dq_perm, dk_perm, dq_raster=None, dk_raster=None):
    """The transpose of ug_permute_rope: ug_rope2d_bwd followed by
    ug_unpermute of dq and dk, in one pass, out of place."""
    _check_tensor(plan, dq_perm, "dq_perm")
    _check_tensor(plan, dk_perm, "dk_perm")
    if dq_raster is None:
        dq_raster = _torch().empty_like(dq_perm)
    if dk_raster is None:
        dk_raster = _torch().empty_like(dk_perm)
    _check_tensor(plan, dq_raster, "dq_raster")
    _check_tensor(plan, dk_raster, "dk_raster")
    _check("ug_permute_rope_bwd", lib().ug_permute_rope_bwd(plan.handle, c_void_p(dq_perm.data_ptr()),
                                                            c_void_p(dk_perm.data_ptr()), c_void_p(dq_raster.data_ptr()),
                                                            c_void_p(dk_raster.data_ptr()), _stream_ptr(dq_perm)))
    return dq_raster, dk_raster


def ug_warm_start(x_lr, noise, rho: int, alpha: float, sharpen: float, x_hr=None):
    """HR start latent alpha * noise + (1 - alpha) * sharpen(upsample(x_lr));
    x_lr [B, h, w, C] and noise [B, H, W, C] CUDA tensors of one dtype
    (float32 or bfloat16), channels last.  x_hr may be `noise` (in place)."""
    torch = _torch()
    if x_lr.dtype != noise.dtype or x_lr.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x_lr and noise must share a dtype, float32 or bfloat16")
    if x_lr.dim() != 4 or noise.dim() != 4 or x_lr.shape[0] != noise.shape[0] or x_lr.shape[3] != noise.shape[3]:
        raise ValueError(f"expected x_lr [B, h, w, C] and noise [B, H, W, C], got {tuple(x_lr.shape)}, "
                         f"{tuple(noise.shape)}")
    if x_hr is None:
        x_hr = torch.empty_like(noise)
    for t, n in ((x_lr, "x_lr"), (noise, "noise"), (x_hr, "x_hr")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n}: expected a contiguous CUDA tensor")
    if x_hr.shape != noise.shape or x_hr.dtype != noise.dtype:
        raise ValueError("x_hr must match noise in shape and dtype")
    B, H, W, C = noise.shape
    d = UgWarmDesc(batch=B, hr_h=H, hr_w=W, lr_h=x_lr.shape[1], lr_w=x_lr.shape[2], channels=C, rho=rho,
                   dtype=UG_BF16 if noise.dtype == torch.bfloat16 else UG_F32, alpha=alpha, sharpen=sharpen)
    _check("ug_warm_start", lib().ug_warm_start(byref(d), c_void_p(x_lr.data_ptr()), c_void_p(noise.data_ptr()),
                                                c_void_p(x_hr.data_ptr()), _stream_ptr(noise)))
    return x_hr


class TrainLayer:
    """Forward that keeps what the backward needs, and the backward of the
    whole layer (raster in, raster out):
      forward:  permute+RoPE Q, K; permute V; attention with LSE; unpermute O
      backward: permute dO; attention backward; RoPE transpose and unpermute
                of dQ, dK in one pass; unpermute dV."""

    def __init__(self, plan: Plan, device="cuda"):
        torch = _torch()
        self.plan = plan
        mk = lambda: torch.empty(plan.shape, dtype=torch.bfloat16, device=device)
        self.qp, self.kp, self.vp, self.op, self.dop = mk(), mk(), mk(), mk(), mk()
        self.dq, self.dk, self.dv = mk(), mk(), mk()
        self.lse = torch.empty(_lse_shape(plan), dtype=torch.float32, device=device)
        self.ws = bwd_workspace(plan, device)

    def forward(self, q, k, v, out):
        p = self.plan
        ug_permute_rope(p, q, k, self.qp, self.kp)
        ug_permute(p, v, self.vp)
        ug_attn_fwd_lse(p, self.qp, self.kp, self.vp, self.op, self.lse)
        ug_unpermute(p, self.op, out)
        return out

    def backward(self, d_out, dq, dk, dv):
        p = self.plan
        ug_permute(p, d_out, self.dop)
        ug_attn_bwd(p, self.qp, self.kp, self.vp, self.op, self.dop, self.lse, self.dq, self.dk, self.dv, self.ws)
        ug_permute_rope_bwd(p, self.dq, self.dk, dq, dk)
        ug_unpermute(p, self.dv, dv)
        return dq, dk, dv


class Layer:
    """One attention layer's whole path with preallocated buffers.

    fused=False: permute Q, K, V -> RoPE on Q, K -> attention -> unpermute O
    (one call per step of the path).  fused=True: permute+RoPE of Q and K in
    one pass, permute V, attention writing O straight in raster order; the
    result is bit-identical.
    """

    def __init__(self, plan: Plan, device="cuda", fused=False):
        torch = _torch()
        self.plan = plan
        self.fused = fused
        dt = torch.bfloat16 if plan.desc.dtype == UG_BF16 else torch.float32
        mk = lambda: torch.empty(plan.shape, dtype=dt, device=device)
        self.qp, self.kp, self.vp = mk(), mk(), mk()
        self.op = None if fused else mk()

    def __call__(self, q, k, v, out):
        p = self.plan
        if self.fused:
            ug_permute_rope(p, q, k, self.qp, self.kp)
            ug_permute(p, v, self.vp)
            ug_attn_fwd_raster(p, self.qp, self.kp, self.vp, out)
            return out
        ug_permute(p, q, self.qp)
        ug_permute(p, k, self.kp)
        ug_permute(p, v, self.vp)
        ug_rope2d(p, self.qp, self.kp)
        ug_attn_fwd(p, self.qp, self.kp, self.vp, self.op)
        ug_unpermute(p, self.op, out)
        return out
