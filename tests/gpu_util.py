"""Helpers shared by the GPU parity tests: moving seeded workload tensors to
the device and back, and per-segment error statistics."""
import numpy as np

import workloads as WL

BF16_TOL = (2e-2, 5e-3)   # max-abs, rel-L2 per segment and head
F32_TOL = (1e-4, 1e-4)


def tol_of(w):
    return BF16_TOL if w.dtype == "bf16" else F32_TOL


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_host_f64(t, dtype):
    import torch
    if dtype == "bf16":
        return WL.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy().astype(np.float64)


def to_host_storage(t, dtype):
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def qkv_device(w):
    return [to_device(WL.tensor_storage(w, t), w.dtype) for t in (WL.Q, WL.K, WL.V)]


def segments(w):
    T, N = w.n_text, w.n_hr
    return (("text", slice(0, T)), ("hr", slice(T, T + N)), ("lr", slice(T + N, w.seq_len)))


def seg_errors(got, ref, w, rows=None):
    """{segment: (max_abs, rel_l2)}; `rows` gives the raster row of each line
    when got/ref hold a sample of rows."""
    out = {}
    idx = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    T, N = w.n_text, w.n_hr
    kinds = np.where(idx < T, 0, np.where(idx < T + N, 1, 2))
    for k, name in enumerate(("text", "hr", "lr")):
        sel = kinds == k
        if not sel.any():
            continue
        g, r = got[sel], ref[sel]
        out[name] = (float(np.max(np.abs(g - r))), float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)))
    return out


def assert_close(errs, tol, what):
    bad = {k: v for k, v in errs.items() if v[0] > tol[0] or v[1] > tol[1]}
    assert not bad, f"{what}: {bad} exceeds (max-abs, rel-L2) {tol}; all: {errs}"
