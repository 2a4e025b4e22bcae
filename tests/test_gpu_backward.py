"""GPU parity of the training path (forward LSE, attention backward, RoPE
transpose) against the fp64 oracle on the same seeded inputs.

Bars for bf16 (8 significant bits: unit roundoff u = 2^-8; a round-to-nearest
step has an RMS relative error of about 0.4u = 1.6e-3), derived from the
rounding steps of the kernels (operands rounded to bf16, fp32 accumulation):
  - the rotated Q, K are bf16, so every logit carries an RMS error of about
    sqrt(2) * 1.6e-3, and P a relative error of about 2.2e-3;
  - P and dS are rounded to bf16 as MFMA operands, O (used for Delta) carries
    the forward's error (~3e-3 rel-L2), and the outputs are rounded to bf16;
  first-order propagation gives rel-L2 of about 3e-3 (dV) to 5e-3 (dK, which
  also passes the RoPE transpose), hence rel-L2 <= 1e-2 per segment and
  max-abs <= 2e-2 * max|ref| (about 5u) per segment; LSE |error| <= 4u *
  q_scale (bf16) or 1e-5 (fp32); a RoPE round trip (two roundings of a
  rotated pair) is within (sqrt(2) + 1)u <= 3u of the pair's norm.
"""
import numpy as np
import pytest

import workloads as WL
from oracle import ultragen_oracle as O
from tests.gpu_util import seg_errors, to_device, to_host_f64

pytestmark = pytest.mark.gpu

BWD_REL = 1e-2
BWD_MAXREL = 2e-2
U_BF16 = 2.0 ** -8  # unit roundoff of bfloat16

SMALL_BWD = ["small_ragged", "small_d64", "small_ragged_corr"]


@pytest.fixture(scope="module")
def U():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import diffusion_transformer_sparse_amd as U
    return U


def permuted_order(w):
    T, N = w.n_text, w.n_hr
    perm = O.window_first_perm(w.hr_h, w.hr_w, w.window)
    lr = O.lr_window_first_perm(O.geometry_of(w)) if w.lr_mode == 1 else np.arange(w.n_lr)
    return np.concatenate([np.arange(T), T + perm, T + N + lr]).astype(np.int64)


def grad_close(got, ref, w, what, rows=None):
    errs = seg_errors(got, ref, w, rows)
    idx = np.arange(got.shape[0]) if rows is None else np.asarray(rows)
    T, N = w.n_text, w.n_hr
    kinds = np.where(idx < T, 0, np.where(idx < T + N, 1, 2))
    bad = {}
    for k, name in enumerate(("text", "hr", "lr")):
        if name not in errs:
            continue
        scale = float(np.abs(ref[kinds == k]).max())
        mx, rel = errs[name]
        if mx > BWD_MAXREL * scale or rel > BWD_REL:
            bad[name] = (mx, scale, rel)
    assert not bad, f"{what}: (max-abs, max|ref|, rel-L2) {bad} exceed ({BWD_MAXREL}*max|ref|, {BWD_REL})"


def inputs(w):
    return [to_device(WL.tensor_storage(w, t), w.dtype) for t in (WL.Q, WL.K, WL.V, WL.DO)]


def oracle_heads(w, heads, b=0):
    geo = O.geometry_of(w)
    for h in heads:
        yield h, geo, [WL.head_f64(w, t, h, b) for t in (WL.Q, WL.K, WL.V, WL.DO)]


# ---------------------------------------------------------------- forward LSE

@pytest.mark.parametrize("name,qscale", [("tiny_masked", 1.0), ("small_ragged", 1.0), ("small_d64", 1.0),
                                         ("small_ragged_corr", 1.0), ("small_ragged", 8.0),
                                         ("small_ragged_f32", 1.0)])
def test_forward_lse_matches_oracle(U, name, qscale):
    import torch
    w = WL.WORKLOADS[name].with_(q_scale=qscale)
    p = U.ug_plan(U.desc_of(w))
    q, k, v, _ = inputs(w)
    qp, kp = U.ug_permute_rope(p, q, k)
    vp = U.ug_permute(p, v)
    o, lse = U.ug_attn_fwd_lse(p, qp, kp, vp)
    o_ref = U.ug_attn_fwd(p, qp, kp, vp)
    torch.cuda.synchronize()
    bits = torch.int16 if w.dtype == "bf16" else torch.int32
    assert torch.equal(o.view(bits), o_ref.view(bits)), "the LSE variant changed O"
    order = permuted_order(w)
    got = lse.cpu().numpy().astype(np.float64)[0]
    tol = 4 * U_BF16 * qscale if w.dtype == "bf16" else 1e-5
    for h, geo, (qh, kh, _, _) in oracle_heads(w, range(w.heads)):
        _, pr, pc, _, _ = O.token_coords(geo)
        ref = O.lse_grouped(geo, O.rope_rotate(qh, pr, pc, w.rope_theta), O.rope_rotate(kh, pr, pc, w.rope_theta))
        err = np.abs(got[h] - ref[order])
        assert err.max() <= tol, (h, float(err.max()), tol)


# ---------------------------------------------------------------- RoPE transpose

@pytest.mark.parametrize("name", ["small_ragged", "small_ragged_f32", "small_ragged_corr"])
def test_rope2d_bwd_inverts_rope2d(U, name):
    import torch
    w = WL.WORKLOADS[name]
    p = U.ug_plan(U.desc_of(w))
    q, k, _, _ = inputs(w)
    qp, kp = U.ug_permute(p, q), U.ug_permute(p, k)
    q0, k0 = qp.clone(), kp.clone()
    U.ug_rope2d(p, qp, kp)
    U.ug_rope2d_bwd(p, qp, kp)
    torch.cuda.synchronize()
    for a, b in ((qp, q0), (kp, k0)):
        a, b = to_host_f64(a, w.dtype), to_host_f64(b, w.dtype)
        # a rotation mixes the two elements of a pair, so each rounding error
        # is bounded by u times the pair's norm, not the element's magnitude
        pair = np.sqrt(b[..., 0::2] ** 2 + b[..., 1::2] ** 2).repeat(2, axis=-1)
        bound = 3 * U_BF16 * pair + 1e-6 if w.dtype == "bf16" else 4e-7 * pair + 1e-6
        assert np.all(np.abs(a - b) <= bound), float((np.abs(a - b) / (pair + 1e-30)).max())


def test_rope2d_bwd_matches_oracle_transpose(U):
    import torch
    w = WL.WORKLOADS["small_ragged_f32"]
    p = U.ug_plan(U.desc_of(w))
    q, k, _, _ = inputs(w)
    qp, kp = U.ug_permute(p, q), U.ug_permute(p, k)
    U.ug_rope2d_bwd(p, qp, kp)
    torch.cuda.synchronize()
    order = permuted_order(w)
    geo = O.geometry_of(w)
    _, pr, pc, _, _ = O.token_coords(geo)
    got = to_host_f64(qp, w.dtype)[0]
    for h in range(w.heads):
        ref = O.rope_rotate_transpose(WL.head_f64(w, WL.Q, h), pr, pc, w.rope_theta)[order]
        assert np.abs(got[:, h] - ref).max() <= 2e-6


# ---------------------------------------------------------------- attention backward

def run_attn_bwd(U, w):
    """permuted layout, no RoPE: forward with LSE, backward; raster results."""
    import torch
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    qp, kp, vp, dop = (U.ug_permute(p, x) for x in (q, k, v, do))
    o, lse = U.ug_attn_fwd_lse(p, qp, kp, vp)
    dq, dk, dv = U.ug_attn_bwd(p, qp, kp, vp, o, dop, lse)
    out = [to_host_f64(U.ug_unpermute(p, x), w.dtype)[0] for x in (dq, dk, dv)]
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,qscale", [(n, 1.0) for n in SMALL_BWD] + [("small_ragged", 8.0)])
def test_attention_backward_matches_oracle(U, name, qscale):
    w = WL.WORKLOADS[name].with_(q_scale=qscale)
    dq, dk, dv = run_attn_bwd(U, w)
    for h, geo, (qh, kh, vh, doh) in oracle_heads(w, range(w.heads)):
        rq, rk, rv = O.attention_backward_grouped(geo, qh, kh, vh, doh)
        grad_close(dq[:, h], rq, w, f"{name} x{qscale} dq h{h}")
        grad_close(dk[:, h], rk, w, f"{name} x{qscale} dk h{h}")
        grad_close(dv[:, h], rv, w, f"{name} x{qscale} dv h{h}")


def run_layer_bwd(U, w, host=True):
    """TrainLayer forward + backward; the results on the host in fp64, or
    (host=False) as device tensors."""
    import torch
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    layer = U.TrainLayer(p)
    out = torch.full_like(q, float("nan"))  # NaN until written: a skipped work item shows up
    layer.forward(q, k, v, out)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    layer.backward(do, dq, dk, dv)
    torch.cuda.synchronize()
    if not host:
        return p, [out, dq, dk, dv]
    return p, [to_host_f64(x, w.dtype) for x in (out, dq, dk, dv)]


def test_layer_backward_two_images_many_heads(U):
    """TrainLayer backward at batch 2 x 8 heads (the work queues group each
    head's long tiles on one XCD): first and last head of both images
    against the oracle."""
    w = WL.WORKLOADS["ragged_b2"]
    _, (_, dq, dk, dv) = run_layer_bwd(U, w)
    for b in range(w.batch):
        for h, geo, (qh, kh, vh, doh) in oracle_heads(w, (0, w.heads - 1), b):
            rq, rk, rv = O.backward_head(geo, qh, kh, vh, doh, w.rope_theta)
            grad_close(dq[b][:, h], rq, w, f"ragged_b2 image {b} dq h{h}")
            grad_close(dk[b][:, h], rk, w, f"ragged_b2 image {b} dk h{h}")
            grad_close(dv[b][:, h], rv, w, f"ragged_b2 image {b} dv h{h}")


@pytest.mark.parametrize("name", SMALL_BWD + ["1k"])
def test_layer_backward_matches_oracle(U, name):
    """TrainLayer (raster in, raster out: RoPE, permutation, attention and
    their backward) against the oracle's full-layer backward."""
    w = WL.WORKLOADS[name]
    _, (out, dq, dk, dv) = run_layer_bwd(U, w)
    heads = range(w.heads) if w.heads <= 4 else (0, 11, w.heads - 1)
    for h, geo, (qh, kh, vh, doh) in oracle_heads(w, heads):
        rq, rk, rv = O.backward_head(geo, qh, kh, vh, doh, w.rope_theta)
        grad_close(dq[0][:, h], rq, w, f"{name} dq h{h}")
        grad_close(dk[0][:, h], rk, w, f"{name} dk h{h}")
        grad_close(dv[0][:, h], rv, w, f"{name} dv h{h}")


EDGE_BWD = {
    "no_text": dict(n_text=0),
    "no_lr": dict(lr_h=0, lr_w=0),
    "one_text": dict(n_text=1),
    "radius0": dict(radius=0),
    "radius2": dict(radius=2),
    "window8": dict(window=8),
    "window_covers_grid": dict(window=64),
    "batch2": dict(batch=2),
    "corr_overhang": dict(lr_mode=1, lr_h=14, lr_w=14),
    "corr_radius2": dict(lr_mode=1, radius=2),
    "corr_window8": dict(lr_mode=1, window=8),
    # 9x9 windows at radius 4: interior windows see 81 windows, more query
    # ranges than one key tile may hold, so plain and grouped (masked) LR
    # key tiles share one dK/dV launch
    "corr_radius4_plain_and_grouped": dict(lr_mode=1, window=8, radius=4, hr_h=72, hr_w=72, lr_h=18, lr_w=18),
}


@pytest.mark.parametrize("case", list(EDGE_BWD))
def test_layer_backward_edge_cases(U, case):
    w = WL.WORKLOADS["small_ragged"].with_(cfg_id=21, heads=2, **EDGE_BWD[case])
    _, (_, dq, dk, dv) = run_layer_bwd(U, w)
    for b in range(w.batch):
        for h, geo, (qh, kh, vh, doh) in oracle_heads(w, range(w.heads), b):
            rq, rk, rv = O.backward_head(geo, qh, kh, vh, doh, w.rope_theta)
            for got, ref, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
                grad_close(got[b][:, h], ref, w, f"{case} {n} b{b} h{h}")


def _random_bf16():
    from tests.test_gpu_parity import RANDOM
    return {k: w for k, w in RANDOM.items() if w.dtype == "bf16"}


@pytest.mark.parametrize("name", list(_random_bf16()))
def test_layer_backward_random_geometries(U, name):
    """The training layer's backward on the seeded random small bf16
    geometries of the forward parity tests: dq, dk, dv of every row of every
    head and image against the oracle."""
    w = _random_bf16()[name]
    _, (_, dq, dk, dv) = run_layer_bwd(U, w)
    for b in range(w.batch):
        for h, geo, (qh, kh, vh, doh) in oracle_heads(w, range(w.heads), b):
            rq, rk, rv = O.backward_head(geo, qh, kh, vh, doh, w.rope_theta)
            grad_close(dq[b][:, h], rq, w, f"{name} dq b{b} h{h}")
            grad_close(dk[b][:, h], rk, w, f"{name} dk b{b} h{h}")
            grad_close(dv[b][:, h], rv, w, f"{name} dv b{b} h{h}")


def test_backward_is_deterministic(U):
    import torch
    w = WL.WORKLOADS["1k"]
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    o, lse = U.ug_attn_fwd_lse(p, q, k, v)
    a = U.ug_attn_bwd(p, q, k, v, o, do, lse)
    b = U.ug_attn_bwd(p, q, k, v, o, do, lse)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_on_two_streams_at_once(U):
    """ug_attn_bwd runs its dK/dV pass on a stream of the plan's, forked from
    and joined back to the caller's stream: two calls on one plan from two
    streams at once give the one-stream gradients bit for bit, and copies
    queued on each caller's stream right after its call see all three."""
    import torch
    w = WL.WORKLOADS["1k"]
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    o, lse = U.ug_attn_fwd_lse(p, q, k, v)
    ref = U.ug_attn_bwd(p, q, k, v, o, do, lse)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    grads, copies = [], []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            g = U.ug_attn_bwd(p, q, k, v, o, do, lse)
            copies.append([t.clone() for t in g])  # queued on s after the call
            grads.append(g)
    torch.cuda.synchronize()
    for i in range(2):
        for name, got, cp, r in zip(("dq", "dk", "dv"), grads[i], copies[i], ref):
            assert torch.equal(got.view(torch.int16), r.view(torch.int16)), f"stream {i} {name}"
            assert torch.equal(cp.view(torch.int16), r.view(torch.int16)), f"stream {i} {name} (copy)"


def test_backward_refuses_stream_capture(U):
    """The backward's dQ pass takes a work-queue cursor slot at launch time,
    so the call refuses stream capture with UG_ERR_UNSUPPORTED before it
    queues anything, and the plan works as before afterwards."""
    import torch
    w = WL.WORKLOADS["small_ragged"]
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    o, lse = U.ug_attn_fwd_lse(p, q, k, v)
    ref = U.ug_attn_bwd(p, q, k, v, o, do, lse)
    outs = [torch.empty_like(q) for _ in range(3)]
    ws = U.bwd_workspace(p, q.device)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(U.UgError) as err:
        with torch.cuda.graph(g):
            U.ug_attn_bwd(p, q, k, v, o, do, lse, *outs, workspace=ws)
    assert err.value.status == 2  # UG_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    again = U.ug_attn_bwd(p, q, k, v, o, do, lse, *outs, workspace=ws)
    torch.cuda.synchronize()
    for x, r in zip(again, ref):
        assert torch.equal(x.view(torch.int16), r.view(torch.int16))


def test_full_size_backward_whole_head(U):
    """The 4K layer's backward: dq, dk and dv of every row of one head
    (text, HR and LR queries and keys) against the oracle's whole-head
    backward."""
    w = WL.WORKLOADS["4k"]
    p, (_, dq_d, dk_d, dv_d) = run_layer_bwd(U, w, host=False)
    h = 9
    got = [to_host_f64(t[0, :, h].contiguous(), w.dtype) for t in (dq_d, dk_d, dv_d)]
    for _, geo, (qh, kh, vh, doh) in oracle_heads(w, (h,)):
        refs = O.backward_head(geo, qh, kh, vh, doh, w.rope_theta)
        for g, r, what in zip(got, refs, ("dq", "dk", "dv")):
            grad_close(g, r, w, f"4k {what} head {h} (all rows)")


@pytest.mark.parametrize("name", ["4k", "4k_corr", "ragged", "8k", "4k_d64"])
def test_full_size_backward_sampled(U, name):
    """A layer's backward at full size (256x256, the ragged 250x380 grid,
    512x512); the oracle recomputes dq of sampled query rows
    (corner, edge, interior HR, text, LR) and dk, dv of sampled HR key rows
    (with lr_mode 1 also LR key rows) one by one."""
    import torch
    w = WL.WORKLOADS[name]
    _, (out_d, dq_d, dk_d, dv_d) = run_layer_bwd(U, w, host=False)
    for t, n in ((out_d, "out"), (dq_d, "dq"), (dk_d, "dk"), (dv_d, "dv")):  # every element written
        assert bool(torch.isfinite(t).all()), f"{name}: {n} has unwritten (NaN) elements"
    geo = O.geometry_of(w)
    T, W, H = w.n_text, w.hr_w, w.hr_h
    qrows = np.array([0, T - 1, T, T + 15 * W + 16, T + 100 * W + 37, T + w.n_hr - 1, T + w.n_hr,
                      w.seq_len - 1])
    krows = [T + 16 * W + 16, T + (H - 1) * W + 3]
    if w.lr_mode == 1:  # an LR key is then seen by nine windows' queries, not all of them
        krows += [T + w.n_hr, T + w.n_hr + 37 * w.lr_w + 5, w.seq_len - 1]
    krows = np.array(krows)
    rows_of = lambda t, r: to_host_f64(t[0, r.tolist()].contiguous(), w.dtype)  # batch 0, sampled rows only
    dq, dk, dv = rows_of(dq_d, qrows), rows_of(dk_d, krows), rows_of(dv_d, krows)
    for h in (0, w.heads - 1):
        qh, kh, vh, doh = (WL.head_f64(w, t, h) for t in (WL.Q, WL.K, WL.V, WL.DO))
        rq = O.backward_query_rows(geo, qh, kh, vh, doh, w.rope_theta, qrows)
        grad_close(dq[:, h], rq, w, f"{name} dq h{h}", qrows)
        rk, rv = O.backward_key_rows(geo, qh, kh, vh, doh, w.rope_theta, krows)
        grad_close(dk[:, h], rk, w, f"{name} dk h{h}", krows)
        grad_close(dv[:, h], rv, w, f"{name} dv h{h}", krows)


def test_backward_argument_errors(U):
    import ctypes
    import torch
    w = WL.WORKLOADS["small_ragged"]
    p = U.ug_plan(U.desc_of(w))
    q, k, v, do = inputs(w)
    o, lse = U.ug_attn_fwd_lse(p, q, k, v)
    lib = U.lib()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = U.bwd_workspace(p)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    assert lib.ug_attn_bwd(p.handle, vp(q), vp(k), vp(v), vp(o), vp(do), vp(lse), vp(dq), vp(dk), vp(dv), None,
                           s) == 1
    assert lib.ug_attn_bwd(p.handle, vp(q), vp(k), vp(v), vp(o), vp(do), vp(lse), vp(dq), vp(dq), vp(dv), vp(ws),
                           s) == 1
    assert lib.ug_attn_bwd(p.handle, vp(q), vp(k), vp(v), vp(o), vp(do), vp(lse), vp(q), vp(dk), vp(dv), vp(ws),
                           s) == 1
    assert lib.ug_attn_fwd_lse(p.handle, vp(q), vp(k), vp(v), vp(o), None, None, s) == 1
    wf = WL.WORKLOADS["small_ragged_f32"]
    pf = U.ug_plan(U.desc_of(wf))
    assert lib.ug_attn_bwd(pf.handle, vp(q), vp(k), vp(v), vp(o), vp(do), vp(lse), vp(dq), vp(dk), vp(dv), vp(ws),
                           s) == 2
    torch.cuda.synchronize()
