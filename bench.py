#!/usr/bin/env python3
"""Benchmark of one hierarchical-local-attention layer on one MI355X.

A step is the whole hot path over one batch of synthetic input already
resident in HBM: window-first permutation of Q, K and V, 2D axial RoPE on Q
and K, the composite-masked attention forward, and the inverse permutation of
O, run as three launches (permutation+RoPE of Q and K fused, permutation of
V, attention with the inverse permutation in its epilogue).  The same path as
one call per step is timed too and reported under "unfused".  The plan (host
tables, built once per resolution and reused by every layer and denoising
step) is built before the timed region.

Prints ONE JSON line.  `value` is effective TFLOP/s of the whole step:
4 * D * (allowed query-key pairs) * heads / step time, i.e. only unmasked
pairs count.  Per-kernel times come from HIP events recorded on the stream
the kernels are launched on (torch's current stream).

For bf16 workloads the line also carries "backward": the training layer's
backward step (permute dO, attention backward, RoPE transpose and unpermute
of dQ, dK in one pass, unpermute dV) after a forward that saved the LSE, with
the attention backward's effective TFLOP/s counted as 10 * D * pairs * heads
(the five products S, dP, dV, dK, dQ of the allowed pairs).  "warm_start" times the warm-start
kernel (once per image, not part of the step) on 256x256 x 64-channel bf16
latents, batch 1 and 16, against HBM bandwidth.

Each timed series that follows an idle period (the process start, the upload
of a layer's inputs) is preceded by about 0.15 s of bf16 matrix products, so
that it runs at the clock the GPU sustains under load (see preheat below;
--no-preheat turns this off).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 (vector / MFMA f32 dense)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
# the attention kernel and the plan that orders its work (the order sets the L2 re-fetches)
KERNEL_SRCS = [os.path.join(ROOT, "diffusion_transformer_sparse_amd", "csrc", n) for n in ("kernels.hip", "plan.cpp")]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counters, or
    None when they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload)
    if not e or e.get("kernel_sha") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_POOL_BARRIER = None


def _pool_init(barrier):
    global _POOL_BARRIER
    _POOL_BARRIER = barrier
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)  # one BLAS thread per process: the processes use the cores
    except Exception:
        pass


def _oracle_head(args):
    """One head of the oracle in a worker: inputs first, then every worker
    starts the oracle call together (barrier) and times it."""
    import workloads as WL
    from oracle import ultragen_oracle as O
    name, h = args
    w = WL.WORKLOADS[name]
    geo = O.geometry_of(w)
    q, k, v = (WL.head_f64(w, t, h) for t in (WL.Q, WL.K, WL.V))
    _POOL_BARRIER.wait()
    t0 = time.perf_counter()  # CLOCK_MONOTONIC: comparable across the processes
    O.forward_head(geo, q, k, v, w.rope_theta)
    return t0, time.perf_counter()


def cpu_baseline(w, max_procs: int):
    """The fp64 oracle (as it stands) on a bounded sample of the same layer:
    whole heads, one per process, on up to `max_procs` host cores at once (one
    BLAS thread each), all started together; the rate is the sample's
    effective FLOP over the wall time from the first start to the last end.
    Runs before the GPU is touched (the workers are forked)."""
    import multiprocessing as mp
    from oracle import ultragen_oracle as O
    nproc = os.cpu_count() or 1
    procs = max(1, min(nproc, max_procs, w.heads))
    ctx = mp.get_context("fork")
    barrier = ctx.Barrier(procs)
    with ctx.Pool(procs, initializer=_pool_init, initargs=(barrier,)) as pool:
        spans = pool.map(_oracle_head, [(w.name, h) for h in range(procs)], chunksize=1)
    wall = max(e for _, e in spans) - min(s0 for s0, _ in spans)
    per_head_flops = 4.0 * w.head_dim * O.pair_count(O.geometry_of(w))
    return {"value": per_head_flops * procs / wall / 1e12, "unit": "TFLOP/s", "cores": procs, "kind": "oracle",
            "sample": f"{procs} of {w.heads} heads of the {w.name} layer, one per process, 1 BLAS thread each, "
                      f"started together (fp64 numpy RoPE + grouped masked attention; input generation not timed)",
            "seconds": round(wall, 2), "nproc": nproc, "cpu_model": _cpu_model(), "processes": procs,
            "blas_threads_per_process": 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="4k")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="most host processes for cpu_baseline (the host's CPU share per GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward step measurement")
    ap.add_argument("--no-warm", action="store_true", help="skip the warm-start kernel measurement")
    ap.add_argument("--no-preheat", action="store_true",
                    help="time each series straight after its inputs are uploaded, without first bringing the GPU "
                         "to its sustained clock")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import workloads as WL

    w = WL.WORKLOADS[args.workload]
    # the CPU baseline first, in forked worker processes, before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_procs)

    import torch
    import diffusion_transformer_sparse_amd as U

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_plan = time.perf_counter()
    plan = U.ug_plan(U.desc_of(w))
    t_plan = time.perf_counter() - t_plan
    info = plan.info

    def to_dev(a, dtype=None):
        if (dtype or w.dtype) == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = (to_dev(WL.tensor_storage(w, t)) for t in (WL.Q, WL.K, WL.V))
    out = torch.empty_like(q)
    layer = U.Layer(plan, dev)  # buffers for the permuted Q, K, V and O
    stream = torch.cuda.current_stream(dev)

    # The timed step: window-first permutation + RoPE of Q and K in one pass,
    # permutation of V, attention writing O in raster order (the inverse
    # permutation folded into its epilogue).
    def step_fused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        U.ug_permute_rope(plan, q, k, layer.qp, layer.kp)
        if ev is not None:
            ev[1].record(stream)
        U.ug_permute(plan, v, layer.vp)
        if ev is not None:
            ev[2].record(stream)
        U.ug_attn_fwd_raster(plan, layer.qp, layer.kp, layer.vp, out)
        if ev is not None:
            ev[3].record(stream)

    # The same path as one call per step: permute x3, RoPE, attention, unpermute.
    def step_unfused(ev=None):
        if ev is not None:
            ev[0].record(stream)
        U.ug_permute(plan, q, layer.qp)
        U.ug_permute(plan, k, layer.kp)
        U.ug_permute(plan, v, layer.vp)
        if ev is not None:
            ev[1].record(stream)
        U.ug_rope2d(plan, layer.qp, layer.kp)
        if ev is not None:
            ev[2].record(stream)
        U.ug_attn_fwd(plan, layer.qp, layer.kp, layer.vp, layer.op)
        if ev is not None:
            ev[3].record(stream)
        U.ug_unpermute(plan, layer.op, out)
        if ev is not None:
            ev[4].record(stream)

    # The GPU leaves its idle power state only over the first tens of
    # milliseconds of load: after an idle period (process start, input
    # uploads) the first launches of a series run up to 20% slower while the
    # clock ramps up.  Inside a denoising loop the layers run back to back, so
    # the sustained clock is the representative one.  Before each timed
    # series that follows such a period, bf16 matrix products (torch.mm: not
    # part of any step, and not this library's kernels) keep the GPU busy for
    # about 0.15 s; the series' own warmup steps then run as usual.
    heat = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    heat_out = torch.empty_like(heat)

    def preheat(seconds=0.15):
        if args.no_preheat:
            return
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                torch.mm(heat, heat, out=heat_out)
            torch.cuda.synchronize()

    def timed(step, n_events, steps, warmup):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(events[i])
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) / steps * 1e3
        avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in events) / len(events)
        return wall_ms, avg

    layer.op = torch.empty_like(q)
    preheat()
    ms_step, avg = timed(step_fused, 4, args.steps, args.warmup)
    ms_prq, ms_pv, ms_attn = avg(0, 1), avg(1, 2), avg(2, 3)
    ums_step, uavg = timed(step_unfused, 5, max(5, args.steps // 2), 2)
    ums_perm3, ums_rope, ums_attn, ums_unperm = uavg(0, 1), uavg(1, 2), uavg(2, 3), uavg(3, 4)

    def measure_training(tw, steps):
        """Training layer of workload tw: the forward that keeps the LSE
        (permute+RoPE, permute V, attention with LSE, unpermute O) and the
        backward step (permute dO, attention backward, RoPE transpose and
        unpermute of dQ and dK, unpermute dV), each timed with HIP events."""
        tplan = plan if tw is w else U.ug_plan(U.desc_of(tw))
        tinfo = tplan.info
        tq, tk, tv = (to_dev(WL.tensor_storage(tw, t)) for t in (WL.Q, WL.K, WL.V))
        d_o = to_dev(WL.tensor_storage(tw, WL.DO))
        tout = torch.empty_like(tq)
        train = U.TrainLayer(tplan, dev)
        grads = [torch.empty_like(tq) for _ in range(3)]

        def step_fwd(ev=None):
            if ev is not None:
                ev[0].record(stream)
            U.ug_permute_rope(tplan, tq, tk, train.qp, train.kp)
            U.ug_permute(tplan, tv, train.vp)
            if ev is not None:
                ev[1].record(stream)
            U.ug_attn_fwd_lse(tplan, train.qp, train.kp, train.vp, train.op, train.lse)
            if ev is not None:
                ev[2].record(stream)
            U.ug_unpermute(tplan, train.op, tout)
            if ev is not None:
                ev[3].record(stream)

        def step_bwd(ev=None):
            if ev is not None:
                ev[0].record(stream)
            U.ug_permute(tplan, d_o, train.dop)
            if ev is not None:
                ev[1].record(stream)
            U.ug_attn_bwd(tplan, train.qp, train.kp, train.vp, train.op, train.dop, train.lse, train.dq, train.dk,
                          train.dv, train.ws)
            if ev is not None:
                ev[2].record(stream)
            U.ug_permute_rope_bwd(tplan, train.dq, train.dk, grads[0], grads[1])
            U.ug_unpermute(tplan, train.dv, grads[2])
            if ev is not None:
                ev[3].record(stream)

        preheat()  # after the uploads of this layer's inputs
        fms_step, favg = timed(step_fwd, 4, steps, 2)
        bms_step, bavg = timed(step_bwd, 4, steps, 2)
        fflops = tinfo["eff_flops"]
        bflops = 2.5 * tinfo["eff_flops"]
        fms_attn, bms_attn = favg(1, 2), bavg(1, 2)
        res = {
            "workload": tw.name,
            "batch": tw.batch,
            "forward": {"ms_per_step": round(fms_step, 4), "attn_fwd_lse_ms": round(fms_attn, 4),
                        "eff_tflops": round(fflops / (fms_attn * 1e-3) / 1e12, 2),
                        "frac_peak": round(fflops / (fms_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "ms_per_step": round(bms_step, 4),
            "step": "ug_permute(dO) + ug_attn_bwd + ug_permute_rope_bwd(dQ,dK) + ug_unpermute(dV)",
            "attn_bwd": {"ms": round(bms_attn, 4), "eff_tflops": round(bflops / (bms_attn * 1e-3) / 1e12, 2),
                         "frac_peak": round(bflops / (bms_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "eff_flop": bflops},
            "layout_ms": round(bavg(0, 1) + bavg(2, 3), 4),
        }
        del train, grads, d_o, tq, tk, tv, tout
        return res

    backward = None
    backward_train = None
    if w.dtype == "bf16" and not args.no_backward:
        backward = measure_training(w, max(5, args.steps // 5))
        # the pages' fine-tuning shape: 1024x1024 images (64x64 latent tokens)
        # with 256x256 guides, one image per GPU
        backward_train = measure_training(WL.WORKLOADS["1k"], max(20, args.steps))

    warm = None
    if not args.no_warm:
        warm = {}
        for wname in ("warm_4k", "warm_4k_b16"):
            ww = WL.WARM_WORKLOADS[wname]
            x_lr = to_dev(WL.warm_storage(ww, WL.WARM_LR), ww.dtype)
            noise = to_dev(WL.warm_storage(ww, WL.WARM_NOISE), ww.dtype)
            x_hr = torch.empty_like(noise)

            # ten launches between two events (each a whole warm start of the
            # batch), so that the event and launch gaps of one launch do not
            # dominate a kernel of tens of microseconds; one launch per event
            # pair is reported beside it
            def step_warm(ev=None, reps=10):
                if ev is not None:
                    ev[0].record(stream)
                for _ in range(reps):
                    U.ug_warm_start(x_lr, noise, ww.rho, ww.alpha, ww.sharpen, x_hr)
                if ev is not None:
                    ev[1].record(stream)

            preheat()
            _, wavg = timed(step_warm, 2, 20, 3)
            wms = wavg(0, 1) / 10
            _, wavg1 = timed(lambda ev=None: step_warm(ev, 1), 2, 20, 3)
            wms1 = wavg1(0, 1)
            nbytes = 2 * noise.numel() * noise.element_size() + x_lr.numel() * x_lr.element_size()
            warm[wname] = {"ms": round(wms, 4), "bytes": nbytes, "gbs": round(nbytes / (wms * 1e-3) / 1e9, 1),
                           "frac_hbm": round(nbytes / (wms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "ms_one_launch": round(wms1, 4),
                           "frac_hbm_one_launch": round(nbytes / (wms1 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            del x_lr, noise, x_hr

    esize = 2 if w.dtype == "bf16" else 4
    tbytes = w.batch * w.seq_len * w.heads * w.head_dim * esize
    rope_bytes = 2 * 2 * w.batch * (w.n_hr + w.n_lr) * w.heads * w.head_dim * esize
    flops = info["eff_flops"]
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    attn_tflops = flops / (ms_attn * 1e-3) / 1e12
    traffic = measured_traffic(w.name)

    def gbs(nbytes, ms):
        return nbytes / (ms * 1e-3) / 1e9

    def hbm(nbytes, ms):
        return {"ms": round(ms, 4), "gbs": round(gbs(nbytes, ms), 1), "frac_hbm": round(gbs(nbytes, ms) / PEAK_HBM_GBS, 4)}

    res = {
        "metric": "effective attn TFLOP/s + ms/layer at 4K (65,536 HR tok), % of bf16 MFMA peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "hr_grid": [w.hr_h, w.hr_w], "lr_grid": [w.lr_h, w.lr_w],
                   "n_text": w.n_text, "heads": w.heads, "head_dim": w.head_dim, "window": w.window,
                   "radius": w.radius, "rho": w.rho, "lr_mode": w.lr_mode, "batch": w.batch, "seq_len": w.seq_len,
                   "pairs_per_head": info["pairs_per_head"], "eff_flop_per_step": flops,
                   "step": "ug_permute_rope(Q,K) + ug_permute(V) + ug_attn_fwd_raster"},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel", "achieved": round(attn_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(attn_tflops / peak, 4),
                     "traffic": traffic},
        "kernels": {
            "attn_fwd_raster": {"ms": round(ms_attn, 4), "eff_tflops": round(attn_tflops, 2),
                                "frac_peak": round(attn_tflops / peak, 4)},
            "permute_rope_qk": hbm(2 * 2 * tbytes, ms_prq),
            "permute_v": hbm(2 * tbytes, ms_pv),
        },
        "unfused": {
            "ms_per_step": round(ums_step, 4),
            "value": round(flops / (ums_step * 1e-3) / 1e12, 2),
            "attn_fwd": {"ms": round(ums_attn, 4), "eff_tflops": round(flops / (ums_attn * 1e-3) / 1e12, 2)},
            "permute_qkv": hbm(3 * 2 * tbytes, ums_perm3),
            "rope2d_qk": hbm(rope_bytes, ums_rope),
            "unpermute_o": hbm(2 * tbytes, ums_unperm),
        },
        "backward": backward,
        "backward_train_1k": backward_train,
        "warm_start": warm,
        "plan_build_s": round(t_plan, 4),
        "clock_preheat_s": None if args.no_preheat else 0.15,
        "kernel_sha": kernel_hash(),
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
