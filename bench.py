#!/usr/bin/env python3
"""Benchmark of the chunkwise-retention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one chunkwise retention forward (out + final state) over the
long-sequence workload: batch 1, 32 heads, T = 65,536, d_k = d_v = 128,
bf16 in / fp32 accumulate, chunk 128, gamma_h = 1 - 2^(-5 - 4h/31).  Inputs
are seeded synthetic tensors already resident in HBM when timing starts.  The
JSON line also carries the other measured parts of the path: the recurrent
decode step (256 sequences x 32 heads, 128 x 128 fp32 state, 1000 consecutive
steps), the elu+1 linear-attention forward (batch 8, 16 heads, T = 8192,
d = 64), the elu+1 decode step on the decode shapes, the backward pass of the
long forward, the long forward with the row-sum floor and GroupNorm fused, the backward again
given the forward's segment states (as a training step keeps them),
the fp32 [4, 8, 2048, 64] forward and gated linear attention on that shape,
each with its own roofline figures.

Only one GPU is used; --gpus above 1 exits with a message.
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

METRIC = ("chunkwise retention fwd tokens/s + TFLOP/s (% MFMA peak); decode GB/s (% HBM)")
PROFILES = os.path.join(ROOT, "profiles")
# sources of the kernels whose HBM counters are committed under profiles/
FWD_SOURCES = ["retention_chunkwise_amd/csrc/seg_kernel.h", "retention_chunkwise_amd/csrc/seg_bwd.h",
               "retention_chunkwise_amd/csrc/kcommon.h", "retention_chunkwise_amd/csrc/internal.h"]
DECODE_SOURCES = ["retention_chunkwise_amd/csrc/decode.hip", "retention_chunkwise_amd/csrc/internal.h"]
F32_SOURCES = ["retention_chunkwise_amd/csrc/walk_kernel.h", "retention_chunkwise_amd/csrc/kcommon.h",
               "retention_chunkwise_amd/csrc/internal.h"]
GLA_SOURCES = ["retention_chunkwise_amd/csrc/gla.hip", "retention_chunkwise_amd/csrc/kcommon.h",
               "retention_chunkwise_amd/csrc/internal.h"]


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, paths) -> dict | None:
    """HBM bytes per launch from committed rocprofv3 counter runs.

    Returns None when no summary exists or when the kernel source changed
    after the counters were taken.
    """
    p = os.path.join(PROFILES, f"hbm_traffic_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_sha") != sources_sha(paths):
        return None
    return d


def measured_mfma(name: str, paths) -> dict | None:
    """Matrix-core counters of a workload from a committed rocprofv3 summary
    (None when absent or taken with other kernel sources)."""
    p = os.path.join(PROFILES, f"mfma_{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    return d if d.get("source_sha") == sources_sha(paths) else None


def time_launches(fn, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """Run fn warmup + steps times; return (avg ms per launch from HIP events,
    wall ms per step).  Events are recorded on torch's current stream, which
    is the stream the library launches on.  min_warm_ms > 0 (the component
    legs) keeps warming up until that much wall time has passed, so that the
    GPU's clocks have settled on this leg's load before the timed steps (the
    long forward's first 55 calls after a cold start ran 3 % slower than the
    next ones)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return ev0.elapsed_time(ev1) / steps, wall / steps


def progress(msg: str) -> None:
    """One line per finished leg on stderr (the JSON result stays alone on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline_fwd(inp, w, target_s: float = 10.0):
    """The fp64 oracle (recurrent form) on the host cores, on a prefix of every
    head's sequence; the rate is scaled to tokens/s of the whole workload."""
    import oracle

    nproc = os.cpu_count() or 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = nproc
    # one GPU's share of a shared host is 16 cores; more threads would take
    # cores from the other GPUs' processes
    cap = 16
    nthreads = min(avail, cap)
    cores = oracle.threads_used(nthreads)
    q, k, v, g = inp["q"], inp["k"], inp["v"], inp["gamma"]
    Ts = 256
    while True:
        t0 = time.perf_counter()
        oracle.retention_recurrent(q[:, :, :Ts], k[:, :, :Ts], v[:, :, :Ts], g, nthreads=nthreads)
        dt = time.perf_counter() - t0
        if dt >= target_s or Ts >= w.T:
            break
        Ts = min(w.T, max(Ts * 2, int(Ts * target_s / max(dt, 1e-3) * 0.9)))
    rate = w.B * Ts / dt  # tokens/s (all heads processed for each token)
    # the same oracle on one thread, on a prefix sized to about 3 s
    T1 = max(256, min(w.T, int(Ts * (3.0 / max(dt * cores, 1e-3)))))
    t0 = time.perf_counter()
    oracle.retention_recurrent(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], g, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": rate, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 recurrent oracle, g++ -O2 + OpenMP over (b, h); first {Ts} of "
                      f"{w.T} tokens of all {w.B * w.H} heads ({dt:.1f} s)",
            "seconds": dt,
            "nproc": nproc, "cpus_available": avail, "thread_cap": cap, "cpu_model": cpu_model(),
            "single_thread": {"value": w.B * T1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"first {T1} tokens of all {w.B * w.H} heads ({dt1:.1f} s)"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true",
                    help="time only the headline forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain device copies of known size (for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this library runs on a single GPU; runs on several GPUs are not "
              "supported (batch and heads shard with no communication, a split sequence needs one "
              "state scan across GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch

    import retention_chunkwise_amd as rc
    from retention_chunkwise_amd import metrics as M
    from retention_chunkwise_amd import workloads as wl

    dev = torch.device("cuda:0")
    rc.load_library()

    # ---------------- headline: chunkwise retention forward, long sequence
    w = wl.WORKLOADS["ret_fwd_long_bf16"]
    inp = wl.make_inputs(w, seed=0)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    out = torch.empty_like(v)
    fs = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)
    gamma = inp["gamma"]
    ws_n = rc.retention_fwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, q.dtype)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def fwd():
        rc.retention_fwd(q, k, v, gamma, chunk=w.chunk, out=out, final_state=fs, workspace=ws)

    kern_ms, step_ms = time_launches(fwd, args.steps, args.warmup)
    tokens = w.B * w.T
    fl_dense = M.fwd_flops(w.B, w.H, w.T, w.dk, w.dv, w.chunk)
    fl_causal = M.fwd_flops(w.B, w.H, w.T, w.dk, w.dv, w.chunk, causal=True)
    by = M.fwd_bytes(w.B, w.H, w.T, w.dk, w.dv, 2, final_state=True)
    tflops = fl_dense / (step_ms * 1e-3) / 1e12
    achieved_gbs = by / (kern_ms * 1e-3) / 1e9
    traffic = measured_traffic("fwd_ret_fwd_long_bf16", FWD_SOURCES)
    mfma = measured_mfma("fwd_ret_fwd_long_bf16", FWD_SOURCES)

    res = {
        "metric": METRIC,
        "value": tokens / (step_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "B": w.B, "H": w.H,
                   "T": w.T, "dk": w.dk, "dv": w.dv, "chunk": w.chunk, "seed": 0},
        "tflops": tflops,
        "tflops_causal_min": fl_causal / (step_ms * 1e-3) / 1e12,
        "mfma_peak_frac": tflops / M.PEAK_TFLOPS["bf16"],
        "hbm_gbs": achieved_gbs,
        "roofline": {
            # one forward call launches seg_state_kernel (segment states) and
            # seg_walk_kernel (outputs); the pair is timed as one unit
            "kernel": "retention_fwd: seg_state_kernel + seg_walk_kernel<C=128, dk=128, dv=128>",
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": M.PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / M.PEAK_HBM_GBS,
            "traffic": (traffic["bytes_per_launch"] if traffic else None),
            "algorithmic_bytes_per_launch": by,
            "kernel_ms": kern_ms,
            # matrix-core counters of the two kernels (rocprofv3 --pmc, committed summary): MFMA busy
            # share of the SIMDs, and the FLOPs the matrix cores issued per call at this call's time
            "mfma_counters": ({"walk_mfma_busy": mfma["walk"]["mfma_busy"],
                               "state_mfma_busy": mfma["state"]["mfma_busy"],
                               "issued_tflops": mfma["issued_bf16_flops_per_call"] / (kern_ms * 1e-3) / 1e12,
                               "issued_peak_frac": mfma["issued_bf16_flops_per_call"] / (kern_ms * 1e-3) / 1e12
                               / M.PEAK_TFLOPS["bf16"]} if mfma else None),
        },
        "pages_flop_comparison": {
            "T": 65536, "d": 128,
            "left_order_flops": M.attention_flops(65536, 128, 128, "left"),
            "right_order_flops": M.attention_flops(65536, 128, 128, "right"),
            "note": "analytic counts from the 'Linear attention' page; no hardware timing",
        },
    }

    progress("headline forward done")

    # ---------------- backward (dq, dk, dv) on the same workload
    if not args.no_components:
        g = torch.Generator().manual_seed(1)
        dout = torch.randn((w.B, w.H, w.T, w.dv), generator=g).to(torch.bfloat16).to(dev)
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(max(rc.retention_bwd_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk, q.dtype), 1),
                          dtype=torch.uint8, device=dev)

        def bstep():
            rc.retention_bwd(q, k, v, gamma, dout, chunk=w.chunk, dq=gq, dk=gk, dv=gv, workspace=bws)

        b_kern, b_wall = time_launches(bstep, max(args.steps // 2, 5), args.warmup, min_warm_ms=50.0)
        b_by = M.bwd_bytes(w.B, w.H, w.T, w.dk, w.dv, 2)
        b_gbs = b_by / (b_kern * 1e-3) / 1e9
        b_tr = measured_traffic("bwd_ret_fwd_long_bf16", FWD_SOURCES)
        res["backward"] = {
            "workload": w.name + " backward (dq, dk, dv given dout)", "ms_per_call": b_kern,
            "tokens_per_s": tokens / (b_wall * 1e-3), "ratio_to_forward": b_kern / kern_ms,
            "tflops": 3 * fl_dense / (b_kern * 1e-3) / 1e12,
            "roofline": {"kernel": "retention_bwd: fused time-reversed walk for dk and dv, then the dq walk",
                         "bound": "hbm", "achieved": b_gbs, "peak": M.PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": b_gbs / M.PEAK_HBM_GBS, "traffic": (b_tr["bytes_per_launch"] if b_tr else None),
                         "algorithmic_bytes_per_launch": b_by},
        }
        # the same backward given the forward's segment states: a training step keeps the forward's
        # workspace (`ws` holds the states of the forward timed above, same q, k, v, gamma and chunk)
        def bstep_ff():
            rc.retention_bwd(q, k, v, gamma, dout, chunk=w.chunk, dq=gq, dk=gk, dv=gv, workspace=bws,
                             fwd_workspace=ws)

        f_kern, f_wall = time_launches(bstep_ff, max(args.steps // 2, 5), args.warmup, min_warm_ms=50.0)
        f_gbs = b_by / (f_kern * 1e-3) / 1e9
        f_tr = measured_traffic("bwd_from_fwd_ret_fwd_long_bf16", FWD_SOURCES)
        res["backward_from_fwd"] = {
            "workload": w.name + " backward given the forward's segment states (retention_bwd_from_fwd)",
            "ms_per_call": f_kern, "tokens_per_s": tokens / (f_wall * 1e-3), "ratio_to_forward": f_kern / kern_ms,
            "roofline": {"kernel": "retention_bwd_from_fwd: fused dk/dv walk + its state pass, dq walk (no state pass)",
                         "bound": "hbm", "achieved": f_gbs, "peak": M.PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": f_gbs / M.PEAK_HBM_GBS, "traffic": (f_tr["bytes_per_launch"] if f_tr else None),
                         "algorithmic_bytes_per_launch": b_by},
        }
        del dout, gq, gk, gv, bws

    progress("backward done")

    # ---------------- the same forward with the row-sum floor and GroupNorm fused
    if not args.no_components:
        nout = torch.empty_like(v)
        nws = torch.empty(max(rc.retention_fwd_normalized_workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, w.chunk,
                                                                          q.dtype), 1), dtype=torch.uint8, device=dev)

        def nstep():
            rc.retention_fwd_normalized(q, k, v, gamma, norm="group", chunk=w.chunk, out=nout, workspace=nws)

        n_kern, n_wall = time_launches(nstep, max(args.steps // 2, 5), args.warmup, min_warm_ms=50.0)
        n_by = M.fwd_bytes(w.B, w.H, w.T, w.dk, w.dv, 2, final_state=False)
        n_gbs = n_by / (n_kern * 1e-3) / 1e9
        n_tr = measured_traffic("fwd_normalized_ret_fwd_long_bf16", FWD_SOURCES)
        res["fwd_normalized"] = {
            "workload": w.name + ", row-sum floor + GroupNorm fused (64-token chunks at d = 128)",
            "ms_per_call": n_kern, "tokens_per_s": tokens / (n_wall * 1e-3), "ratio_to_forward": n_kern / kern_ms,
            "roofline": {"kernel": "retention_fwd_normalized: seg_state_kernel + seg_walk_kernel<C=64, dk=128, dv=128, "
                                   "GroupNorm>", "bound": "hbm", "achieved": n_gbs, "peak": M.PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": n_gbs / M.PEAK_HBM_GBS,
                         "traffic": (n_tr["bytes_per_launch"] if n_tr else None)},
        }
        del nout, nws

    progress("normalised forward done")

    # ---------------- decode step and linear attention
    if not args.no_components:
        wd = wl.WORKLOADS["decode_bf16"]
        di = wl.make_inputs(wd, seed=0)
        dq, dk_, dv_ = (di[n].to(dev) for n in ("q", "k", "v"))
        state = di["state"].to(dev)
        dout = torch.empty_like(dv_)

        def dstep():
            rc.retention_decode_step(dq, dk_, dv_, di["gamma"], state, out=dout)

        d_kern, d_wall = time_launches(dstep, args.decode_steps, 10, min_warm_ms=50.0)
        d_bytes = M.decode_bytes(wd.B, wd.H, wd.dk, wd.dv, 2)
        d_gbs = d_bytes / (d_kern * 1e-3) / 1e9
        d_tr = measured_traffic("decode_kernel_decode_bf16", DECODE_SOURCES)
        res["decode"] = {
            "workload": wd.name, "steps_timed": args.decode_steps,
            "us_per_step": d_kern * 1e3, "wall_us_per_step": d_wall * 1e3,
            "tokens_per_s": wd.B / (d_wall * 1e-3),
            "gbs": d_gbs, "hbm_frac": d_gbs / M.PEAK_HBM_GBS,
            "tflops": M.decode_flops(wd.B, wd.H, wd.dk, wd.dv) / (d_kern * 1e-3) / 1e12,
            "roofline": {"bound": "hbm", "achieved": d_gbs, "peak": M.PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": d_gbs / M.PEAK_HBM_GBS,
                         "traffic": (d_tr["bytes_per_launch"] if d_tr else None)},
        }

        # the elu+1 decode step on the same shapes: (S, z) from about 100 earlier tokens
        g = torch.Generator().manual_seed(0)
        lz = (100.0 + 10.0 * torch.rand((wd.B, wd.H, wd.dk), generator=g)).to(dev)
        lS = (torch.randn((wd.B, wd.H, wd.dk, wd.dv), generator=g) * 10.0).to(dev)

        def lstep_dec():
            rc.linear_attn_decode_step(dq, dk_, dv_, lS, lz, out=dout)

        ld_kern, ld_wall = time_launches(lstep_dec, args.decode_steps, 10, min_warm_ms=50.0)
        ld_bytes = M.linattn_decode_bytes(wd.B, wd.H, wd.dk, wd.dv, 2)
        ld_gbs = ld_bytes / (ld_kern * 1e-3) / 1e9
        ld_tr = measured_traffic("linattn_decode_kernel_decode_bf16", DECODE_SOURCES)
        res["linear_attn_decode"] = {
            "workload": "linattn elu+1 decode, 256 sequences x 32 heads, 128 x 128 fp32 state + normaliser, "
                        "bf16 tokens", "steps_timed": args.decode_steps,
            "us_per_step": ld_kern * 1e3, "wall_us_per_step": ld_wall * 1e3,
            "tokens_per_s": wd.B / (ld_wall * 1e-3),
            "gbs": ld_gbs, "hbm_frac": ld_gbs / M.PEAK_HBM_GBS,
            "roofline": {"bound": "hbm", "achieved": ld_gbs, "peak": M.PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": ld_gbs / M.PEAK_HBM_GBS,
                         "traffic": (ld_tr["bytes_per_launch"] if ld_tr else None)},
        }
        del dq, dk_, dv_, state, dout, lS, lz

        wa = wl.WORKLOADS["linattn_elu1_bf16"]
        li = wl.make_inputs(wa, seed=0)
        lq, lk, lv = (li[n].to(dev) for n in ("q", "k", "v"))
        lout = torch.empty_like(lv)
        lws = torch.empty(max(rc.linear_attn_workspace_bytes(wa.B, wa.H, wa.T, wa.dk, wa.dv, lq.dtype), 1),
                          dtype=torch.uint8, device=dev)

        def lstep():
            rc.linear_attn_fwd(lq, lk, lv, out=lout, workspace=lws)

        l_kern, l_wall = time_launches(lstep, args.steps, args.warmup, min_warm_ms=50.0)
        l_fl = M.fwd_flops(wa.B, wa.H, wa.T, wa.dk, wa.dv, wa.chunk)
        l_by = M.fwd_bytes(wa.B, wa.H, wa.T, wa.dk, wa.dv, 2, final_state=False)
        l_gbs = l_by / (l_kern * 1e-3) / 1e9
        l_tr = measured_traffic("linattn_linattn_elu1_bf16", FWD_SOURCES)
        res["linear_attn"] = {
            "workload": wa.name, "ms_per_call": l_kern, "tokens_per_s": wa.B * wa.T / (l_wall * 1e-3),
            "tflops": l_fl / (l_kern * 1e-3) / 1e12,
            "mfma_peak_frac": l_fl / (l_kern * 1e-3) / 1e12 / M.PEAK_TFLOPS["bf16"],
            "gbs": l_gbs, "hbm_frac": l_gbs / M.PEAK_HBM_GBS,
            "roofline": {"kernel": "linear_attn_fwd: seg_state_kernel + seg_walk_kernel<C=128, dk=64, dv=64, LIN>",
                         "bound": "hbm", "achieved": l_gbs, "peak": M.PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": l_gbs / M.PEAK_HBM_GBS,
                         "traffic": (l_tr["bytes_per_launch"] if l_tr else None)},
        }
        del lq, lk, lv, lout, lws

    progress("decode and linear attention done")

    # ---------------- fp32 forward with final state, [4, 8, 2048, 64], chunk 64
    if not args.no_components:
        wf = wl.WORKLOADS["ret_fwd_mh_f32"]
        fi = wl.make_inputs(wf, seed=0)
        fq, fk, fv = (fi[n].to(dev) for n in ("q", "k", "v"))
        fout = torch.empty_like(fv)
        ffs = torch.empty((wf.B, wf.H, wf.dk, wf.dv), dtype=torch.float32, device=dev)

        def f32step():
            rc.retention_fwd(fq, fk, fv, fi["gamma"], chunk=wf.chunk, out=fout, final_state=ffs)

        f_kern, f_wall = time_launches(f32step, max(args.steps, 200), args.warmup, min_warm_ms=50.0)
        f_fl = M.fwd_flops(wf.B, wf.H, wf.T, wf.dk, wf.dv, wf.chunk)
        f_by = M.fwd_bytes(wf.B, wf.H, wf.T, wf.dk, wf.dv, 4, final_state=True)
        f_tf = f_fl / (f_kern * 1e-3) / 1e12
        f_tr = measured_traffic("fwd_f32_ret_fwd_mh_f32", F32_SOURCES)
        res["fwd_f32"] = {
            "workload": wf.name, "ms_per_call": f_kern, "wall_ms_per_call": f_wall,
            "tokens_per_s": wf.B * wf.T / (f_kern * 1e-3),
            "tflops": f_tf, "gbs": f_by / (f_kern * 1e-3) / 1e9,
            "roofline": {"kernel": "retention_fwd fp32: walk_kernel<fp32, C=64, dk=64>", "bound": "mfma",
                         "achieved": f_tf, "peak": M.PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                         "frac": f_tf / M.PEAK_TFLOPS["f32"],
                         "traffic": (f_tr["bytes_per_launch"] if f_tr else None),
                         "algorithmic_bytes_per_launch": f_by},
        }
        del fq, fk, fv, fout, ffs

    progress("fp32 forward done")

    # ---------------- gated linear attention (per-token, per-key-channel gates), [4, 8, 2048, 64],
    # q, k, v and out in fp32 and in bf16 (log-gates and arithmetic fp32)
    if not args.no_components:
        wf = wl.WORKLOADS["ret_fwd_mh_f32"]
        fi = wl.make_inputs(wf, seed=0)
        g = torch.Generator().manual_seed(2)
        glg = torch.nn.functional.logsigmoid(torch.randn((wf.B, wf.H, wf.T, wf.dk), generator=g) + 2.0).to(dev)
        for tag, tdt, esz in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
            gq, gk, gv = (fi[n].to(dev).to(tdt) for n in ("q", "k", "v"))
            gout = torch.empty_like(gv)
            gfs = torch.empty((wf.B, wf.H, wf.dk, wf.dv), dtype=torch.float32, device=dev)

            def glastep():
                rc.gla_fwd(gq, gk, gv, glg, out=gout, final_state=gfs)

            g_kern, g_wall = time_launches(glastep, max(args.steps, 100), args.warmup, min_warm_ms=50.0)
            g_fl = M.fwd_flops(wf.B, wf.H, wf.T, wf.dk, wf.dv, 64)
            g_tf = g_fl / (g_kern * 1e-3) / 1e12
            g_tr = measured_traffic(f"gla_gla_mh_{tag}", GLA_SOURCES)
            # q, k, v read and out written in the input type, fp32 log-gates read, fp32 final state written
            g_by = M.fwd_bytes(wf.B, wf.H, wf.T, wf.dk, wf.dv, esz, final_state=True) + wf.B * wf.H * wf.T * wf.dk * 4
            res[f"gla_{tag}"] = {
                "workload": f"gated linear attention, {tag} q/k/v/out, fp32 log-gates logsigmoid(N(2, 1)), "
                            "[4, 8, 2048, 64]",
                "ms_per_call": g_kern, "wall_ms_per_call": g_wall,
                "tokens_per_s": wf.B * wf.T / (g_kern * 1e-3), "tflops": g_tf,
                "roofline": {"kernel": "gla_fwd: state-only pass + walk, gla_kernel<dk=64, 64-column slice>",
                             "bound": "mfma", "achieved": g_tf, "peak": M.PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                             "frac": g_tf / M.PEAK_TFLOPS["f32"],
                             "traffic": (g_tr["bytes_per_launch"] if g_tr else None),
                             "algorithmic_bytes_per_launch": g_by},
            }
            del gq, gk, gv, gout, gfs
        del glg

    progress("gated linear attention done")

    # ---------------- context: a plain device copy of 1 GiB (read + write), the
    # ceiling a kernel that streams each byte once in and once out can expect
    if not args.no_components:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        c_ms, _ = time_launches(lambda: dst.copy_(src), 10, 2)
        res["hbm_copy_gbs"] = 2 * n * 4 / (c_ms * 1e-3) / 1e9
        del src, dst

    if args.calibrate_copy:
        # plain device-to-device copies of a known size, for scaling HBM counters
        n = 1 << 28  # 1 GiB of fp32
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = n * 4
        del src, dst

    progress("copy done")

    # ---------------- CPU baseline (the oracle on the host cores)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_fwd(inp, w)

    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
