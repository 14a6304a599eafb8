"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

    python -m retention_chunkwise_amd.profsum stats STATS_CSV BENCH_LOG
        kernel durations (rocprofv3 --kernel-trace --stats) next to bench.py's
        own HIP-event figures -> profiles/kernel_stats_bench_workloads.md
    python -m retention_chunkwise_amd.profsum traffic FETCH_CSV WRITE_CSV
        HBM bytes per call of each bench workload from two counter runs
        (--pmc FETCH_SIZE, then --pmc WRITE_SIZE) -> profiles/hbm_traffic_*.json
    python -m retention_chunkwise_amd.profsum mfma MFMA_CSV STATS_CSV
        matrix-core counters per kernel (issued MFMA FLOPs, MFMA busy share)
        with the kernel-trace durations -> profiles/mfma_bench_workloads.md
    python -m retention_chunkwise_amd.profsum sq SQ_CSV
        shader counters per kernel (instruction mix, LDS bank conflicts,
        waits) -> profiles/sq_bench_workloads.md

In the recorded commands $REPO is the repository root and $OUT the directory
the run writes its CSVs to.

Counter scaling: each counter is divided by what it reads, per byte, for the
plain 1 GiB device copies that `bench.py --calibrate-copy` runs in the same
process (FETCH_SIZE and WRITE_SIZE are KiB per dispatch).  A summary records
the hash of the kernel sources it was taken with; bench.py reports no traffic
once those sources change.
"""
from __future__ import annotations

import collections
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30

STATS_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats --output-format csv "
             "-d $OUT/prof_stats -o stats -- python3 $REPO/bench.py --steps 20 --warmup 3 "
             "--decode-steps 200 --no-cpu-baseline")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {ctr} --output-format csv "
           "-d $OUT/pmc_{tag} -o pmc -- python3 $REPO/bench.py --steps 3 --warmup 1 "
           "--decode-steps 20 --no-cpu-baseline --calibrate-copy")

SEG = "::seg_"
# One call of each bench workload: (part of the kernel name, dispatches per call).
# The dq walk of the backward is an ordinary forward walk with the same
# shapes as the long forward, so both share those two kernels' averages.
WORKLOADS = {
    "fwd_ret_fwd_long_bf16": {
        "what": "retention_fwd, [1, 32, 65536, 128] bf16, chunk 128",
        "kernels": [(SEG + "state_kernel<128, 128, 0, false>", 1),
                    (SEG + "walk_kernel<128, 128, 128, 0>", 1)],
        "algorithmic": 2149580800, "sources": "FWD_SOURCES"},
    "bwd_ret_fwd_long_bf16": {
        "what": "retention_bwd on the long workload: the fused reverse walk for dk and dv (with its state "
                "pass), then the dq walk (forward, with its state pass)",
        "kernels": [(SEG + "state_kernel<128, 128, 0, true>", 1),
                    (SEG + "bwd_kv_kernel<128, 128>", 1),
                    (SEG + "state_kernel<128, 128, 0, false>", 1),
                    (SEG + "walk_kernel<128, 128, 128, 0>", 1)],
        "algorithmic": 3758096384, "sources": "FWD_SOURCES"},
    "bwd_from_fwd_ret_fwd_long_bf16": {
        "what": "retention_bwd_from_fwd on the long workload: as retention_bwd, but the dq walk reads the "
                "forward's segment states and runs no state pass",
        "kernels": [(SEG + "state_kernel<128, 128, 0, true>", 1),
                    (SEG + "bwd_kv_kernel<128, 128>", 1),
                    (SEG + "walk_kernel<128, 128, 128, 0>", 1)],
        "algorithmic": 3758096384, "sources": "FWD_SOURCES"},
    "fwd_normalized_ret_fwd_long_bf16": {
        "what": "retention_fwd_normalized (row-sum floor + GroupNorm) on the long workload",
        "kernels": [(SEG + "state_kernel<128, 128, 2, false>", 1),
                    (SEG + "walk_kernel<64, 128, 128, 3>", 1)],
        "algorithmic": 2147483648, "sources": "FWD_SOURCES"},
    "linattn_linattn_elu1_bf16": {
        "what": "linear_attn_fwd, elu+1, [8, 16, 8192, 64] bf16",
        "kernels": [(SEG + "state_kernel<64, 64, 1, false>", 1),
                    (SEG + "walk_kernel<128, 64, 64, 1>", 1)],
        "algorithmic": 536870912, "sources": "FWD_SOURCES"},
    "decode_kernel_decode_bf16": {
        "what": "retention_decode_step, 256 x 32 heads, 128 x 128 fp32 state",
        "kernels": [("::decode_kernel<true, 128, 128, false>", 1)],
        "algorithmic": 1082130432, "sources": "DECODE_SOURCES"},
    "linattn_decode_kernel_decode_bf16": {
        "what": "linear_attn_decode_step, 256 x 32 heads, 128 x 128 fp32 state + normaliser",
        "kernels": [("::decode_kernel<true, 128, 128, true>", 1)],
        "algorithmic": 1082130432 + 2 * 256 * 32 * 128 * 4, "sources": "DECODE_SOURCES"},
    "fwd_f32_ret_fwd_mh_f32": {
        "what": "retention_fwd fp32 [4, 8, 2048, 64], chunk 64, final state",
        "kernels": [("::slice_state_kernel<false, 64, 64, 0>", 1),
                    ("walk::walk_kernel<false, 64, 64, 2, 0>", 1)],
        "algorithmic": 4 * 8 * 2048 * 64 * 4 * 4 + 4 * 8 * 64 * 64 * 4, "sources": "F32_SOURCES"},
    "gla_gla_mh_f32": {
        "what": "gla_fwd fp32 [4, 8, 2048, 64], final state (state-only pass + walk)",
        "kernels": [("::gla_kernel<false, 64, 4, true>", 1),
                    ("::gla_kernel<false, 64, 4, false>", 1)],
        "algorithmic": 4 * 8 * 2048 * 64 * 4 * 5 + 4 * 8 * 64 * 64 * 4, "sources": "GLA_SOURCES"},
    "gla_gla_mh_bf16": {
        "what": "gla_fwd bf16 q/k/v/out, fp32 log-gates, [4, 8, 2048, 64], final state",
        "kernels": [("::gla_kernel<true, 64, 4, true>", 1),
                    ("::gla_kernel<true, 64, 4, false>", 1)],
        "algorithmic": 4 * 8 * 2048 * 64 * (4 * 2 + 4) + 4 * 8 * 64 * 64 * 4, "sources": "GLA_SOURCES"},
}


def _bench():
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (for the source lists and their hash)

    return bench


def _strip_args(name: str) -> str:
    """Kernel name without its parameter list (the last parenthesised part)."""
    return name[:name.rfind("(")] if name.endswith(")") else name


def _per_dispatch(path: str) -> dict[str, list[float]]:
    """Counter value per dispatch, grouped by kernel name (signature dropped)."""
    per = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            per[d] += float(r["Counter_Value"])
            names[d] = _strip_args(r["Kernel_Name"])
    out = collections.defaultdict(list)
    for d in sorted(per):
        out[names[d]].append(per[d])
    return out


def _find(groups: dict[str, list[float]], key: str) -> list[float]:
    hits = [v for k, v in groups.items() if key in k]
    if len(hits) != 1:
        raise SystemExit(f"profsum: expected one kernel whose name contains {key!r}, found {len(hits)}")
    return hits[0]


def traffic(fetch_csv: str, write_csv: str, out_dir: str = PROFILES) -> None:
    b = _bench()
    fetch, write = _per_dispatch(fetch_csv), _per_dispatch(write_csv)
    cf, cw = _find(fetch, COPY_KERNEL), _find(write, COPY_KERNEL)
    cf_kib, cw_kib = sum(cf) / len(cf), sum(cw) / len(cw)
    fscale, wscale = COPY_BYTES / (cf_kib * 1024), COPY_BYTES / (cw_kib * 1024)
    for name, spec in WORKLOADS.items():
        srcs = getattr(b, spec["sources"])
        ks, fb, wb = [], 0.0, 0.0
        for prefix, per_call in spec["kernels"]:
            fv, wv = _find(fetch, prefix), _find(write, prefix)
            fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
            ks.append({"kernel": prefix, "per_call": per_call, "dispatches_fetch": len(fv),
                       "dispatches_write": len(wv), "fetch_kib_raw": fk, "write_kib_raw": wk,
                       "fetch_bytes": fk * 1024 * fscale, "write_bytes": wk * 1024 * wscale})
            fb += per_call * fk * 1024 * fscale
            wb += per_call * wk * 1024 * wscale
        d = {"workload": spec["what"], "kernels": ks, "source_sha": b.sources_sha(srcs), "sources": srcs,
             "fetch_scale": fscale, "write_scale": wscale, "fetch_bytes": fb, "write_bytes": wb,
             "bytes_per_launch": fb + wb, "algorithmic_bytes_per_launch": spec["algorithmic"],
             "traffic_over_algorithmic": (fb + wb) / spec["algorithmic"],
             "calibration": (f"plain 1 GiB device copy ({COPY_KERNEL}): FETCH_SIZE read {cf_kib:.1f} KiB, "
                             f"WRITE_SIZE {cw_kib:.1f} KiB"),
             "commands": [PMC_CMD.format(ctr="FETCH_SIZE", tag="fetch"),
                          PMC_CMD.format(ctr="WRITE_SIZE", tag="write")]}
        with open(os.path.join(out_dir, f"hbm_traffic_{name}.json"), "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
        print(f"{name}: {(fb + wb) / 1e9:.3f} GB per call ({(fb + wb) / spec['algorithmic']:.2f}x algorithmic)")


MFMA_COUNTERS = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"
MFMA_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + MFMA_COUNTERS + " --output-format csv "
            "-d $OUT/pmc_mfma -o pmc -- python3 $REPO/bench.py --steps 3 --warmup 1 "
            "--decode-steps 20 --no-cpu-baseline")
SIMDS = 256 * 4        # MI355X: 256 CUs, 4 SIMDs each
XCDS = 8               # GRBM_GUI_ACTIVE arrives summed over the XCDs; one XCD's count is the busy time
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense matrix-core peaks


def _per_dispatch_counters(path: str):
    """{dispatch: (kernel, {counter: value})}; every counter summed over the
    rows of its dispatch."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            name, ctrs = out.setdefault(d, (_strip_args(r["Kernel_Name"]), {}))
            c, v = r["Counter_Name"], float(r["Counter_Value"])
            ctrs[c] = ctrs.get(c, 0.0) + v
    return out


def mfma(mfma_csv: str, stats_csv: str, out_dir: str = PROFILES) -> None:
    per = _per_dispatch_counters(mfma_csv)
    dur = {}
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            dur[_strip_args(r["Name"])] = float(r["AverageNs"])
    agg = collections.OrderedDict()
    for d in sorted(per):
        name, c = per[d]
        if not name.startswith("void ret::"):
            continue
        a = agg.setdefault(name, collections.defaultdict(float))
        a["n"] += 1
        for k, v in c.items():
            a[k] += v
    out = ["# Matrix-core counters — bench workloads on one MI355X", "",
           "Command ($REPO: repository root, $OUT: output directory):", "", "    " + MFMA_CMD, "",
           "Issued FLOPs are the MFMA operation counters times 512 (the counters count 512-FLOP units), "
           "averaged per dispatch; they include the masked and zero-padded parts of tiles and the recomputed "
           "products, so they exceed the algorithmic FLOPs. MFMA busy is SQ_VALU_MFMA_BUSY_CYCLES summed over "
           f"the {SIMDS} SIMDs divided by {SIMDS} x the busy cycles of one XCD (rocprofv3's MfmaUtil). "
           f"GRBM_GUI_ACTIVE arrives summed over the {XCDS} XCDs: divided by {XCDS} it matches the kernel's duration "
           "at a 2.0 GHz clock (372,078 cycles for the 185.8 µs state kernel). The issued rate "
           "divides the issued FLOPs by the kernel's average duration from profiles/kernel_stats_bench_workloads.md "
           "and compares it with the dense peak of its own dtype (bf16 2.5 PFLOP/s, fp32 157.3 TFLOP/s).", "",
           "| kernel | dispatches | issued bf16 GFLOP | issued fp32 GFLOP | MFMA busy | avg µs | issued TFLOP/s | % of dtype peak |",
           "|---|---|---|---|---|---|---|---|"]
    for name, a in agg.items():
        n = a["n"]
        fb = a.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512 / n
        ff = a.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512 / n
        busy = a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n
        act = a.get("GRBM_GUI_ACTIVE", 0.0) / n / XCDS
        util = 100.0 * busy / (act * SIMDS) if act > 0 else float("nan")
        us = dur.get(name, float("nan")) / 1e3
        dt = "bf16" if fb >= ff else "f32"
        fl = fb if dt == "bf16" else ff
        rate = fl / (us * 1e-6) / 1e12 if us == us and us > 0 else float("nan")
        out.append(f"| `{name.replace('void ret::', '')}` | {n:.0f} | {fb / 1e9:,.2f} | {ff / 1e9:,.2f} | "
                   f"{util:.1f} % | {us:,.1f} | {rate:,.1f} ({dt}) | {100 * rate / PEAK_TFLOPS[dt]:.1f} % |")
    from retention_chunkwise_amd import metrics as M

    b = _bench()
    f_dense = M.fwd_flops(1, 32, 65536, 128, 128, 128)
    f_causal = M.fwd_flops(1, 32, 65536, 128, 128, 128, causal=True)
    walk = agg.get("void ret::seg::seg_walk_kernel<128, 128, 128, 0>")
    state = agg.get("void ret::seg::seg_state_kernel<128, 128, 0, false>")
    if walk and state:
        def one(a):
            n = a["n"]
            return {"issued_bf16_flops": a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / n,
                    "mfma_busy": a["SQ_VALU_MFMA_BUSY_CYCLES"] / n / (a["GRBM_GUI_ACTIVE"] / n / XCDS * SIMDS)}
        w1, s1 = one(walk), one(state)
        issued = w1["issued_bf16_flops"] + s1["issued_bf16_flops"]
        out += ["", f"One long forward ([1, 32, 65536, 128] bf16, chunk 128) issues {issued / 1e9:.1f} GFLOP on the "
                f"matrix cores: the walk {w1['issued_bf16_flops'] / 1e9:.1f} (causal tiles only) and the state kernel "
                f"{s1['issued_bf16_flops'] / 1e9:.1f} (the segment sums, computed a second time by the segment "
                f"decomposition). The algorithmic count is {f_dense / 1e9:.1f} GFLOP dense (F_dense, the headline "
                f"figure) and {f_causal / 1e9:.1f} GFLOP causal minimum."]
        d = {"workload": "retention_fwd, [1, 32, 65536, 128] bf16, chunk 128", "walk": w1, "state": s1,
             "issued_bf16_flops_per_call": issued, "algorithmic_flops_dense": f_dense,
             "algorithmic_flops_causal": f_causal, "source_sha": b.sources_sha(b.FWD_SOURCES),
             "sources": b.FWD_SOURCES, "command": MFMA_CMD,
             "note": "mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x one XCD's GRBM_GUI_ACTIVE)"}
        with open(os.path.join(out_dir, "mfma_fwd_ret_fwd_long_bf16.json"), "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
    out += ["", _source_hashes(b)]
    with open(os.path.join(out_dir, "mfma_bench_workloads.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


SQ_COUNTERS = ("SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE "
               "SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE")
SQ_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + SQ_COUNTERS + " --output-format csv "
          "-d $OUT/pmc_sq -o pmc -- python3 $REPO/bench.py --steps 3 --warmup 1 --decode-steps 20 --no-cpu-baseline")


def sq(sq_csv: str, out_dir: str = PROFILES) -> None:
    per = _per_dispatch_counters(sq_csv)
    agg = collections.OrderedDict()
    for d in sorted(per):
        name, c = per[d]
        if not name.startswith("void ret::"):
            continue
        a = agg.setdefault(name, collections.defaultdict(float))
        a["n"] += 1
        for k, v in c.items():
            a[k] += v
    out = ["# Shader counters — bench workloads on one MI355X", "",
           "Command ($REPO: repository root, $OUT: output directory):", "", "    " + SQ_CMD, "",
           "Per dispatch, averaged over the run's dispatches of each kernel. Instruction counts are per wave "
           "(SQ_INSTS_* / SQ_WAVES). LDS conflict share: SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE, the share of "
           "LDS-indexing cycles lost to bank conflicts. Wait: SQ_WAIT_INST_ANY per wave, in units of "
           "one XCD's active cycles (GRBM_GUI_ACTIVE / " + str(XCDS) + "), i.e. roughly how much of the kernel's time "
           "an average wave spent waiting for any instruction's operands (memory or LDS); the counter samples "
           "every fourth cycle on some parts, so read it as a relative figure between kernels.", "",
           "| kernel | waves | VALU / wave | MFMA / wave | LDS / wave | LDS conflict share | wait / active |",
           "|---|---|---|---|---|---|---|"]
    for name, a in agg.items():
        n = a["n"]
        waves = a.get("SQ_WAVES", 0.0) / n
        w = max(waves, 1.0)
        valu, mfma_, lds = (a.get(k, 0.0) / n / w for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS"))
        conf = a.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(a.get("SQ_LDS_IDX_ACTIVE", 0.0), 1.0)
        act = a.get("GRBM_GUI_ACTIVE", 0.0) / n / XCDS
        wait = a.get("SQ_WAIT_INST_ANY", 0.0) / n / w / act if act > 0 else float("nan")
        out.append(f"| `{name.replace('void ret::', '')}` | {waves:,.0f} | {valu:,.0f} | {mfma_:,.0f} | {lds:,.0f} | "
                   f"{100 * conf:.1f} % | {wait:.2f} |")
    out += ["", _source_hashes(_bench())]
    with open(os.path.join(out_dir, "sq_bench_workloads.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


BENCH_LINES = [("retention forward (long bf16, state + walk kernels)", ("roofline", "kernel_ms"), 1e6, "ns per call"),
               ("backward (dq, dk, dv) of the long forward", ("backward", "ms_per_call"), 1e6, "ns per call"),
               ("backward given the forward's segment states", ("backward_from_fwd", "ms_per_call"), 1e6,
                "ns per call"),
               ("forward with row-sum floor + GroupNorm (long bf16)", ("fwd_normalized", "ms_per_call"), 1e6,
                "ns per call"),
               ("decode step", ("decode", "us_per_step"), 1e3, "ns per step"),
               ("elu+1 decode step", ("linear_attn_decode", "us_per_step"), 1e3, "ns per step"),
               ("linear attention [8, 16, 8192, 64] bf16", ("linear_attn", "ms_per_call"), 1e6, "ns per call"),
               ("fp32 forward [4, 8, 2048, 64]", ("fwd_f32", "ms_per_call"), 1e6, "ns per call"),
               ("gated linear attention fp32 [4, 8, 2048, 64]", ("gla_f32", "ms_per_call"), 1e6, "ns per call"),
               ("gated linear attention bf16 [4, 8, 2048, 64]", ("gla_bf16", "ms_per_call"), 1e6, "ns per call")]


def _source_hashes(b) -> str:
    """The hashes of the kernel sources a summary was taken with (bench.py's source lists)."""
    return ("Source hashes: segment kernels " + b.sources_sha(b.FWD_SOURCES) + ", decode "
            + b.sources_sha(b.DECODE_SOURCES) + ", fp32 walk " + b.sources_sha(b.F32_SOURCES) + ", GLA "
            + b.sources_sha(b.GLA_SOURCES) + ".")


def stats(stats_csv: str, bench_log: str, out_dir: str = PROFILES) -> None:
    b = _bench()
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            n = r["Name"]
            if n.startswith("void ret::"):
                rows.append((_strip_args(n).replace("void ret::", ""), int(r["Calls"]), float(r["AverageNs"]),
                             float(r["MinNs"]), float(r["MaxNs"]), float(r["TotalDurationNs"])))
    rows.sort(key=lambda x: -x[5])
    line = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    out = ["# Kernel durations — bench workloads on one MI355X", "",
           "Command ($REPO: repository root, $OUT: output directory):", "", "    " + STATS_CMD, "",
           "| kernel | calls | avg ns | min ns | max ns |", "|---|---|---|---|---|"]
    for n, c, a, mn, mx, _ in rows:
        out.append(f"| `{n}` | {c} | {a:,.0f} | {mn:,.0f} | {mx:,.0f} |")
    out += ["", "bench.py's own HIP-event figures in the same run:", ""]
    for label, (k1, k2), mul, unit in BENCH_LINES:
        if k1 in res and k2 in res[k1]:
            out.append(f"- {label}: {res[k1][k2] * mul:,.0f} {unit}")
    out += ["", _source_hashes(b)]
    with open(os.path.join(out_dir, "kernel_stats_bench_workloads.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 4 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 4 and sys.argv[1] == "mfma":
        mfma(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 3 and sys.argv[1] == "sq":
        sq(sys.argv[2])
    else:
        raise SystemExit(__doc__)
