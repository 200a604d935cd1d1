#!/usr/bin/env python3
"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

--pass bwd times fa_bwd instead (the backward pass, fed by one forward
call), and --varlen S times fa_fwd_varlen on the workload's tokens cut into
S sequences; both print separate lines, not the default one.

One step is one call of fa_fwd_ws (the whole forward pass: the attention
kernel and, when the plan splits long query tiles, the kernel that combines
the parts) over the workload's synthetic inputs, which are resident in
device memory before timing starts; --entry fa_fwd times the unsplit entry.
W untimed steps are followed by exactly K timed steps, bracketed by device
synchronisation.  Prints ONE JSON line: throughput in TFLOP/s counting
4*B*H*Nq*Nk*D flops (halved when causal), the roofline of the attention
kernel (HIP-event time per step on the launch stream, which also holds the
short combine kernel when the plan splits, against the dense MFMA peak of
the input type), and the CPU oracle's throughput on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak (B8 N4096 D128 causal)"
METRIC_BWD = "attention bwd TFLOP/s + % bf16 MFMA peak (2.5x fwd flops)"
# MI355X published dense peaks (TFLOP/s).
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
# Transcendental rate for the exp roofline of small head dims: v_exp_f32
# issues a wave64 every 8 cycles per SIMD on MI355X (measured with
# independent chains, two waves per SIMD: half the 64-lane VALU rate), so 32
# per clock per CU (256 CUs, 2.4 GHz).
EXP_PEAK_T = 32 * 256 * 2.4e9 / 1e12
# dense bf16/fp16 MFMA work per clock per CU (v_mfma_f32_32x32x16: 32768 flop
# in 32 cycles on each of the 4 SIMDs): the peak derived from the device
BF16_FLOP_PER_CLK_CU = 4096
HBM_GBPS = 8000.0
CSRC = os.path.join(ROOT, "transformer_attention_07_amd", "csrc")
FWD_SOURCES = ("fa_fwd.hip", "stream_plan.h")
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def source_digest() -> str:
    """sha256 over the forward pass's kernel sources (in name order): the
    traffic record is valid while these are unchanged."""
    h = hashlib.sha256()
    for name in FWD_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per step (every kernel of one call) from committed rocprofv3
    counter runs, if they were taken on the current kernel source; else None."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_digest():
        return None
    return t.get("bytes_per_step")


def write_traffic(run_dir: str, workload: str = "bf16_b8_n4096_d128_causal") -> dict:
    """Builds profiles/traffic_<workload>.json from two rocprofv3 counter runs
    of this script on the workload (run_dir/fetch: --pmc FETCH_SIZE,
    run_dir/write: --pmc WRITE_SIZE; both with --copy-probe-mib 256 and
    --output-format csv).  Each counter, in KiB per dispatch, is scaled by
    what it reads for the probe's plain copy of 256 MiB; the record is keyed
    to the forward sources' digest, so bench.py ignores it once they change."""
    import csv
    import statistics

    def read(kind, counter):
        by = {}
        with open(os.path.join(run_dir, kind, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return by

    fetch, write = read("fetch", "FETCH_SIZE"), read("write", "WRITE_SIZE")
    copy = [n for n in fetch if "copyBuffer" in n]
    if not copy:
        raise SystemExit("no copy kernel in the fetch run (run with --copy-probe-mib 256)")
    copy_bytes = 256 * (1 << 20)
    copy_f = fetch[copy[0]][0]
    copy_w = write[[n for n in write if "copyBuffer" in n][0]][0]
    ff, wf = copy_bytes / (copy_f * 1024), copy_bytes / (copy_w * 1024)
    from workloads import WORKLOADS

    w = WORKLOADS[workload]
    out = {"workload": workload, "entry": "fa_fwd_ws (every kernel of one call)",
           "source_sha256": source_digest(), "source_files": list(FWD_SOURCES), "kernels": {}}
    total = 0.0
    counts = {"fetch": {}, "write": {}}
    for name in sorted(n for n in fetch if "fa_" in n):
        fk, wk = fetch[name], write.get(name, [])
        if not wk:
            continue
        b = statistics.mean(fk) * 1024 * ff + statistics.mean(wk) * 1024 * wf
        out["kernels"][name] = {"fetch_kib_per_launch": round(statistics.mean(fk), 1),
                                "write_kib_per_launch": round(statistics.mean(wk), 1),
                                "bytes": int(b)}
        counts["fetch"][name] = len(fk)
        counts["write"][name] = len(wk)
        total += b
    out["calibration"] = {"copy_bytes": copy_bytes, "copy_fetch_kib": round(copy_f, 1),
                          "copy_write_kib": round(copy_w, 1), "fetch_factor": round(ff, 5),
                          "write_factor": round(wf, 5)}
    out["bytes_per_step"] = int(total)
    s_in = 4 if w.dtype == "f32" else 2
    out["algorithmic_bytes_per_step"] = (3 * w.B * w.H * w.N * w.D * s_in
                                         + w.B * w.H * w.N * (w.D * s_in + 4))
    out["launches_counted"] = counts
    out["commands"] = [
        f"cd /tmp && rocprofv3 --pmc {c} -d <out>/{k} -o run --output-format csv -- python3 "
        f"/root/repo/bench.py --workload {workload} --steps 20 --warmup 2 --no-cpu-baseline "
        f"--copy-probe-mib 256" for c, k in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"))]
    out["commands"].append(f"python3 /root/repo/bench.py --write-traffic <out>")
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def masked_visible(N: int, W: int, G: int, causal):
    """Visible keys of each row of an N x N local-window + global-token mask
    (the library's rule): causal, all j <= i for a global row, else the
    window [i - W + 1, i] plus the global keys before it; non-causal, every
    key for a global row, else the band |i - j| < W plus the global keys
    outside it."""
    import numpy as np

    i = np.arange(N, dtype=np.int64)
    lo = np.maximum(0, i - W + 1)
    if causal:
        return np.where(i < G, i + 1, (i - lo + 1) + np.minimum(G, lo))
    hi = np.minimum(N - 1, i + W - 1)
    band = (hi - lo + 1) + np.minimum(G, lo) + np.maximum(0, np.minimum(G, N) - hi - 1)
    return np.where(i < G, N, band)


def device_facts(torch, dev):
    """What the box reports about itself: compute units, the maximum shader
    clock (HIP device attribute, else the highest level the driver lists in
    sysfs), the bf16 peak they give (CUs x 4096 flop/clk x clock), the ROCm
    version and the host CPU."""
    import ctypes
    import glob

    props = torch.cuda.get_device_properties(dev)
    facts = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
             "cus": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        # hipDeviceAttributeMultiprocessorCount checks the enum numbering
        # before hipDeviceAttributeClockRate (kHz) is trusted
        if (hip.hipDeviceGetAttribute(ctypes.byref(val), 65, dev.index or 0) == 0
                and val.value == props.multi_processor_count
                and hip.hipDeviceGetAttribute(ctypes.byref(val), 7, dev.index or 0) == 0):
            facts["max_sclk_mhz"] = val.value / 1000.0
    except OSError:
        pass
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                lv = f.read().split()
        except OSError:
            continue
        facts["sclk_levels"] = " ".join(lv)
        mhz = [float(x.lower().replace("mhz", "")) for x in lv if x.lower().endswith("mhz")]
        if mhz and "max_sclk_mhz" not in facts:
            facts["max_sclk_mhz"] = max(mhz)  # the highest clock level the driver lists
        break
    if "max_sclk_mhz" in facts:
        facts["peak_bf16_derived_tflops"] = round(
            facts["cus"] * BF16_FLOP_PER_CLK_CU * facts["max_sclk_mhz"] * 1e6 / 1e12, 1)
    try:
        with open("/opt/rocm/.info/version") as f:
            facts["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    facts["host_cpu"] = ln.split(":", 1)[1].strip()
                    break
        facts["host_threads"] = len(os.sched_getaffinity(0))
    except OSError:
        pass
    return facts


def cpu_baseline_one_core(w, rows_n: int = 256):
    """The same oracle on ONE host thread over rows_n seeded sampled rows
    (seed 9), its time scaled to the whole workload by the count of visible
    keys (extrapolated)."""
    import numpy as np
    import oracle
    from workloads import gen_workload, sample_rows

    q, k, v = gen_workload(w)
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    scale = 1.0 / math.sqrt(w.D)
    lib = oracle.load()

    def visible(rows):
        i = rows % w.N
        return float((i + 1).sum() if w.causal else len(rows) * w.N)

    rows = sample_rows(w.rows, min(rows_n, w.rows), 9).numpy()
    prev = oracle.set_threads(1, lib)
    try:
        t0 = time.perf_counter()
        oracle.attention(qn, kn, vn, scale, w.causal, rows=rows, lib=lib)
        el = time.perf_counter() - t0
    finally:
        oracle.set_threads(prev, lib)
    t_full = el * visible(np.arange(w.rows)) / visible(rows)
    return {"value": w.flops() / t_full / 1e12, "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(rows)} of {w.rows} rows drawn uniformly (seed 9) on one thread; "
                      f"time extrapolated to the whole workload by the count of visible keys",
            "seconds": round(el, 3), "seconds_full_workload_extrapolated": round(t_full, 3)}


def cpu_baseline(w, target_s: float):
    """Time the fp64 oracle on the host cores over a bounded sample of rows and
    express it in the metric's unit (flops of the whole workload / time)."""
    import numpy as np
    import oracle
    from workloads import gen_workload, sample_rows

    q, k, v = gen_workload(w)
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    scale = 1.0 / math.sqrt(w.D)
    lib = oracle.load()
    total = w.rows

    def visible(rows):
        i = rows % w.N
        return (i + 1).sum() if w.causal else len(rows) * w.N

    all_rows = np.arange(total)
    work_total = float(visible(all_rows))
    probe = sample_rows(total, 64, 7).numpy()
    t0 = time.perf_counter()
    oracle.attention(qn, kn, vn, scale, w.causal, rows=probe, lib=lib)
    t_probe = time.perf_counter() - t0
    est_full = t_probe * work_total / float(visible(probe))
    reps = 1
    if est_full <= target_s:
        # the whole workload fits the time budget: repeat it to fill the budget
        reps = int(max(1, min(50, target_s / max(est_full, 1e-9))))
        rows, desc = None, f"all {total} rows of the workload, {reps} passes"
        work = work_total * reps
    else:
        n = int(max(64, min(total, 64 * target_s / max(t_probe, 1e-9))))
        rows = sample_rows(total, n, 8).numpy()
        work = float(visible(rows))
        desc = (f"{n} of {total} rows drawn uniformly (seed 8); time scaled to the "
                f"whole workload by the count of visible keys")
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attention(qn, kn, vn, scale, w.causal, rows=rows, lib=lib)
    elapsed = time.perf_counter() - t0
    t_full = elapsed * work_total / work
    return {
        "value": w.flops() / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(lib),
        "kind": "oracle",
        "sample": desc,
        "seconds": round(elapsed, 3),
        "seconds_full_workload": round(t_full, 6),
    }


def cpu_baseline_bwd(w, target_s: float):
    """Time the fp64 oracle's backward pass on the host cores over the whole
    workload (repeated to fill the time budget when it is short)."""
    import oracle
    from workloads import gen_grad_out, gen_workload

    q, k, v = gen_workload(w)
    g = gen_grad_out(w.B, w.H, w.N, w.D, seed=w.seed + 10000, dtype=w.dtype)
    qn, kn, vn, gn = (t.double().numpy() for t in (q, k, v, g))
    scale = 1.0 / math.sqrt(w.D)
    lib = oracle.load()
    t0 = time.perf_counter()
    oracle.attention_bwd(qn, kn, vn, gn, scale, w.causal, lib=lib)
    first = time.perf_counter() - t0
    reps = int(max(0, min(20, target_s / max(first, 1e-9) - 1)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.attention_bwd(qn, kn, vn, gn, scale, w.causal, lib=lib)
    elapsed = first + (time.perf_counter() - t0)
    t_full = elapsed / (reps + 1)
    return {
        "value": 2.5 * w.flops() / t_full / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(lib),
        "kind": "oracle",
        "sample": f"the whole workload's dQ, dK, dV, {reps + 1} passes",
        "seconds": round(elapsed, 3),
        "seconds_full_workload": round(t_full, 6),
    }


def cpu_baseline_rows(run_rows, total_rows: int, flops_total: float, work_of, target_s: float,
                      desc: str):
    """Time an oracle on a uniform sample of its rows (64 first, to size the
    sample for about target_s), scaled to the whole workload by the rows'
    share of the work (work_of(rows) / work_of(all rows))."""
    import numpy as np
    import oracle
    from workloads import sample_rows

    probe = sample_rows(total_rows, min(64, total_rows), 7).numpy()
    t0 = time.perf_counter()
    run_rows(probe)
    t_probe = time.perf_counter() - t0
    n = int(max(64, min(total_rows, 64 * target_s / max(t_probe, 1e-9))))
    rows = sample_rows(total_rows, n, 8).numpy()
    t0 = time.perf_counter()
    run_rows(rows)
    elapsed = time.perf_counter() - t0
    frac = work_of(rows) / work_of(np.arange(total_rows))
    t_full = elapsed / frac
    return {"value": flops_total / t_full / 1e12, "unit": "TFLOP/s",
            "cores": oracle.threads(), "kind": "oracle",
            "sample": f"{n} of {total_rows} rows drawn uniformly (seed 8), {desc}; time "
                      f"scaled to the whole workload by the rows' share of the work",
            "seconds": round(elapsed, 3), "seconds_full_workload": round(t_full, 6)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: B=8 N=4096 D=128 causal bf16)")
    ap.add_argument("--out-f32", action="store_true",
                    help="store O in fp32 (FA_BF16_OF32) instead of the input type")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy this many MiB device-to-device once "
                         "(a plain copy of known size, to calibrate HBM byte "
                         "counters in a profiler run)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--entry", choices=("fa_fwd_ws", "fa_fwd"), default="fa_fwd_ws",
                    help="C entry point to time (default: fa_fwd_ws, with scratch)")
    ap.add_argument("--varlen", type=int, default=0, metavar="S",
                    help="time fa_fwd_varlen instead: the workload's tokens (B*N, one "
                         "head) cut into S sequences of seeded lengths (seed 77, at "
                         "least 64 tokens each), flops summed per sequence")
    ap.add_argument("--split", action="store_true",
                    help="with --varlen: time fa_fwd_varlen_ws (long tiles cut over their "
                         "keys, caller-owned workspace) instead of fa_fwd_varlen")
    ap.add_argument("--masked", default=None, metavar="W,G",
                    help="time fa_fwd_masked instead: B=1 H=8 N=32768 D=128 causal bf16 "
                         "under a local window W with G global tokens; flops counted "
                         "over the visible pairs only (4*D each)")
    ap.add_argument("--noncausal", action="store_true",
                    help="with --masked: the rule without causality (global queries see "
                         "every key; fa_fwd_masked_ws with its workspace)")
    ap.add_argument("--write-traffic", default=None, metavar="DIR",
                    help="write profiles/traffic_<workload>.json from the rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE runs under DIR (no GPU work)")
    ap.add_argument("--fp8-nows", action="store_true",
                    help="with --fp8: time fa_fwd_fp8 (no workspace, the query-stationary "
                         "kernel) instead of fa_fwd_fp8_ws")
    ap.add_argument("--fp8", action="store_true",
                    help="time fa_fwd_fp8_ws on the workload's shape with e4m3 inputs (scores on "
                         "FP8 MFMA, P.V in bf16: roofline peak 1/(0.5/5000 + 0.5/2516.6) "
                         "TFLOP/s)")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward pass (default) or the backward pass "
                         "(fa_bwd, fed by one forward call; flops counted as 2.5x "
                         "the forward's: the five N x N contractions of the "
                         "recomputing backward)")
    args = ap.parse_args()

    if args.write_traffic:
        from workloads import HEADLINE

        rec = write_traffic(args.write_traffic, args.workload or HEADLINE)
        print(json.dumps({k: rec[k] for k in ("workload", "bytes_per_step",
                                              "algorithmic_bytes_per_step")}))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(sharded over batch*heads, each GPU would run this same "
              "single-GPU path with no exchange)", file=sys.stderr)
        return 2

    import torch
    import transformer_attention_07_amd as fa
    from workloads import HEADLINE, WORKLOADS, gen_workload

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (t.to(dev) for t in gen_workload(w))
    in_dt = q.dtype
    out_dt = torch.float32 if (args.out_f32 or in_dt == torch.float32) else in_dt
    code = fa._dtype_code(torch, in_dt, out_dt)
    o = torch.empty(q.shape, dtype=out_dt, device=dev)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(w.D)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    lib = fa.library()
    argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.N, w.N, w.D, scale, int(w.causal), code)
    ws_bytes = 0
    if args.entry == "fa_fwd_ws":
        st, ws_bytes = fa.fa_fwd_workspace_size(w.B, w.H, w.N, w.N, w.D, int(w.causal),
                                                code)
        if st != 0:
            raise RuntimeError(f"fa_fwd_workspace_size failed: {fa.fa_status_str(st)}")
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        argv = argv + (ws.data_ptr(), ws_bytes, sp)
        call = lib.fa_fwd_ws
    else:
        argv = argv + (sp,)
        call = lib.fa_fwd

    bwd = args.which == "bwd"
    lens = None
    masked = None
    if args.masked:
        import numpy as np
        from workloads import gen_qkv

        if args.varlen:
            raise SystemExit("--masked and --varlen are separate modes")
        W, G = (int(x) for x in args.masked.split(","))
        MB, MH, MN, MD = 1, 8, 32768, 128
        q, k, v = (t.to(dev) for t in gen_qkv(MB, MH, MN, MN, MD, seed=2601, dtype="bf16"))
        o = torch.empty(q.shape, dtype=out_dt, device=dev)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(MD)
        MC = 0 if args.noncausal else 1
        per_row = masked_visible(MN, W, G, MC)
        masked = {"window": W, "global": G, "visible_pairs": int(per_row.sum()) * MB * MH,
                  "shape": [MB, MH, MN, MD], "causal": bool(MC)}
        if MC:
            argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), MB,
                    MH, MN, MN, MD, scale, 1, W, G, code, sp)
            call = lib.fa_fwd_masked
            args.entry = "fa_fwd_masked"
        else:
            st, fws_bytes = fa.fa_fwd_masked_workspace_size(MB, MH, MN, MN, MD, 0, W, G, code)
            if st != 0:
                raise RuntimeError(f"fa_fwd_masked_workspace_size: {fa.fa_status_str(st)}")
            fws = torch.empty(max(fws_bytes, 16), dtype=torch.uint8, device=dev)
            argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), MB,
                    MH, MN, MN, MD, scale, 0, W, G, code, fws.data_ptr(), fws_bytes, sp)
            call = lib.fa_fwd_masked_ws
            args.entry = "fa_fwd_masked_ws"
        ws_bytes = 0
        if bwd:
            from workloads import gen_grad_out

            st = call(*argv)  # the masked forward whose O and L the backward consumes
            if st != 0:
                raise RuntimeError(f"forward failed: {fa.fa_status_str(st)}")
            g = gen_grad_out(MB, MH, MN, MD, seed=2602, dtype="bf16").to(dev)
            dq, dk, dv = (torch.empty(x.shape, dtype=out_dt, device=dev) for x in (q, k, v))
            st, ws_bytes = fa.fa_bwd_masked_workspace_size(MB, MH, MN, MN, MD, MC, W, G, code)
            if st != 0:
                raise RuntimeError(f"fa_bwd_masked_workspace_size failed: "
                                   f"{fa.fa_status_str(st)}")
            bws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    g.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), MB, MH, MN, MN,
                    MD, scale, MC, W, G, code, bws.data_ptr(), ws_bytes, sp)
            call = lib.fa_bwd_masked
            args.entry = "fa_bwd_masked"
    if args.varlen:
        from workloads import varlen_lengths

        if w.H != 1:
            raise SystemExit("--varlen takes a single-head workload")
        lens = varlen_lengths(w.B * w.N, args.varlen, seed=77, min_len=64)
        cu = torch.tensor([0] + [sum(lens[:i + 1]) for i in range(len(lens))],
                          dtype=torch.int32, device=dev)
        T = w.B * w.N
        argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                cu.data_ptr(), cu.data_ptr(), len(lens), 1, T, T, max(lens), w.D, scale,
                int(w.causal), code, sp)
        call = lib.fa_fwd_varlen
        args.entry = "fa_fwd_varlen"
        ws_bytes = 0
        if args.split and not bwd:
            st, ws_bytes = fa.fa_fwd_varlen_workspace_size(len(lens), 1, T, T, max(lens),
                                                           max(lens), w.D, int(w.causal), code)
            if st != 0:
                raise RuntimeError(f"fa_fwd_varlen_workspace_size: {fa.fa_status_str(st)}")
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            argv = argv[:12] + (max(lens),) + argv[12:16] + (ws.data_ptr(), ws_bytes, sp)
            call = lib.fa_fwd_varlen_ws
            args.entry = "fa_fwd_varlen_ws"
    fp8 = None
    if args.fp8:
        from workloads import gen_qkv_fp8

        if bwd or args.varlen or args.masked or w.dtype == "f32":
            raise SystemExit("--fp8 times the forward pass of a 16-bit workload's shape")
        q8, k8, v8, (sq, sk, sv) = gen_qkv_fp8(w.B, w.H, w.N, w.N, w.D, w.seed,
                                               q_mult=w.q_mult)
        q, k, v = q8.to(dev), k8.to(dev), v8.to(dev)
        argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.H,
                w.N, w.N, w.D, scale, sq, sk, sv, int(w.causal), int(out_dt == torch.float32))
        if args.fp8_nows:
            argv = argv + (sp,)
            call = lib.fa_fwd_fp8
            args.entry = "fa_fwd_fp8"
            ws_bytes = 0
        else:
            st, ws_bytes = fa.fa_fwd_fp8_workspace_size(w.B, w.H, w.N, w.N, w.D, int(w.causal),
                                                        int(out_dt == torch.float32))
            if st != 0:
                raise RuntimeError(f"fa_fwd_fp8_workspace_size: {fa.fa_status_str(st)}")
            ws8 = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            argv = argv + (ws8.data_ptr(), ws_bytes, sp)
            call = lib.fa_fwd_fp8_ws
            args.entry = "fa_fwd_fp8_ws"
        fp8 = 1.0 / (0.5 / 5000.0 + 0.5 / PEAK_TFLOPS["bf16"])
    if masked is not None or fp8 is not None:
        pass
    elif bwd and lens is not None:
        from workloads import gen_grad_out

        st = call(*argv)  # the forward pass whose O and L the backward consumes
        if st != 0:
            raise RuntimeError(f"forward failed: {fa.fa_status_str(st)}")
        g = gen_grad_out(w.B, w.H, w.N, w.D, seed=w.seed + 10000, dtype=w.dtype).to(dev)
        bcode = fa._dtype_code(torch, in_dt, out_dt)
        dq, dk, dv = (torch.empty(x.shape, dtype=out_dt, device=dev) for x in (q, k, v))
        ws_bytes = T * 4
        bws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                g.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu.data_ptr(),
                cu.data_ptr(), len(lens), 1, T, T, max(lens), max(lens), w.D, scale,
                int(w.causal), bcode, bws.data_ptr(), ws_bytes, sp)
        call = lib.fa_bwd_varlen
        args.entry = "fa_bwd_varlen"
    elif bwd:
        from workloads import gen_grad_out

        st = call(*argv)  # the forward pass whose O and L the backward consumes
        if st != 0:
            raise RuntimeError(f"forward failed: {fa.fa_status_str(st)}")
        g = gen_grad_out(w.B, w.H, w.N, w.D, seed=w.seed + 10000, dtype=w.dtype).to(dev)
        grad_dt = out_dt
        bcode = fa._dtype_code(torch, in_dt, grad_dt)
        dq = torch.empty(q.shape, dtype=grad_dt, device=dev)
        dk = torch.empty(k.shape, dtype=grad_dt, device=dev)
        dv = torch.empty(v.shape, dtype=grad_dt, device=dev)
        st, ws_bytes = fa.fa_bwd_workspace_size(w.B, w.H, w.N, w.N, w.D, int(w.causal),
                                                bcode)
        if st != 0:
            raise RuntimeError(f"fa_bwd_workspace_size failed: {fa.fa_status_str(st)}")
        bws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                g.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), w.B, w.H, w.N,
                w.N, w.D, scale, int(w.causal), bcode, bws.data_ptr(), ws_bytes, sp)
        call = lib.fa_bwd
        args.entry = "fa_bwd"

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    for _ in range(args.warmup):
        st = call(*argv)
        if st != 0:
            raise RuntimeError(f"{args.entry} failed: {fa.fa_status_str(st)} "
                               f"{fa.fa_last_hip_error()}")
    torch.cuda.synchronize(dev)

    facts = device_facts(torch, dev)
    # events at five evenly spaced points of the timed steps as well (no
    # synchronisation between them) give the spread of the per-step time
    groups = min(5, args.steps)
    marks = sorted({args.steps * g // groups for g in range(groups + 1)})
    evs = {m: torch.cuda.Event(enable_timing=True) for m in marks}
    ev0, ev1 = evs[0], evs[args.steps]
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        call(*argv)
        if i + 1 in evs and i + 1 != args.steps:
            evs[i + 1].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    group_ms = sorted(evs[a].elapsed_time(evs[b]) / (b - a) for a, b in zip(marks, marks[1:]))

    ms_per_step = wall * 1e3 / args.steps
    flops = w.flops() * (2.5 if bwd else 1.0)
    if lens is not None:
        flops = sum(4.0 * n * n * w.D / (2 if w.causal else 1) for n in lens)
        flops *= 2.5 if bwd else 1.0
    if masked is not None:
        flops = 4.0 * masked["shape"][3] * masked["visible_pairs"] * (2.5 if bwd else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    dkey = "f32" if in_dt == torch.float32 else ("bf16" if in_dt == torch.bfloat16 else "f16")
    peak = PEAK_TFLOPS[dkey] if fp8 is None else round(fp8, 1)
    if fp8 is not None:
        dkey = "fp8e4m3+bf16"
    achieved = flops / (kernel_ms * 1e-3) / 1e12

    metric = METRIC if not bwd else METRIC_BWD
    shape = {"B": w.B, "H": w.H, "Nq": w.N, "Nk": w.N, "D": w.D, "causal": w.causal}
    if masked is not None:
        # the masked mode runs its own long-sequence shape, named as such
        MB, MH, MN, MD = masked["shape"]
        cz = "causal" if masked["causal"] else "non-causal"
        tag = f"B{MB} H{MH} N{MN} D{MD} {cz}, window {masked['window']}, " \
              f"{masked['global']} global, visible pairs"
        metric = (f"attention {'bwd' if bwd else 'fwd'} TFLOP/s + % bf16 MFMA peak "
                  f"(masked {tag})")
        name = (f"bf16_b{MB}_h{MH}_n{MN}_d{MD}_{cz.replace('-', '')}_w{masked['window']}"
                f"_g{masked['global']}")
        shape = {"B": MB, "H": MH, "Nq": MN, "Nk": MN, "D": MD, "causal": masked["causal"]}
    line = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dkey,
        "data": "synthetic (seeded i.i.d. Gaussian q, k, v)",
        "config": {"workload": name, **shape, "out": str(out_dt).replace("torch.", ""),
                   "flops_per_step": flops, "entry": args.entry,
                   **({"varlen_lengths": lens} if lens is not None else {}),
                   **({"masked": masked} if masked is not None else {}),
                   "workspace_bytes": ws_bytes},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": None if (bwd or lens is not None or masked is not None or fp8 is not None)
        else measured_traffic(name),
                     "kernel_ms": round(kernel_ms, 5),
                     "group_ms": {"groups": len(group_ms),
                                  "median": round(group_ms[len(group_ms) // 2], 5),
                                  "min": round(group_ms[0], 5), "max": round(group_ms[-1], 5)}},
        "device": facts,
    }
    if w.D <= 64 and not bwd and masked is None:
        # one exp per visible score (half of them when causal): at small head
        # dims the softmax's transcendentals, not the MFMAs, bound the kernel
        exps = w.B * w.H * w.N * w.N / (2 if w.causal else 1)
        rate = exps / (kernel_ms * 1e-3) / 1e12
        line["exp_roofline"] = {"achieved": round(rate, 3), "peak": round(EXP_PEAK_T, 3),
                                "unit": "Texp/s", "frac": round(rate / EXP_PEAK_T, 4)}
    if not args.no_cpu_baseline:
        import numpy as np
        import oracle

        if bwd and (lens is not None or masked is not None or fp8 is not None):
            pass  # the backward's oracle baseline is timed on the dense workload only
        elif lens is not None:
            # each packed sequence through the dense oracle, all of them
            qn, kn, vn = (x.reshape(1, -1, w.D).double().cpu().numpy() for x in (q, k, v))
            cu_h = [0] + [sum(lens[:i + 1]) for i in range(len(lens))]
            t0 = time.perf_counter()
            oracle.attention_varlen(qn, kn, vn, cu_h, cu_h, scale, w.causal)
            el = time.perf_counter() - t0
            line["cpu_baseline"] = {"value": flops / el / 1e12, "unit": "TFLOP/s",
                                    "cores": oracle.threads(), "kind": "oracle",
                                    "sample": "the whole varlen workload, once",
                                    "seconds": round(el, 3)}
        elif masked is not None:
            MB, MH, MN, MD = masked["shape"]
            qn, kn, vn = (x.double().cpu().numpy() for x in (q, k, v))
            W, G = masked["window"], masked["global"]
            per_row = masked_visible(MN, W, G, masked["causal"])
            line["cpu_baseline"] = cpu_baseline_rows(
                lambda r: oracle.attention_masked(qn, kn, vn, scale, masked["causal"], W, G,
                                                  rows=r),
                MB * MH * MN, flops, lambda r: float(per_row[np.asarray(r) % MN].sum()),
                args.cpu_seconds, "masked oracle")
        elif fp8 is not None:
            real = [x.float().cpu().double().numpy() * f for x, f in ((q, sq), (k, sk), (v, sv))]
            ii = lambda r: (np.asarray(r) % w.N) + 1 if w.causal else np.full(len(r), w.N)
            line["cpu_baseline"] = cpu_baseline_rows(
                lambda r: oracle.attention(*real, scale, w.causal, rows=r), w.rows, flops,
                lambda r: float(ii(r).sum()), args.cpu_seconds,
                "dense oracle on the dequantized inputs")
        else:
            line["cpu_baseline"] = (cpu_baseline_bwd(w, args.cpu_seconds) if bwd
                                    else cpu_baseline(w, args.cpu_seconds))
            if not bwd:
                line["cpu_baseline_one_core"] = cpu_baseline_one_core(w)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
