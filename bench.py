#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd over the headline prefill workload (the
32 packed sequences of U[128, 8192] tokens, H=32, d_k=d_v=128, bf16, fp32
initial states, chunk 16) followed by one kda_decode_step over the decode
workload (B=256, H=HV=32, K=V=128, pool of 512 fp32 states, 8 pad rows).
Inputs are generated on the host, copied to HBM, and are resident before any
timed region starts.

Printed: one JSON line.  `value` is the headline prefill's throughput in
Mtok*head/s (token-heads per call / mean device time per call).  Device times
come from HIP events recorded on the stream the kernels run on.  `roofline`
describes the headline prefill's kernel (one launch per call on this
workload) against MI355X's HBM peak, from the workload's algorithmic bytes.
`configs` gives every workload of the set, keyed 0-4: the fp32 tiny prefill (0), the
B=4 T=4096 prefill (1), the headline (2), the T=131072 single-sequence
prefill (3) and the decode step (4), each with its time, throughput, achieved
GB/s and TFLOP/s and their fractions of the HBM and bf16 MFMA peaks.
`cpu_baseline` is the fp64 oracle (plain C, OpenMP over chains) on a bounded
sample of the headline workload, timed on the host cores.  Outside the step,
on the B=4 T=4096 prefill's shapes: the pool-addressed prefill, the materialised form
(kda_chunk_fwd_states, then the chunk-parallel output pass) and kda_backward;
on the decode workload's rows: kda_decode_extend (T = 4) and
kda_conv_decode_step (width 4).  `copy_reference` is a plain device copy of
256 MiB timed the same way: the streaming bandwidth this GPU reaches in
practice, beside the 8 TB/s peak.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
F32_MFMA_PEAK_TFLOPS = 157.3    # dense fp32 MFMA
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = 2                    # key of the prefill workload the headline is quoted on


def prefill_flops_per_tokhead(dk, dv, C=16):
    """State contractions k~S, q~S, k^r U (6 dk dv) + intra-chunk L, Mqk,
    INV u, Mqk U (4 C (dk + dv)) + Neumann inverse (6 x 2 C^3 per chunk)."""
    return 6 * dk * dv + 4 * C * (dk + dv) + 12 * C * C


def prefill_bytes(p):
    """Algorithmic HBM bytes: read q, k, a (dk each), v (dv), b (1); write o
    (dv) per token-head; plus h0 read (if any) and h_T write per chain."""
    elem = 4 if p.dtype == "f32" else 2
    per_tok = elem * (3 * p.dk + p.dv + 1) + elem * p.dv
    state = 4 * p.dv * p.dk * p.n_seq * p.H
    return p.tokens * p.H * per_tok + state * (2 if p.h0 is not None else 1)


def decode_bytes(d):
    """State read + write per live (row, head), plus packed qkv, a, b, o and
    the per-head parameters."""
    live = int((d.state_idx >= 0).sum())
    state = 2 * 4 * d.V * d.K * live * d.HV
    act = 2 * d.B * (2 * d.H * d.K + d.HV * d.V) + 2 * d.B * d.HV * d.K + 2 * d.B * d.HV
    out = 2 * d.B * d.HV * d.V
    par = 4 * d.HV + 4 * d.HV * d.K + 4 * d.B
    return state + act + out + par


def extend_bytes(d, T):
    """decode_bytes with T tokens' activations and outputs per row (the state
    is still read and written once)."""
    live = int((d.state_idx >= 0).sum())
    state = 2 * 4 * d.V * d.K * live * d.HV
    act = T * (2 * d.B * (2 * d.H * d.K + d.HV * d.V) + 2 * d.B * d.HV * d.K + 2 * d.B * d.HV)
    out = T * 2 * d.B * d.HV * d.V
    par = 4 * d.HV + 4 * d.HV * d.K + 4 * d.B
    return state + act + out + par


EXTEND_T = 4
CONV_W = 4


def conv_decode_bytes(d):
    """decode_bytes plus the conv state read and written per live row and the
    conv weights and bias read once."""
    live = int((d.state_idx >= 0).sum())
    D = 2 * d.H * d.K + d.HV * d.V
    return decode_bytes(d) + 2 * 2 * (d.W - 1) * D * live + 2 * D * d.W + 2 * D


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_C = "kimi_delta_attention_kda_amd/csrc/"
_COMMON = [_C + "kda_device.hpp", _C + "kda_launch.hpp", "kimi_delta_attention_kda_amd/build.py"]
_CHUNK = [_C + "kda_chunk.hpp"] + _COMMON
KERNEL_SOURCES = {
    "fwd": [_C + "kda_fwd.hip"] + _CHUNK,
    "prep": [_C + "kda_fwd.hip"] + _CHUNK,
    "rec": [_C + "kda_fwd.hip"] + _CHUNK,
    "decode": [_C + "kda_decode.hip"] + _COMMON,
    "extend": [_C + "kda_decode.hip"] + _COMMON,
    "conv_decode": [_C + "kda_decode.hip"] + _COMMON,
    "backward": [_C + "kda_backward.hip"] + _CHUNK,
    "bwd_rec": [_C + "kda_backward.hip"] + _CHUNK,
    "bwd_prep": [_C + "kda_backward.hip"] + _CHUNK,
    "chunk_o": [_C + "kda_chunk_o.hip"] + _COMMON,
}
# kernel-name patterns of the instantiations the workloads launch: the
# headline's one-pass kernel (many chains), the two passes of the few-chain prefills
# (fewer chains than compute units), the decode family, the backward's three
# passes (chunk-parallel gradients, reverse chain, operands) and the
# chunk-parallel output kernel
KERNEL_MATCH = {"fwd": "kda::fwd_kernel<128, 128, 4, 2, false>", "prep": "kda::prep_kernel<128>",
                "rec": "kda::rec_kernel<128, 128, 2, false>", "decode": "kda::decode_kernel",
                "extend": "kda::extend_kernel", "conv_decode": "kda::conv_decode_kernel",
                "backward": "kda::bwd_chunk_kernel", "bwd_rec": "kda::bwd_rec_kernel",
                "bwd_prep": "kda::bwd_prep_kernel", "chunk_o": "kda::chunk_o_kernel"}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return t.get("bytes_per_launch")


COPY_CALIB_ELEMS = 64 << 20     # float32 elements read and written by the calibration copy


def _counter_rows(d):
    """(kernel name, counter name, value) from every rocprofv3 counter CSV under d."""
    rows = []
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    for r in csv.DictReader(fh):
                        rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def traffic_summary(fetch_dir, write_dir):
    """HBM bytes per launch of each hot kernel from two rocprofv3 --pmc runs of
    `bench.py --copy-calib` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by bytes / counter of the calibration copy (an
    elementwise negate reading and writing COPY_CALIB_ELEMS float32), then the
    per-kernel mean over dispatches is written to profiles/<kernel>_traffic.json
    with the hash of the kernel's sources."""
    import numpy as np
    known = 4.0 * COPY_CALIB_ELEMS
    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r[1] == counter]
        if not rows:
            raise SystemExit(f"no {counter} rows under {d}")
        calib = [v for k, _, v in rows if "neg" in k.lower()]
        if not calib:
            raise SystemExit(f"no calibration copy dispatch in {d}")
        scale = known / (1024.0 * float(np.median(calib)))
        for kern, pat in KERNEL_MATCH.items():
            vals = [v for k, _, v in rows if pat in k]
            if vals:
                out.setdefault(kern, {})[counter] = {"kib_per_dispatch": float(np.mean(vals)),
                                                     "dispatches": len(vals), "scale": scale,
                                                     "bytes": 1024.0 * float(np.mean(vals)) * scale}
    for kern, c in out.items():
        if "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        rec = {"kernel": kern, "source_hash": source_hash(KERNEL_SOURCES[kern]),
               "bytes_per_launch": round(c["FETCH_SIZE"]["bytes"] + c["WRITE_SIZE"]["bytes"]),
               "fetch_bytes": round(c["FETCH_SIZE"]["bytes"]), "write_bytes": round(c["WRITE_SIZE"]["bytes"]),
               "counters": c, "calibration": f"torch.neg over {COPY_CALIB_ELEMS} float32 "
                                              f"({int(known)} B read, {int(known)} B written)"}
        with open(os.path.join(PROFILES, f"{kern}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps({k: rec[k] for k in ("kernel", "bytes_per_launch", "fetch_bytes", "write_bytes")}))


MFMA_COUNTERS = ("MfmaUtil", "MfmaFlopsBF16", "MfmaFlopsF32")


def mfma_summary(pmc_dir):
    """MFMA use of the headline prefill kernel from one rocprofv3 --pmc run with
    the derived counters MfmaUtil (MFMA busy cycles over GPU-active cycles x
    SIMDs, percent) and MfmaFlopsBF16 / MfmaFlopsF32 (MFMA math ops x 512 per
    dispatch): the per-dispatch mean goes to profiles/fwd_mfma.json with the
    hash of the kernel's sources."""
    import numpy as np
    rows = _counter_rows(pmc_dir)
    rec = {"kernel": "fwd", "source_hash": source_hash(KERNEL_SOURCES["fwd"])}
    for c in MFMA_COUNTERS:
        vals = [v for k, n, v in rows if n == c and KERNEL_MATCH["fwd"] in k]
        if not vals:
            raise SystemExit(f"no {c} rows for the prefill kernel under {pmc_dir}")
        rec[c] = {"mean_per_dispatch": float(np.mean(vals)), "dispatches": len(vals)}
    rec["mfma_flops_per_launch"] = rec["MfmaFlopsBF16"]["mean_per_dispatch"] + rec["MfmaFlopsF32"]["mean_per_dispatch"]
    rec["mfma_util_pct"] = rec["MfmaUtil"]["mean_per_dispatch"]
    with open(os.path.join(PROFILES, "fwd_mfma.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({k: rec[k] for k in ("kernel", "mfma_flops_per_launch", "mfma_util_pct")}))


def measured_mfma():
    """(MFMA flops per launch, MFMA busy percent) of the headline prefill kernel
    from the committed counter summary, if taken on the current kernel source."""
    path = os.path.join(PROFILES, "fwd_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(KERNEL_SOURCES["fwd"]):
        return None
    return t["mfma_flops_per_launch"], t["mfma_util_pct"]


def trace_summary(trace_dir, title, command, out_name):
    """profiles/<out_name>.md: the per-kernel table of a rocprofv3 --kernel-trace
    --stats run (its kernel_stats.csv), with the command that made it.  Where the
    run also left its kernel_trace.csv and the command names `--steps N`, a
    column gives each kernel's mean over its last N dispatches: the timed steps
    (warm-up dispatches, run while the GPU's clocks still ramp, excluded)."""
    stats = trace = None
    for root, _, files in os.walk(trace_dir):
        for f in files:
            if f.endswith("kernel_stats.csv"):
                stats = os.path.join(root, f)
            elif f.endswith("kernel_trace.csv"):
                trace = os.path.join(root, f)
    if stats is None:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    with open(stats) as fh:
        rows = list(csv.DictReader(fh))
    m = re.search(r"--steps (\d+)", command)
    last = {}
    if trace is not None and m:
        n = int(m.group(1))
        durs = {}
        with open(trace) as fh:
            for r in csv.DictReader(fh):
                durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        last = {k: sum(v[-n:]) / n for k, v in durs.items() if len(v) >= n}
    head = "| kernel | calls | average ns | min ns | max ns | share of GPU time |"
    rule = "|---|---|---|---|---|---|"
    if last:
        head += f" average ns, last {n} dispatches |"
        rule += "---|"
    lines = [f"# {title}", "", "One MI355X (gfx950), ROCm 7.2, rocprofv3.  Command (from the repository root"
             " on the GPU machine, `$R` = that root):", "", "```", command, "```", "", head, rule]
    for r in rows:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:90]
        line = (f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                f"{float(r['MaxNs']):.0f} | {float(r['Percentage']):.1f} % |")
        if last:
            line += f" {last[r['Name']]:.0f} |" if r["Name"] in last else " |"
        lines.append(line)
    with open(os.path.join(PROFILES, out_name + ".md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(os.path.join(PROFILES, out_name + ".md"))


def copy_reference(dev, reps=20):
    """Device-to-device copy of COPY_CALIB_ELEMS float32 (read + write), timed with
    events on the current stream: the bandwidth a plain streaming kernel reaches on
    this GPU, a second reference beside the 8 TB/s peak."""
    import torch
    x = torch.ones(COPY_CALIB_ELEMS, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del x, y
    return 2 * 4 * COPY_CALIB_ELEMS / t / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def time_calls(fn, reps, torch):
    """Mean seconds per call of fn() over reps back-to-back calls, from two HIP
    events recorded on the current stream before the first call and after the
    last (no marker between the calls, so none adds its own gap)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        fn()
    ev[1].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]) * 1e-3 / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", type=int, default=None, choices=[0, 1, 2, 3],
                    help="time this prefill config only (plus the decode step): for traces and counters")
    ap.add_argument("--profile", action="store_true",
                    help="for counter and trace runs: skip the timings outside the step (pool, states, "
                         "chunk-parallel, backward, extend, conv decode), which launch other kernels or "
                         "other instantiations on other work")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one calibration copy kernel of known size (for --pmc runs)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/<kernel>_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write profiles/fwd_mfma.json from a rocprofv3 --pmc run of "
                         + " ".join(MFMA_COUNTERS) + " and exit")
    ap.add_argument("--trace-summary", nargs=4, metavar=("TRACE_DIR", "TITLE", "COMMAND", "NAME"),
                    help="write profiles/NAME.md from a rocprofv3 --kernel-trace --stats run and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on one GPU only (the path shards by head/sequence with "
              "no exchange between GPUs; a multi-GPU run is not implemented). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kimi_delta_attention_kda_amd as kda
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_t(x, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)

    def bf16(x):
        return dev_t(x, "bf16")

    def prefill_inputs(p):
        B, T = (p.B, p.T) if p.cu_seqlens is None else (1, p.tokens)
        sh = lambda x, d: x.reshape(B, T, p.H, d)
        pin = dict(q=dev_t(sh(p.q, p.dk), p.dtype), k=dev_t(sh(p.k, p.dk), p.dtype), v=dev_t(sh(p.v, p.dv), p.dtype),
                   g_raw=dev_t(sh(p.a, p.dk), p.dtype), beta_raw=dev_t(p.b.reshape(B, T, p.H), p.dtype),
                   A_log=torch.from_numpy(p.A_log).to(dev), dt_bias=torch.from_numpy(p.dt_bias).to(dev),
                   h0=None if p.h0 is None else torch.from_numpy(p.h0).to(dev),
                   cu_seqlens=None if p.cu_seqlens is None else torch.from_numpy(p.cu_seqlens).to(dev))
        act = torch.bfloat16 if p.dtype == "bf16" else torch.float32
        o = torch.empty((B, T, p.H, p.dv), dtype=act, device=dev)
        hT = torch.empty((p.n_seq, p.H, p.dv, p.dk), dtype=torch.float32, device=dev)
        # the default workspace ("auto") for the form the launcher picks, allocated once here
        ws = kda.chunk_fwd_workspace_bytes(B, T, p.H, p.dk, p.dv, p.n_seq, p.cu_seqlens is not None)
        n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
        wst = (torch.empty(ws, dtype=torch.uint8, device=dev)
               if p.dtype == "bf16" and p.n_seq * p.H < n_cu and ws > 0 else None)
        return pin, o, hT, wst

    # ---------------- inputs (host -> HBM, outside the timed regions)
    cfg_ids = [args.only] if args.only is not None else [0, 1, 2, 3]
    head_id = HEADLINE if args.only is None else args.only
    probs, calls = {}, {}
    for i in cfg_ids:
        p = synth.prefill_workload(i)
        pin, o, hT, wst = prefill_inputs(p)
        probs[i] = (p, pin, o, hT, wst)
        calls[i] = (lambda pin=pin, o=o, hT=hT, wst=wst, p=p:
                    kda.chunk_fwd(**pin, scale=p.scale, o=o, h_T=hT, workspace=wst))

    d = synth.decode_workload()
    din = dict(qkv=bf16(d.qkv), a=bf16(d.a), b=bf16(d.b), A_log=torch.from_numpy(d.A_log).to(dev),
               dt_bias=torch.from_numpy(d.dt_bias).to(dev))
    pool = torch.from_numpy(d.pool).to(dev)
    sidx = torch.from_numpy(d.state_idx).to(dev)
    od = torch.empty((d.B, d.HV, d.V), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def decode_call():
        kda.decode_step(**din, state_pool=pool, state_idx=sidx, num_heads=d.H,
                        num_v_heads=d.HV, scale=d.scale, o=od)

    if args.copy_calib:
        xc = torch.ones(COPY_CALIB_ELEMS, dtype=torch.float32, device=dev)
        yc = torch.empty_like(xc)
        torch.neg(xc, out=yc)
        torch.cuda.synchronize()
        del xc, yc

    prefill_call = calls[head_id]
    for _ in range(args.warmup):
        prefill_call()
        decode_call()
    torch.cuda.synchronize()

    # ---------------- timed region: K steps, events on the launch stream.  The K
    # headline prefills run back to back, then the K decode steps (a decode loop, as
    # in serving); each step is one prefill plus one decode step.
    K = args.steps
    evp_ = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evd_ = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    host_dec = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evp_[0].record()
    for s in range(K):
        prefill_call()
        evp_[s + 1].record()
    evd_[0].record()
    for s in range(K):
        th = time.perf_counter()
        decode_call()
        host_dec += time.perf_counter() - th
        evd_[s + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_avg = float(np.mean([evp_[s].elapsed_time(evp_[s + 1]) for s in range(K)])) * 1e-3
    dec_avg = float(np.mean([evd_[s].elapsed_time(evd_[s + 1]) for s in range(K)])) * 1e-3
    slot_err = kda.device_check()   # sticky device error word: must be clear after the timed region
    if slot_err != 0:
        raise SystemExit(f"bench.py: a kernel reported a pool slot out of range ({slot_err})")

    # the same K decode steps recorded in one HIP graph and replayed (how a serving
    # loop issues decode): the per-step time without per-call launch gaps
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        for _ in range(K):
            decode_call()
    dgraph.replay()
    torch.cuda.synchronize()
    evg = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evg[0].record()
    dgraph.replay()
    evg[1].record()
    torch.cuda.synchronize()
    dec_graph_avg = evg[0].elapsed_time(evg[1]) * 1e-3 / K
    del dgraph

    # ---------------- every prefill workload, timed the same way (the headline's own
    # timing is the step's)
    per_cfg = {}
    for i in cfg_ids:
        p = probs[i][0]
        if i == head_id:
            t = pre_avg
        else:
            for _ in range(3):
                calls[i]()
            t = time_calls(calls[i], max(5, min(K, 20)), torch)
        tokheads = p.tokens * p.H
        fl = tokheads * prefill_flops_per_tokhead(p.dk, p.dv)
        by = prefill_bytes(p)
        mfma_peak = BF16_MFMA_PEAK_TFLOPS if p.dtype == "bf16" else F32_MFMA_PEAK_TFLOPS
        two_pass = probs[i][4] is not None
        per_cfg[str(i)] = {
            "workload": p.name, "dtype": p.dtype, "token_heads": tokheads,
            "form": ("two passes (prep_kernel, rec_kernel)" if two_pass else
                     "one pass (fwd_kernel)" if p.dtype == "bf16" else "fp32 kernel (fwd_f32_kernel)"),
            "us": round(t * 1e6, 2), "Mtok_head_s": round(tokheads / t / 1e6, 2),
            "algorithmic_bytes": by, "gbs": round(by / t / 1e9, 1),
            "hbm_frac": round(by / t / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(fl / t / 1e12, 3), "mfma_frac": round(fl / t / 1e12 / mfma_peak, 5),
            "roofline_us": round(by / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}
        assert kda.device_check() == 0
    dbytes = decode_bytes(d)
    dec_gbs = dbytes / dec_graph_avg / 1e9
    per_cfg["4"] = {"workload": d.name, "dtype": "bf16", "us": round(dec_graph_avg * 1e6, 2),
                    "us_eager": round(dec_avg * 1e6, 2), "algorithmic_bytes": dbytes,
                    "gbs": round(dec_gbs, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                    "roofline_us": round(dbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                    "timing": "HIP graph of the K decode steps, per step"}

    # ---------------- outside the step, on the B=4 T=4096 prefill's shapes and the decode workload
    extra = {}
    if not args.profile and 1 in probs:
        p1, pin1, o1, hT1, _ = probs[1]
        # the pool-addressed prefill (states in a pool of 2 N slots, sequence s in slot 2 s)
        ppool = torch.zeros((2 * p1.n_seq, p1.H, p1.dv, p1.dk), dtype=torch.float32, device=dev)
        pidx = torch.arange(0, 2 * p1.n_seq, 2, dtype=torch.int32, device=dev)
        pin_noh0 = {k_: v_ for k_, v_ in pin1.items() if k_ != "h0"}
        pool_call = lambda: kda.chunk_fwd_pool(**pin_noh0, state_pool=ppool, state_idx=pidx, scale=p1.scale, o=o1)
        pool_call()
        extra["prefill_pool_us"] = round(time_calls(pool_call, 10, torch) * 1e6, 2)
        # the materialised form: pass 1 also stores the fp32 state entering every
        # chunk, pass 2 recomputes the outputs with every chunk an independent chain
        nc = kda.n_chunks(p1.T, p1.B)
        hcb = torch.empty((nc, p1.H, p1.dv, p1.dk), dtype=torch.float32, device=dev)
        states_call = lambda: kda.chunk_fwd_states(**pin1, scale=p1.scale, o=o1, h_T=hT1, h_chunks=hcb)
        chunk_o_call = lambda: kda.chunk_o(**pin_noh0, h_chunks=hcb, scale=p1.scale, o=o1)
        route_call = lambda: kda.chunk_o_from_states(**pin_noh0, h_chunks=hcb, scale=p1.scale, o=o1)
        mat = []
        for fn in (states_call, chunk_o_call, route_call):
            fn()
            mat.append(time_calls(fn, 10, torch))
        snap = 4 * nc * p1.H * p1.dv * p1.dk
        act_b = p1.tokens * p1.H * (2 * (3 * p1.dk + p1.dv + 1) + 2 * p1.dv)
        extra.update(states_us=round(mat[0] * 1e6, 2), states_gbs=round((prefill_bytes(p1) + snap) / mat[0] / 1e9, 1),
                     chunk_o_us=round(mat[1] * 1e6, 2), chunk_o_gbs=round((act_b + snap) / mat[1] / 1e9, 1),
                     chunk_o_fwd_route_us=round(mat[2] * 1e6, 2))
        # the backward from those stored states (seeded do, no dh_T)
        do_bits, _ = synth.cotangents(1, p1.tokens, p1.H, p1.dv, p1.dk, p1.n_seq, with_dhT=False)
        dob = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(dev).reshape(o1.shape)
        wsb = torch.empty(kda.backward_workspace_bytes(p1.n_seq, p1.H, p1.tokens), dtype=torch.uint8, device=dev)
        bwd_call = lambda: kda.backward(**pin_noh0, h_chunks=hcb, do=dob, scale=p1.scale, workspace=wsb)
        bwd_call()
        extra["backward_us"] = round(time_calls(bwd_call, 5, torch) * 1e6, 2)
        extra["backward_over_forward"] = round(extra["backward_us"] / per_cfg["1"]["us"], 2)
        # algorithmic bytes: q, k, g_raw, v, beta and do read, the five gradients
        # written (activation dtype), the stored states read once
        bwd_bytes = p1.tokens * p1.H * (4 * (3 * p1.dk + p1.dv + 1) + 2 * p1.dv) + snap
        extra["backward_gbs"] = round(bwd_bytes / (extra["backward_us"] * 1e-6) / 1e9, 1)
        del hcb, wsb, dob, ppool
        # T = 4 tokens per row through kda_decode_extend on the decode workload's rows
        de = synth.extend(4, T=EXTEND_T, **{k_: v_ for k_, v_ in synth.DECODE_WORKLOAD.items() if k_ != "name"})
        dein = dict(qkv=bf16(de.qkv), a=bf16(de.a), b=bf16(de.b), A_log=torch.from_numpy(de.A_log).to(dev),
                    dt_bias=torch.from_numpy(de.dt_bias).to(dev))
        epool = torch.from_numpy(de.pool).to(dev)
        eidx = torch.from_numpy(de.state_idx).to(dev)
        oe = torch.empty((de.B, EXTEND_T, de.HV, de.V), dtype=torch.bfloat16, device=dev)
        ext_call = lambda: kda.decode_extend(**dein, state_pool=epool, state_idx=eidx, num_heads=de.H,
                                             num_v_heads=de.HV, scale=de.scale, o=oe)
        ext_call()
        t_ext = time_calls(ext_call, K, torch)
        extra.update(extend_T=EXTEND_T, extend_us=round(t_ext * 1e6, 2),
                     extend_gbs=round(extend_bytes(de, EXTEND_T) / t_ext / 1e9, 1),
                     extend_hbm_frac=round(extend_bytes(de, EXTEND_T) / t_ext / 1e9 / HBM_PEAK_GBS, 4),
                     extend_traffic=measured_traffic("extend"))
        del epool
        # the short convolution fused with the decode step (width 4)
        dc = synth.conv_decode(4, W=CONV_W, **{k_: v_ for k_, v_ in synth.DECODE_WORKLOAD.items() if k_ != "name"})
        dcin = dict(mixed_qkv=bf16(dc.qkv), conv_state=bf16(dc.conv_state), conv_weight=bf16(dc.conv_weight),
                    conv_bias=bf16(dc.conv_bias), a=bf16(dc.a), b=bf16(dc.b),
                    A_log=torch.from_numpy(dc.A_log).to(dev), dt_bias=torch.from_numpy(dc.dt_bias).to(dev))
        cpool = torch.from_numpy(dc.pool).to(dev)
        cidx = torch.from_numpy(dc.state_idx).to(dev)
        conv_call = lambda: kda.conv_decode_step(**dcin, state_pool=cpool, state_idx=cidx, num_heads=dc.H,
                                                 num_v_heads=dc.HV, scale=dc.scale, o=od)
        conv_call()
        t_conv = time_calls(conv_call, K, torch)
        extra.update(conv_decode_W=CONV_W, conv_decode_us=round(t_conv * 1e6, 2),
                     conv_decode_gbs=round(conv_decode_bytes(dc) / t_conv / 1e9, 1),
                     conv_decode_hbm_frac=round(conv_decode_bytes(dc) / t_conv / 1e9 / HBM_PEAK_GBS, 4),
                     conv_decode_traffic=measured_traffic("conv_decode"))
        del cpool, dcin
        assert kda.device_check() == 0
    copy_gbs = copy_reference(dev)

    # ---------------- CPU baseline: the fp64 oracle on a bounded sample of the headline workload
    ph = probs[head_id][0]
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        heads = [0] if ph.H == 1 else [0, 1]
        nchain = ph.n_seq * len(heads)
        sample = f"heads {heads} of {ph.H}, all {ph.n_seq} sequences ({nchain} chains, {ph.tokens} tokens each head)"
        f = ph.f64(heads)
        # repeated until about 10 s of CPU time have passed (at least once, at most 30 s)
        reps, tc = 0, time.perf_counter()
        while True:
            oracle.fwd(f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], h0=f["h0"],
                       cu_seqlens=f["cu_seqlens"], scale=f["scale"], n_threads=threads)
            reps += 1
            el = time.perf_counter() - tc
            if el >= 10.0 or el * (reps + 1) / reps > 30.0:
                break
        tcpu = el / reps
        th_cnt = f["q"].shape[0] * f["q"].shape[1]
        cpu = {"value": round(th_cnt / tcpu / 1e6, 4), "unit": "Mtok*head/s", "cores": threads,
               "threads": threads, "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"{sample}, run {reps} times", "seconds": round(el, 3)}

    hc = per_cfg[str(head_id)]
    on_profiled = head_id == HEADLINE
    traffic = measured_traffic("fwd") if on_profiled else None
    mfma = measured_mfma() if on_profiled else None
    line = {
        "metric": "KDA chunk-fwd Mtok*head/s (+ % of HBM/MFMA roofline); decode step us at B=256",
        "value": hc["Mtok_head_s"],
        "unit": "Mtok*head/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill: {ph.name}, chunk 16 + decode: {d.name}",
                   "prefill_config": head_id, "prefill_tokens": ph.tokens, "sequences": ph.n_seq,
                   "heads": ph.H, "d_k": ph.dk, "d_v": ph.dv, "decode_rows": d.B, "parallelism": "single GPU"},
        "prefill_us": hc["us"],
        "prefill_tflops": hc["tflops"],
        "prefill_mfma_frac": hc["mfma_frac"],
        "prefill_mfma_counters": (None if mfma is None else
                                  {"mfma_flops_per_launch": mfma[0],
                                   "mfma_tflops": round(mfma[0] / pre_avg / 1e12, 2),
                                   "mfma_busy_pct": round(mfma[1], 2)}),
        "decode_us": round(dec_avg * 1e6, 2),
        "decode_graph_us": round(dec_graph_avg * 1e6, 2),
        "decode_host_us_per_call": round(host_dec / K * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": hc["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": hc["hbm_frac"], "traffic": traffic,
                     "kernel": KERNEL_MATCH["fwd"] if hc["form"].startswith("one pass") else hc["form"],
                     "algorithmic_bytes": hc["algorithmic_bytes"]},
        "roofline_decode": {"bound": "hbm", "timing": "HIP graph of the K decode steps, per step",
                            "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode"),
                            "kernel": "decode_kernel<128,128>", "algorithmic_bytes": dbytes},
        "configs": per_cfg,
        **extra,
        "copy_reference": {"kernel": f"torch copy_ of {4 * COPY_CALIB_ELEMS >> 20} MiB float32",
                           "gbs": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                           "decode_frac_of_copy": round(dec_gbs / copy_gbs, 4),
                           "prefill_frac_of_copy": round(hc["gbs"] / copy_gbs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
