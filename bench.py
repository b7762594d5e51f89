#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one kda_chunk_fwd over the prefill workload (bf16, B=4, H=16,
T=4096, d_k=d_v=128, chunk 16, zero initial state, final states returned)
followed by one kda_decode_step over the decode workload (B=256, H=HV=32,
K=V=128, pool of 512 fp32 states, 8 pad rows).  Inputs are generated on the
host, copied to HBM, and are resident before the timed region starts.

Printed: one JSON line.  `value` is the prefill throughput in Mtok*head/s
(token-heads per step / mean chunk_fwd device time); the decode step time is
reported next to it.  Device times come from HIP events recorded on the
stream the kernels run on.  `roofline` describes the prefill kernel against
MI355X's HBM peak, `roofline_decode` the decode kernel.  `cpu_baseline` is the
fp64 oracle (plain C, OpenMP over chains) timed on the host cores on the same
prefill workload.  Outside the step, the pool-addressed prefill (same
workload) and kda_decode_extend with T = 4 tokens per row (decode workload's
rows, heads and pool) are timed the same way and reported as extra fields,
as is kda_conv_decode_step (width-4 convolution fused with the decode step)
and the two passes of the materialised form on the prefill workload
(kda_chunk_fwd_states, then the chunk-parallel output pass), and
kda_backward from those states.  `copy_reference` is a plain device copy
of 256 MiB timed the same way: the streaming bandwidth this GPU reaches in
practice, beside the 8 TB/s peak.
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def prefill_flops_per_tokhead(dk, dv, C=16):
    """State contractions k~S, q~S, k^r U (6 dk dv) + intra-chunk L, Mqk,
    INV u, Mqk U (4 C (dk + dv)) + Neumann inverse (6 x 2 C^3 per chunk)."""
    return 6 * dk * dv + 4 * C * (dk + dv) + 12 * C * C


def prefill_bytes(p, elem=2):
    """Algorithmic HBM bytes: read q, k, a (dk each), v (dv), b (1); write o
    (dv) per token-head; plus h0 read (if any) and h_T write per chain."""
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


KERNEL_SOURCES = {
    "chunk_fwd": ["kimi_delta_attention_kda_amd/csrc/kda_chunk_fwd.hip",
                  "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
    "decode": ["kimi_delta_attention_kda_amd/csrc/kda_decode.hip",
               "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
    "extend": ["kimi_delta_attention_kda_amd/csrc/kda_decode.hip",
               "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
    "conv_decode": ["kimi_delta_attention_kda_amd/csrc/kda_decode.hip",
                    "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
    "backward": ["kimi_delta_attention_kda_amd/csrc/kda_backward.hip",
                 "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
    "chunk_o": ["kimi_delta_attention_kda_amd/csrc/kda_chunk_o.hip",
                "kimi_delta_attention_kda_amd/csrc/kda_device.hpp"],
}


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
# the prefill workload's instantiation only (the state-storing variant and the
# chunk-parallel pass are other instantiations of the same template)
KERNEL_MATCH = {"chunk_fwd": "kda::chunk_fwd_kernel<true, 128, 128, 32, false>", "decode": "kda::decode_kernel",
                "extend": "kda::extend_kernel", "conv_decode": "kda::conv_decode_kernel",
                "backward": "kda::bwd_kernel", "chunk_o": "kda::chunk_o_kernel"}


def _counter_rows(d):
    """(kernel name, counter name, value) from every rocprofv3 counter CSV under d."""
    import csv
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
    """MFMA use of the prefill kernel from one rocprofv3 --pmc run with the
    derived counters MfmaUtil (MFMA busy cycles over GPU-active cycles x SIMDs,
    percent) and MfmaFlopsBF16 / MfmaFlopsF32 (MFMA math ops x 512 per
    dispatch): the per-dispatch mean goes to profiles/chunk_fwd_mfma.json with
    the hash of the kernel's sources."""
    import numpy as np
    rows = _counter_rows(pmc_dir)
    rec = {"kernel": "chunk_fwd", "source_hash": source_hash(KERNEL_SOURCES["chunk_fwd"])}
    for c in MFMA_COUNTERS:
        vals = [v for k, n, v in rows if n == c and KERNEL_MATCH["chunk_fwd"] in k]
        if not vals:
            raise SystemExit(f"no {c} rows for the prefill kernel under {pmc_dir}")
        rec[c] = {"mean_per_dispatch": float(np.mean(vals)), "dispatches": len(vals)}
    rec["mfma_flops_per_launch"] = rec["MfmaFlopsBF16"]["mean_per_dispatch"] + rec["MfmaFlopsF32"]["mean_per_dispatch"]
    rec["mfma_util_pct"] = rec["MfmaUtil"]["mean_per_dispatch"]
    with open(os.path.join(PROFILES, "chunk_fwd_mfma.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps({k: rec[k] for k in ("kernel", "mfma_flops_per_launch", "mfma_util_pct")}))


def measured_mfma():
    """(MFMA flops per launch, MFMA busy percent) of the prefill kernel from the
    committed counter summary, if taken on the current kernel source."""
    path = os.path.join(PROFILES, "chunk_fwd_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(KERNEL_SOURCES["chunk_fwd"]):
        return None
    return t["mfma_flops_per_launch"], t["mfma_util_pct"]


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--prefill-workload", type=int, default=1, choices=[1, 2, 3])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="for counter and trace runs: skip the pool-addressed prefill and the "
                         "chunk-parallel pass through kda_chunk_fwd, which launch the prefill's "
                         "kernel instantiation on other work and would mix into its per-kernel figures")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one calibration copy kernel of known size (for --pmc runs)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/<kernel>_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write profiles/chunk_fwd_mfma.json from a rocprofv3 --pmc run of "
                         + " ".join(MFMA_COUNTERS) + " and exit")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
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

    def bf16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- inputs (host -> HBM, outside the timed region)
    p = synth.prefill_workload(args.prefill_workload)
    B, T = (p.B, p.T) if p.cu_seqlens is None else (1, p.tokens)
    sh = lambda x, d: x.reshape(B, T, p.H, d)
    pin = dict(q=bf16(sh(p.q, p.dk)), k=bf16(sh(p.k, p.dk)), v=bf16(sh(p.v, p.dv)),
               g_raw=bf16(sh(p.a, p.dk)), beta_raw=bf16(p.b.reshape(B, T, p.H)),
               A_log=torch.from_numpy(p.A_log).to(dev), dt_bias=torch.from_numpy(p.dt_bias).to(dev),
               h0=None if p.h0 is None else torch.from_numpy(p.h0).to(dev),
               cu_seqlens=None if p.cu_seqlens is None else torch.from_numpy(p.cu_seqlens).to(dev))
    o = torch.empty((B, T, p.H, p.dv), dtype=torch.bfloat16, device=dev)
    hT = torch.empty((p.n_seq, p.H, p.dv, p.dk), dtype=torch.float32, device=dev)

    d = synth.decode_workload()
    din = dict(qkv=bf16(d.qkv), a=bf16(d.a), b=bf16(d.b), A_log=torch.from_numpy(d.A_log).to(dev),
               dt_bias=torch.from_numpy(d.dt_bias).to(dev))
    pool = torch.from_numpy(d.pool).to(dev)
    sidx = torch.from_numpy(d.state_idx).to(dev)
    od = torch.empty((d.B, d.HV, d.V), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def prefill_call():
        kda.chunk_fwd(**pin, scale=p.scale, o=o, h_T=hT)

    def decode_call():
        kda.decode_step(**din, state_pool=pool, state_idx=sidx, num_heads=d.H,
                        num_v_heads=d.HV, scale=d.scale, o=od)

    if args.copy_calib:
        xc = torch.ones(COPY_CALIB_ELEMS, dtype=torch.float32, device=dev)
        yc = torch.empty_like(xc)
        torch.neg(xc, out=yc)
        torch.cuda.synchronize()
        del xc, yc

    for _ in range(args.warmup):
        prefill_call()
        decode_call()
    torch.cuda.synchronize()

    # ---------------- timed region: K steps, events on the launch stream.  The K
    # prefills run back to back, then the K decode steps (a decode loop, as in
    # serving); each step is one prefill plus one decode step.
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
    pre_ms = [evp_[s].elapsed_time(evp_[s + 1]) for s in range(K)]
    dec_ms = [evd_[s].elapsed_time(evd_[s + 1]) for s in range(K)]
    pre_avg = float(np.mean(pre_ms)) * 1e-3
    dec_avg = float(np.mean(dec_ms)) * 1e-3

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

    # the pool-addressed prefill on the same workload (states in a pool of 2 N slots,
    # sequence s in slot 2 s), timed the same way outside the step
    ppool = torch.zeros((2 * p.n_seq, p.H, p.dv, p.dk), dtype=torch.float32, device=dev)
    pidx = torch.arange(0, 2 * p.n_seq, 2, dtype=torch.int32, device=dev)
    pin_pool = {k_: v_ for k_, v_ in pin.items() if k_ != "h0"}

    def prefill_pool_call():
        kda.chunk_fwd_pool(**pin_pool, state_pool=ppool, state_idx=pidx, scale=p.scale, o=o)

    pool_avg = None
    if not args.profile:
        for _ in range(2):
            prefill_pool_call()
        evp = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for s_ in range(K):
            evp[s_][0].record()
            prefill_pool_call()
            evp[s_][1].record()
        torch.cuda.synchronize()
        pool_avg = float(np.mean([evp[s_][0].elapsed_time(evp[s_][1]) for s_ in range(K)])) * 1e-3

    # the materialised form on the same prefill workload: pass 1 also stores the
    # fp32 state entering every chunk, pass 2 recomputes the outputs with every
    # chunk an independent chain started from its stored state
    nc = kda.n_chunks(p.T, p.B) if p.cu_seqlens is None else kda.n_chunks(0, 1, pin["cu_seqlens"])
    hcb = torch.empty((nc, p.H, p.dv, p.dk), dtype=torch.float32, device=dev)
    pin_noh0 = {k_: v_ for k_, v_ in pin.items() if k_ != "h0"}

    def states_call():
        kda.chunk_fwd_states(**pin, scale=p.scale, o=o, h_T=hT, h_chunks=hcb)

    def chunk_o_call():
        kda.chunk_o(**pin_noh0, h_chunks=hcb, scale=p.scale, o=o)

    def chunk_o_fwd_route_call():
        kda.chunk_o_from_states(**pin_noh0, h_chunks=hcb, scale=p.scale, o=o)

    mat_avg = []
    for fn in (states_call, chunk_o_call) + (() if args.profile else (chunk_o_fwd_route_call,)):
        for _ in range(2):
            fn()
        evm = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        evm[0].record()
        for s_ in range(K):
            fn()
            evm[s_ + 1].record()
        torch.cuda.synchronize()
        mat_avg.append(float(np.mean([evm[s_].elapsed_time(evm[s_ + 1]) for s_ in range(K)])) * 1e-3)
    snap_bytes = 4 * nc * p.H * p.dv * p.dk
    act_bytes = p.tokens * p.H * (2 * (3 * p.dk + p.dv + 1) + 2 * p.dv)
    states_gbs = (prefill_bytes(p) + snap_bytes) / mat_avg[0] / 1e9
    chunk_o_gbs = (act_bytes + snap_bytes) / mat_avg[1] / 1e9

    # the backward from those stored states (seeded do, no dh_T), timed the same way
    do_bits, _ = synth.cotangents(1, p.tokens, p.H, p.dv, p.dk, p.n_seq, with_dhT=False)
    dob = torch.from_numpy(do_bits.view(np.int16)).view(torch.bfloat16).to(dev).reshape(o.shape)
    wsb = torch.empty(kda.backward_workspace_bytes(p.n_seq, p.H, p.tokens),
                      dtype=torch.uint8, device=dev)

    def backward_call():
        kda.backward(**pin_noh0, h_chunks=hcb, do=dob, scale=p.scale, workspace=wsb)

    backward_call()
    evb = [torch.cuda.Event(enable_timing=True) for _ in range(min(K, 5) + 1)]
    torch.cuda.synchronize()
    evb[0].record()
    for s_ in range(len(evb) - 1):
        backward_call()
        evb[s_ + 1].record()
    torch.cuda.synchronize()
    bwd_avg = float(np.mean([evb[s_].elapsed_time(evb[s_ + 1]) for s_ in range(len(evb) - 1)])) * 1e-3
    del hcb, wsb, dob

    # T = 4 tokens per row through kda_decode_extend (speculative-verify shape) on
    # the decode workload's rows, heads and pool, timed the same way
    de = synth.extend(4, T=EXTEND_T, **{k_: v_ for k_, v_ in synth.DECODE_WORKLOAD.items() if k_ != "name"})
    dein = dict(qkv=bf16(de.qkv), a=bf16(de.a), b=bf16(de.b), A_log=torch.from_numpy(de.A_log).to(dev),
                dt_bias=torch.from_numpy(de.dt_bias).to(dev))
    epool = torch.from_numpy(de.pool).to(dev)
    eidx = torch.from_numpy(de.state_idx).to(dev)
    oe = torch.empty((de.B, EXTEND_T, de.HV, de.V), dtype=torch.bfloat16, device=dev)

    def extend_call():
        kda.decode_extend(**dein, state_pool=epool, state_idx=eidx, num_heads=de.H,
                          num_v_heads=de.HV, scale=de.scale, o=oe)

    for _ in range(2):
        extend_call()
    eve = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    eve[0].record()
    for s_ in range(K):
        extend_call()
        eve[s_ + 1].record()
    torch.cuda.synchronize()
    ext_avg = float(np.mean([eve[s_].elapsed_time(eve[s_ + 1]) for s_ in range(K)])) * 1e-3
    ext_gbs = extend_bytes(de, EXTEND_T) / ext_avg / 1e9
    del epool

    # the short convolution fused with the decode step (width 4) on the decode
    # workload's rows, heads and pool, timed the same way
    dc = synth.conv_decode(4, W=CONV_W, **{k_: v_ for k_, v_ in synth.DECODE_WORKLOAD.items() if k_ != "name"})
    dcin = dict(mixed_qkv=bf16(dc.qkv), conv_state=bf16(dc.conv_state), conv_weight=bf16(dc.conv_weight),
                conv_bias=bf16(dc.conv_bias), a=bf16(dc.a), b=bf16(dc.b),
                A_log=torch.from_numpy(dc.A_log).to(dev), dt_bias=torch.from_numpy(dc.dt_bias).to(dev))
    cpool = torch.from_numpy(dc.pool).to(dev)
    cidx = torch.from_numpy(dc.state_idx).to(dev)

    def conv_decode_call():
        kda.conv_decode_step(**dcin, state_pool=cpool, state_idx=cidx, num_heads=dc.H,
                             num_v_heads=dc.HV, scale=dc.scale, o=od)

    for _ in range(2):
        conv_decode_call()
    evc = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evc[0].record()
    for s_ in range(K):
        conv_decode_call()
        evc[s_ + 1].record()
    torch.cuda.synchronize()
    conv_avg = float(np.mean([evc[s_].elapsed_time(evc[s_ + 1]) for s_ in range(K)])) * 1e-3
    conv_gbs = conv_decode_bytes(dc) / conv_avg / 1e9
    del cpool, dcin

    tokheads = p.tokens * p.H
    flops = tokheads * prefill_flops_per_tokhead(p.dk, p.dv)
    pbytes = prefill_bytes(p)
    dbytes = decode_bytes(d)
    value = tokheads / pre_avg / 1e6
    pre_gbs = pbytes / pre_avg / 1e9
    dec_gbs = dbytes / dec_graph_avg / 1e9
    copy_gbs = copy_reference(dev)

    # ---------------- CPU baseline: fp64 oracle on the same prefill workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        if args.prefill_workload == 1:
            heads, sample = None, "whole prefill workload (64 chains x 4096 tokens)"
        else:
            heads, sample = [0, 1], "2 of the workload's heads, all sequences"
        f = p.f64(heads)
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
        cpu = {"value": th_cnt / tcpu / 1e6, "unit": "Mtok*head/s", "cores": threads,
               "kind": "oracle", "sample": f"{sample}, run {reps} times", "seconds": round(el, 3)}

    # the committed counter summaries were taken on the default prefill workload
    on_profiled = args.prefill_workload == 1
    traffic = measured_traffic("chunk_fwd") if on_profiled else None
    traffic_d = measured_traffic("decode")
    mfma = measured_mfma() if on_profiled else None
    line = {
        "metric": "KDA chunk-fwd Mtok*head/s (+ % of HBM/MFMA roofline); decode step us at B=256",
        "value": round(value, 2),
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
        "config": {"workload": f"prefill: {p.name}, chunk 16 + decode: {d.name}",
                   "prefill_tokens": p.tokens, "heads": p.H, "d_k": p.dk, "d_v": p.dv,
                   "decode_rows": d.B, "parallelism": "single GPU"},
        "prefill_us": round(pre_avg * 1e6, 2),
        "prefill_tflops": round(flops / pre_avg / 1e12, 2),
        "prefill_mfma_frac": round(flops / pre_avg / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
        # counter evidence (rocprofv3 MfmaFlops*, MfmaUtil) when taken on the current source
        "prefill_mfma_counters": (None if mfma is None else
                                  {"mfma_flops_per_launch": mfma[0],
                                   "mfma_tflops": round(mfma[0] / pre_avg / 1e12, 2),
                                   "mfma_busy_pct": round(mfma[1], 2)}),
        "prefill_pool_us": None if pool_avg is None else round(pool_avg * 1e6, 2),
        "states_us": round(mat_avg[0] * 1e6, 2),
        "states_gbs": round(states_gbs, 1),
        "chunk_o_us": round(mat_avg[1] * 1e6, 2),
        "chunk_o_gbs": round(chunk_o_gbs, 1),
        "chunk_o_fwd_route_us": round(mat_avg[2] * 1e6, 2) if len(mat_avg) > 2 else None,
        "backward_us": round(bwd_avg * 1e6, 2),
        "decode_us": round(dec_avg * 1e6, 2),
        "decode_graph_us": round(dec_graph_avg * 1e6, 2),
        "decode_host_us_per_call": round(host_dec / K * 1e6, 2),
        "extend_T": EXTEND_T,
        "extend_us": round(ext_avg * 1e6, 2),
        "extend_gbs": round(ext_gbs, 1),
        "extend_hbm_frac": round(ext_gbs / HBM_PEAK_GBS, 4),
        "extend_traffic": measured_traffic("extend"),
        "conv_decode_W": CONV_W,
        "conv_decode_us": round(conv_avg * 1e6, 2),
        "conv_decode_gbs": round(conv_gbs, 1),
        "conv_decode_hbm_frac": round(conv_gbs / HBM_PEAK_GBS, 4),
        "conv_decode_traffic": measured_traffic("conv_decode"),
        "roofline": {"bound": "hbm", "achieved": round(pre_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(pre_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "chunk_fwd_kernel<bf16,128,128>",
                     "algorithmic_bytes": pbytes},
        "roofline_decode": {"bound": "hbm", "timing": "HIP graph of the K decode steps, per step",
                            "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                            "traffic": traffic_d, "kernel": "decode_kernel<128,128>",
                            "algorithmic_bytes": dbytes},
        "copy_reference": {"kernel": f"torch copy_ of {4 * COPY_CALIB_ELEMS >> 20} MiB float32",
                           "gbs": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                           "decode_frac_of_copy": round(dec_gbs / copy_gbs, 4),
                           "prefill_frac_of_copy": round(pre_gbs / copy_gbs, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
