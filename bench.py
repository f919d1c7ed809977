"""Throughput of the causal context-parallel attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: the ring
forward of every virtual rank r = 0..cp-1 of the workload, one after another,
with every K/V shard already resident in HBM (index maps are built once, in
set-up).  ``value`` is the algorithmic work of those passes (4*d*Hq per
unmasked (query, key) pair, exact pair counts from the index builder) divided
by the time of the timed steps, in TFLOP/s: the time-weighted mean throughput
of one virtual rank.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one
GPU and every figure is that GPU's.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal ring-attention TFLOP/s per virtual rank (fwd, fwd+bwd); % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {"fwd": ["context_causal_attention_amd/csrc/attn_fwd.hip"]}


def source_hash(paths):
    """sha256 over the kernel sources, to tell whether stored counters still
    describe the kernel being timed."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kind, workload):
    """HBM bytes per launch from the committed counter summary
    profiles/<kind>_traffic_<workload>.txt (lines 'key: value'), or None when
    the summary is missing or was taken on a different kernel source."""
    path = os.path.join(PROFILES, f"{kind}_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kind]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_s128k_cp8")
    ap.add_argument("--ranks", default="all", help="'all' or a comma list of virtual ranks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the cpu_baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (the reference for HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, three times: its FETCH_SIZE and
    WRITE_SIZE counter readings against the known 1 GiB give the scale for the
    attention kernel's HBM traffic counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "repeats": 3}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is one GPU's share; "
              "see DESIGN.md for how it would shard.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import context_causal_attention_amd as cpa
    import seeded_inputs as si

    w = si.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    t0 = time.time()
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    q, k, v = full
    cu = si.cu_seqlens_from_lengths(si.doc_lengths(total=w.S, seed=w.seed)) if w.varlen else None
    ranks = list(range(w.cp)) if args.ranks == "all" else [int(x) for x in args.ranks.split(",")]

    if cu is None:
        allp = cpa.cp_unshard_zigzag(w.S, w.cp)
        idx = {r: (cpa.cp_shard_zigzag(w.S, w.cp, r), None) for r in ranks}
    else:
        allp = np.concatenate([cpa.cp_varlen_index(cu, w.cp, r)[0] for r in range(w.cp)])
        idx = {r: cpa.cp_varlen_index(cu, w.cp, r) for r in ranks}
    ai = torch.from_numpy(allp.astype(np.int64))
    k_all = k.index_select(2, ai).to(dev)
    v_all = v.index_select(2, ai).to(dev)
    plans, flops = {}, {}
    for r in ranks:
        pos, lo = idx[r]
        q_loc = q.index_select(2, torch.from_numpy(pos.astype(np.int64))).to(dev)
        plans[r] = cpa.RingFwdPlan(q_loc, k_all, v_all, w.cp, r, pos, lo, allp, scale=w.scale)
        flops[r] = 4.0 * w.d * w.Hq * w.B * cpa.cp_pairs(pos, lo, allp)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] set-up {setup_s:.1f}s: {w.name} ranks {ranks}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        for r in ranks:
            if events is not None:
                events[r][0].record(stream)
            plans[r].run()
            if events is not None:
                events[r][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [{r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in ranks}
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    per_rank_ms = {r: float(np.mean([ev[s][r][0].elapsed_time(ev[s][r][1]) for s in range(args.steps)]))
                   for r in ranks}
    step_flops = sum(flops.values())
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (wall / args.steps) / 1e12
    launch_ms = float(np.mean(list(per_rank_ms.values())))
    launch_flops = step_flops / len(ranks)
    achieved = launch_flops / (launch_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    print(f"[bench] per-rank ms: " + ", ".join(f"{r}:{per_rank_ms[r]:.3f}" for r in ranks), file=sys.stderr,
          flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, full, idx[ranks[0]], allp, cu, args.cpu_seconds, ranks[0])

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "fwd", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "S": w.S,
                   "cp": w.cp, "ranks": ranks, "varlen": w.varlen,
                   "step": "ring forward of each listed virtual rank, sequential, K/V resident"},
        "pct_peak": round(100 * value / peak, 2),
        "per_rank_ms": {str(r): round(x, 4) for r, x in per_rank_ms.items()},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": stored_traffic("fwd", w.name),
                     "kernel": "cp_attn_ring_fwd launch (V-transpose prep + fwd_bf16_kernel), HIP events "
                               "on the launch stream; traffic = calibrated FETCH_SIZE + WRITE_SIZE per launch"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, full, idx_r, allp, cu, target_s, rank_id):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    one virtual rank's rows for as many query heads as fit in ~target_s."""
    import numpy as np
    import oracle as orc
    import context_causal_attention_amd as cpa

    pos, lo = idx_r
    q, k, v = full
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:
        cores = len(os.sched_getaffinity(0))
    g = w.Hq // w.Hkv
    pairs = cpa.cp_pairs(pos, lo, allp)
    t0 = time.perf_counter()
    done = 0
    while done < w.Hq:
        h = done
        qh = q[:, h:h + 1].double().numpy()
        kh = k[:, h // g:h // g + 1].double().numpy()
        vh = v[:, h // g:h // g + 1].double().numpy()
        orc.attention_fwd(qh, kh, vh, w.scale, cu_seqlens=cu, rows=pos)
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    fl = 4.0 * w.d * done * pairs
    return {"value": round(fl / el / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{w.name}: the rows of virtual rank {rank_id}, {done} of {w.Hq} query heads, "
                      f"fp64 numpy, {el:.1f}s"}


if __name__ == "__main__":
    main()
