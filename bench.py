"""Throughput of the causal context-parallel attention hot path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input, for every
virtual rank r = 0..cp-1 of the workload, one after another, with every K/V
shard already resident in HBM (index maps are built once, in set-up):
  --pass fwdbwd (default): zero the fp32 gradient buffers, then per rank the
      ring forward (final O, LSE), delta = rowsum(dO * O) and the ring backward
      (dQ of the rank's rows, dK/dV of every shard accumulated in place);
  --pass fwd: the ring forward of each rank only;
  --pass rotate: the ring forward of each rank as separate steps (a partial
      forward per step, merged into the running output in its epilogue,
      cp_attn_ring_fwd_stepwise), four ways: the
      fused resident ring, steps reading the shards in place, steps whose
      shards are copied into a two-slot stage on a second stream (a rotation
      ring's receive, overlapped), and the same copies on the compute stream.
      ``value`` is the staged, overlapped rate; ``rotate`` gives all four,
      the copies alone, and one LSE merge (cp_attn_merge) of a rank-sized
      fp32 partial alone with its HBM rate;
  --pass a2a: the head exchange layout calls of hierarchical CP's all-to-all
      level (cp_a2a_pack, cp_a2a_unpack and their inverses) on one rank's
      shard of the workload's queries ([S/cp, Hq, d]), for a2a group sizes
      --a2a-groups; ``value`` is their HBM rate in GB/s (bytes read + written).
``value`` is the algorithmic work of a step divided by the time of the timed
steps, in TFLOP/s, with exact pair counts from the index builder: 4*d*Hq flops
per allowed (query, key) pair for the forward (Q K^T and P V) and 8*d*Hq for
the backward (dO V^T, P^T dO, dS K and dS^T Q), twice the forward, as in the
per-token cost of attention the Accelerate context-parallel guide quotes
(12 H d per token for forward plus backward).  The rate that also counts the
backward's recomputed Q K^T (10*d*Hq, 14*d*Hq for forward plus backward) is
reported beside it, and so is the rate of the MFMA work the kernels execute.
The clocks sampled during the timed steps give the peak at the measured sclk.
With the backward, ``delta_alone`` times cp_attn_bwd_delta on the first rank's
(dO, O) after the timed steps, launched back to back, with its HBM rate.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: the bench measures one
GPU's share of the ring and every figure is that GPU's.
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
KERNEL_SOURCES = {
    "fwd": ["context_causal_attention_amd/csrc/attn_fwd.hip", "context_causal_attention_amd/csrc/device_common.h"],
    "bwd": ["context_causal_attention_amd/csrc/attn_bwd.hip", "context_causal_attention_amd/csrc/device_common.h"],
    "a2a": ["context_causal_attention_amd/csrc/a2a.hip", "context_causal_attention_amd/csrc/device_common.h"],
}
FLOPS_PER_PAIR_HEAD_DIM = {"fwd": 4.0, "bwd": 8.0}
# The backward with its recomputed Q K^T counted, and what the kernels execute:
# the forward kernel 4*d; the dK/dV kernel S, dP, dV, dK (8*d) and the dQ
# kernel S, dP, dQ (6*d).
FLOPS_RECOMPUTE_COUNTED = {"fwd": 4.0, "bwd": 10.0}
FLOPS_EXECUTED = {"fwd": 4.0, "bwd": 14.0}
MFMA_FLOP_PER_CLK = 256 * 4096  # CUs x dense bf16 flop per CU per clock


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
    ap.add_argument("--pass", dest="mode", choices=["fwd", "fwdbwd", "rotate", "a2a", "probe"], default="fwdbwd")
    ap.add_argument("--a2a-groups", default="2,8", help="--pass a2a: comma list of all-to-all group sizes")
    ap.add_argument("--varlen-mode", choices=["stream", "per_doc", "whole_doc"], default="stream",
                    help="how a varlen workload's packed stream is dealt to ranks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the cpu_baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (the reference for HBM byte counters) and exit")
    return ap.parse_args()


class ClockSampler:
    """Samples the GPU's current sclk and mclk (MHz) from sysfs (the level the
    power-play tables mark as current) every `period` seconds on a host thread
    while the timed steps run.  Reports None where the files are missing."""

    def __init__(self, period=0.05):
        import glob
        import threading
        self.period = period
        self.samples = {"sclk": [], "mclk": []}
        self.files = {}
        for kind in ("sclk", "mclk"):
            for f in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}")):
                if self._read(f) is not None:
                    self.files[kind] = f
                    break
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        import re
        try:
            with open(path) as fh:
                for line in fh:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for kind, f in self.files.items():
                v = self._read(f)
                if v is not None:
                    self.samples[kind].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        import numpy as np
        out = {}
        for kind, vals in self.samples.items():
            out[kind + "_mhz"] = (None if not vals else
                                  {"median": float(np.median(vals)), "min": min(vals), "max": max(vals)})
        out["samples"] = len(self.samples["sclk"])
        out["source"] = ", ".join(self.files.values()) or None
        return out


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


PROBES = {
    0: ("mfma", "v_mfma_f32_32x32x16_bf16, 4 independent accumulators per wave"),
    5: ("mfma_chain", "v_mfma_f32_32x32x16_bf16, one dependent accumulator chain per wave"),
    1: ("exp", "v_exp_f32, 8 independent chains per lane"),
    2: ("fma", "v_fma_f32, 8 independent chains per lane"),
    3: ("mix_same_wave", "per MFMA: 2 FMA + 2 exp + 1 bf16 pack + 2 add, all in every wave"),
    4: ("mix_split_waves", "the same work, MFMAs in waves 0-3 and the vector part in waves 4-7"),
    8: ("mfma_agpr", "as mfma, accumulators in AGPRs"),
    6: ("mix_same_wave_agpr", "as mix_same_wave, MFMA accumulators in AGPRs"),
    7: ("mix_split_waves_agpr", "as mix_split_waves, MFMA accumulators in AGPRs"),
    9: ("mix_same_wave_2mfma", "as mix_same_wave with two MFMAs per step (the forward's ratio)"),
    10: ("mfma_lds", "as mfma with each MFMA's A operand read from LDS (1 KB a wave, four steps ahead)"),
    11: ("mix_same_wave_lds", "as mix_same_wave with the MFMA operand read from LDS (the forward's score phase)"),
    12: ("mix_same_wave_2mfma_lds", "as mix_same_wave_2mfma with both MFMA operands read from LDS"),
    13: ("mix_same_wave_lds_noexp", "as mix_same_wave_lds with each exponential replaced by an FMA"),
    14: ("mix_same_wave_lds_2step", "as mix_same_wave_lds with two steps between scheduling barriers"),
}


def dq_atomics_probe(L, args, np, torch):
    """The dQ reduction traffic a single-pass backward would add on the
    131072-token cp = 8 workload (rank 0): every (256-key dK/dV workgroup,
    query head, 64-row query tile) pair with allowed keys adds a 64 x 128 fp32
    block into dQ with float atomics, in the dK/dV kernel's grid and order
    (cp_probe_dq_atomics)."""
    import ctypes
    import context_causal_attention_amd as cpa
    S, cp, hkv, g, d = 131072, 8, 8, 4, 128
    R = S // cp
    qp = cpa.cp_shard_zigzag(S, cp, 0).astype(np.int32)
    kp = cpa.cp_unshard_zigzag(S, cp).astype(np.int32)
    # allowed (key block, query tile) pairs: a query at or after the block's first key
    kmin = kp.reshape(-1, 256).min(1)
    qmax = qp.reshape(-1, 64).max(1)
    pairs = int((qmax[None, :] >= kmin[:, None]).sum()) * hkv * g
    nbytes = pairs * 64 * d * 4
    dev = torch.device("cuda:0")
    qd, kd = torch.from_numpy(qp).to(dev), torch.from_numpy(kp).to(dev)
    dq = torch.zeros(hkv * g * R * d, dtype=torch.float32, device=dev)
    L.cp_probe_dq_atomics.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = L.cp_probe_dq_atomics(ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kd.data_ptr()),
                                   ctypes.c_void_p(dq.data_ptr()), R, R, cp, hkv, g, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"dq atomics probe: hip error {rc}")
    launch()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(3, args.steps)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(); launch(); b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.median(times))
    r = {"what": "fp32 atomic adds of the dQ partials of a single-pass backward, 131072 tokens, cp = 8, rank 0, "
                 "in the dK/dV grid and order", "ms": round(ms, 3), "block_pairs": pairs,
         "atomic_GB": round(nbytes / 1e9, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    print(f"[probe] dq_atomics: {r}", file=sys.stderr, flush=True)
    return r


def probe_bench(args):
    """Unit throughput of one MI355X under the attention kernels' occupancy
    (one 8-wave workgroup per CU, two waves per SIMD), from the probe kernels
    of libcpattn_probe.so: sustained bf16 MFMA rate, exp and FMA issue rates,
    and the forward's MFMA + exponential mix with the two kinds of work in the
    same waves or in different waves of each SIMD.  The clock each probe ran
    at is its workgroups' shader clock cycles (s_memtime readings at the start
    and end of each workgroup, median over workgroups) over the kernel's
    duration; cycles per unit are counted at that clock."""
    import ctypes
    import numpy as np
    import torch
    from context_causal_attention_amd import build as cpb
    if not os.path.exists(cpb.PROBE_LIB):
        raise RuntimeError(f"{cpb.PROBE_LIB} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(cpb.PROBE_LIB)
    L.cp_probe_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p]
    blocks = 256
    out = torch.empty(blocks * 512, device="cuda:0")
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    # iterations per launch, sized for ~20-60 ms per launch
    iters = {0: 20000, 5: 20000, 8: 20000, 1: 100000, 2: 100000, 3: 40000, 4: 40000, 6: 40000, 7: 40000, 9: 40000,
             10: 40000, 11: 40000, 12: 40000, 13: 40000, 14: 40000}
    res = {}
    for kind, (name, what) in PROBES.items():
        def launch():
            rc = L.cp_probe_run(kind, blocks, iters[kind], ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(clk.data_ptr()), ctypes.c_void_p(stream))
            if rc != 0:
                raise RuntimeError(f"probe {name}: hip error {rc}")
        launch()
        torch.cuda.synchronize()
        times, mhzs = [], []
        for _ in range(max(3, args.steps)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(); launch(); b.record()
            b.synchronize()
            dt = a.elapsed_time(b) / 1e3
            c = clk.view(blocks, 2).cpu().numpy()
            times.append(dt)
            mhzs.append(float(np.median(c[:, 1] - c[:, 0])) / dt / 1e6)
        t = float(np.median(times))
        mhz = round(float(np.median(mhzs)), 1)
        it = iters[kind]
        per_simd = {}
        if kind in (0, 5, 8):
            n = 2 * it * 4 if kind == 5 else 2 * it * 16           # MFMAs per SIMD
            flop = blocks * 8 * (it * (4 if kind == 5 else 16)) * 32768
            per_simd = {"mfma_per_simd": n, "TFLOP/s": round(flop / t / 1e12, 1),
                        "pct_of_2516.6": round(100 * flop / t / 1e12 / PEAK_BF16_TFLOPS, 1)}
            unit = n
        elif kind in (1, 2):
            unit = 2 * it * 32                                      # wave64 instructions per SIMD
            per_simd = {"instructions_per_simd": unit}
        elif kind >= 10:
            per_it = 16 if kind == 12 else 8                         # MFMAs per wave per iteration
            unit = 2 * it * per_it                                  # MFMAs per SIMD
            flop = blocks * 8 * it * per_it * 32768
            per_simd = {"mfma_per_simd": unit, "TFLOP/s": round(flop / t / 1e12, 1),
                        "pct_of_2516.6": round(100 * flop / t / 1e12 / PEAK_BF16_TFLOPS, 1)}
        elif kind == 9:
            unit = 2 * it * 8                                       # steps (two MFMAs each) per SIMD
            flop = blocks * 8 * it * 8 * 2 * 32768
            per_simd = {"mfma_steps_per_simd": unit, "TFLOP/s": round(flop / t / 1e12, 1)}
        else:
            same = kind in (3, 6)
            unit = 2 * it * 8 if same else it * 8                   # MFMA steps per SIMD
            flop = blocks * (8 if same else 4) * it * 8 * 32768
            per_simd = {"mfma_steps_per_simd": unit, "TFLOP/s": round(flop / t / 1e12, 1)}
        r = {"what": what, "ms": round(t * 1e3, 3), **per_simd, "sclk_mhz": mhz}
        if mhz:
            r["cycles_per_unit"] = round(t * mhz * 1e6 / unit, 2)
        res[name] = r
        print(f"[probe] {name}: {r}", file=sys.stderr, flush=True)
    res["dq_atomics"] = dq_atomics_probe(L, args, np, torch)
    line = {"metric": "unit throughput probes (one 8-wave workgroup per CU)", "value": res["mfma"]["TFLOP/s"],
            "unit": "TFLOP/s (sustained bf16 MFMA)", "n_gpus": 1, "steps": max(3, args.steps), "warmup": 1,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic", "config": {"workload": "probe"},
            "probes": res}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the path is one GPU's share; "
              "the multi-GPU sharding is a design, not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import context_causal_attention_amd as cpa
    import seeded_inputs as si

    if args.mode == "probe":
        probe_bench(args)
        return
    w = si.WORKLOADS[args.workload]
    if args.mode == "rotate":
        rotate_bench(args, w)
        return
    if args.mode == "a2a":
        a2a_bench(args, w)
        return
    bwd = args.mode == "fwdbwd"
    if bwd and w.dtype != "bf16":
        print(f"the backward takes bf16 inputs; {w.name} is {w.dtype} (use --pass fwd)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    t0 = time.time()
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed, with_dout=bwd)
    q, k, v = full[:3]
    cu = si.workload_cu_seqlens(w)
    ranks = list(range(w.cp)) if args.ranks == "all" else [int(x) for x in args.ranks.split(",")]

    balance = None
    if cu is None:
        allp = cpa.cp_unshard_zigzag(w.S, w.cp)
        idx = {r: (cpa.cp_shard_zigzag(w.S, w.cp, r), None) for r in ranks}
    else:
        vmode = {"stream": cpa.CP_STREAM, "per_doc": cpa.CP_PER_DOC, "whole_doc": cpa.CP_WHOLE_DOC}[args.varlen_mode]
        every = [cpa.cp_varlen_index(cu, w.cp, r, vmode) for r in range(w.cp)]
        allp = np.concatenate([e[0] for e in every])
        idx = {r: every[r] for r in ranks}
        # Causal work per rank under this deal: exact unmasked pairs per head.
        rp = [cpa.cp_pairs(e[0], e[1], allp) for e in every]
        balance = {"deal": args.varlen_mode, "pairs_per_rank": rp,
                   "max_over_mean": round(max(rp) / (sum(rp) / len(rp)), 4)}
    ai = torch.from_numpy(allp.astype(np.int64))
    k_all = k.index_select(2, ai).to(dev)
    v_all = v.index_select(2, ai).to(dev)
    passes = ["fwd", "bwd"] if bwd else ["fwd"]
    fplans, bplans, deltas, pairs = {}, {}, {}, {}
    dk_all = torch.zeros(k_all.shape, dtype=torch.float32, device=dev) if bwd else None
    dv_all = torch.zeros(v_all.shape, dtype=torch.float32, device=dev) if bwd else None
    for r in ranks:
        pos, lo = idx[r]
        pi = torch.from_numpy(pos.astype(np.int64))
        q_loc = q.index_select(2, pi).to(dev)
        fplans[r] = cpa.RingFwdPlan(q_loc, k_all, v_all, w.cp, r, pos, lo, allp, scale=w.scale)
        pairs[r] = cpa.cp_pairs(pos, lo, allp)
        if bwd:
            do_loc = full[3].index_select(2, pi).to(dev)
            deltas[r] = (do_loc, torch.empty(fplans[r].lse.shape, dtype=torch.float32, device=dev))
            bplans[r] = cpa.RingBwdPlan(q_loc, k_all, v_all, do_loc, fplans[r].lse, deltas[r][1], w.cp, r, pos, lo,
                                        allp, scale=w.scale, dk=dk_all, dv=dv_all)
    flops = {ps: {r: FLOPS_PER_PAIR_HEAD_DIM[ps] * w.d * w.Hq * w.B * pairs[r] for r in ranks} for ps in passes}
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] set-up {setup_s:.1f}s: {w.name} ranks {ranks} pass {args.mode}", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(events=None):
        if bwd:
            dk_all.zero_()
            dv_all.zero_()
        for r in ranks:
            if events is not None:
                events["fwd"][r][0].record(stream)
            o, _ = fplans[r].run()
            if events is not None:
                events["fwd"][r][1].record(stream)
            if bwd:
                bplans[r].dq.zero_()
                cpa.cp_attn_bwd_delta(deltas[r][0], o, deltas[r][1])
                if events is not None:
                    events["bwd"][r][0].record(stream)
                bplans[r].run()
                if events is not None:
                    events["bwd"][r][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [{ps: {r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in ranks}
           for ps in passes} for _ in range(args.steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t_start = time.perf_counter()
        for s in range(args.steps):
            step(ev[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
    clocks = clk.summary()

    every_ms = {ps: {r: [ev[s][ps][r][0].elapsed_time(ev[s][ps][r][1]) for s in range(args.steps)] for r in ranks}
                for ps in passes}
    launch_ms = {ps: {r: float(np.mean(every_ms[ps][r])) for r in ranks} for ps in passes}
    step_flops = sum(sum(f.values()) for f in flops.values())
    ms_per_step = wall * 1e3 / args.steps
    value = step_flops / (wall / args.steps) / 1e12
    recount = sum(FLOPS_RECOMPUTE_COUNTED[ps] / FLOPS_PER_PAIR_HEAD_DIM[ps] * sum(flops[ps].values()) for ps in passes)
    value_recompute = recount / (wall / args.steps) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    sclk = clocks["sclk_mhz"]["median"] if clocks.get("sclk_mhz") else None
    peak_at_sclk = MFMA_FLOP_PER_CLK * sclk * 1e6 / 1e12 if (sclk and w.dtype == "bf16") else None
    for ps in passes:
        print(f"[bench] {ps} per-rank ms: " + ", ".join(f"{r}:{launch_ms[ps][r]:.3f}" for r in ranks),
              file=sys.stderr, flush=True)

    def roof(ps):
        ms = float(np.mean(list(launch_ms[ps].values())))
        fl = sum(flops[ps].values()) / len(ranks)
        ach = fl / (ms * 1e-3) / 1e12
        kern = {"fwd": "cp_attn_ring_fwd launch (prep_kernel: bounds, and V^T on dense rings of 65536 keys or more; "
                       "under document masks order_cost_kernel and order_sort_kernel; fwd_bf16_kernel)",
                "bwd": "cp_attn_ring_bwd launch (key_prep_kernel, query_prep_kernel; on short or document-masked rings "
                       "the dispatch-order kernels; dkdv_kernel, dq_kernel)"}[ps]
        r = {"bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
             "frac": round(ach / peak, 4), "traffic": stored_traffic(ps, w.name), "launch_ms": round(ms, 4)}
        if ps == "bwd":
            r["achieved_recompute_counted"] = round(ach * FLOPS_RECOMPUTE_COUNTED[ps] / FLOPS_PER_PAIR_HEAD_DIM[ps], 3)
        r["executed_mfma"] = round(ach * FLOPS_EXECUTED[ps] / FLOPS_PER_PAIR_HEAD_DIM[ps], 3)
        if peak_at_sclk:
            r["frac_at_measured_sclk"] = round(ach / peak_at_sclk, 4)
        r["kernel"] = (kern + f"; achieved = algorithmic flops per launch ({FLOPS_PER_PAIR_HEAD_DIM[ps]:g}*d*Hq "
                       "per allowed pair) / mean launch time from HIP events on the launch stream; executed_mfma "
                       "counts the MFMA work the kernels run; traffic = calibrated FETCH_SIZE + WRITE_SIZE bytes "
                       "per launch")
        return r

    rooflines = {ps: roof(ps) for ps in passes}
    dominant = max(passes, key=lambda ps: rooflines[ps]["launch_ms"])

    # delta alone, after the timed steps: launches back to back on the first
    # rank's (dO, O), so no other kernel's dirty cache lines drain during it
    # (inside a step it follows the forward's output writes and the zeroing of
    # dQ).
    delta_alone = None
    if bwd:
        r0 = ranks[0]
        o_r, (do_r, dl_r) = fplans[r0].out, deltas[r0]
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        torch.cuda.synchronize()
        for a, b in dev_ev:
            a.record(stream)
            cpa.cp_attn_bwd_delta(do_r, o_r, dl_r)
            b.record(stream)
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in dev_ev)
        dbytes = do_r.numel() * do_r.element_size() + o_r.numel() * o_r.element_size() + dl_r.numel() * 4
        med = ts[len(ts) // 2]
        delta_alone = {"launches": len(ts), "median_us": round(med * 1e3, 2), "bytes": dbytes,
                       "GB/s": round(dbytes / (med * 1e-3) / 1e9, 1), "peak_GB/s": PEAK_HBM_GBS}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, full, idx[ranks[0]], allp, cu, args.cpu_seconds, ranks[0], bwd)

    per_pass = {}
    for ps in passes:
        tot_ms = sum(launch_ms[ps].values())
        rate = sum(flops[ps].values()) / (tot_ms * 1e-3) / 1e12
        every = [x for r in ranks for x in every_ms[ps][r]]
        per_pass[ps] = {"TFLOP/s": round(rate, 3), "pct_peak": round(100 * rate / peak, 2)}
        if ps == "bwd":
            per_pass[ps]["TFLOP/s_recompute_counted"] = round(
                rate * FLOPS_RECOMPUTE_COUNTED[ps] / FLOPS_PER_PAIR_HEAD_DIM[ps], 3)
        if peak_at_sclk:
            per_pass[ps]["pct_peak_at_measured_sclk"] = round(100 * rate / peak_at_sclk, 2)
        per_pass[ps]["launch_ms"] = {"median": round(float(np.median(every)), 4), "min": round(min(every), 4),
                                     "max": round(max(every), 4), "launches": len(every)}
        per_pass[ps]["per_rank_ms"] = {str(r): round(x, 4) for r, x in launch_ms[ps].items()}
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
        "config": {"workload": w.name, "pass": "fwd+bwd" if bwd else "fwd", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "d": w.d, "S": w.S, "cp": w.cp, "ranks": ranks, "varlen": w.varlen,
                   **({"varlen_deal": args.varlen_mode, "docs": len(cu) - 1} if cu is not None else {}),
                   "step": ("per rank: ring forward, delta, ring backward (fp32 dQ/dK/dV zeroed once a step)"
                            if bwd else "ring forward of each listed virtual rank") +
                           ", ranks sequential, K/V resident"},
        "pct_peak": round(100 * value / peak, 2),
        **({"value_recompute_counted": round(value_recompute, 3),
            "flops_per_pair_head_dim": "fwd 4*d, bwd 8*d (value); bwd 10*d (value_recompute_counted)"}
           if bwd else {}),
        **({"pct_peak_at_measured_sclk": round(100 * value / peak_at_sclk, 2)} if peak_at_sclk else {}),
        "clocks": clocks,
        "passes": per_pass,
        "roofline": rooflines[dominant],
        "roofline_by_pass": rooflines,
        **({"delta_alone": delta_alone} if delta_alone else {}),
        "cpu_baseline": cpu,
    }
    if balance is not None:
        out["balance"] = balance
    print(json.dumps(out), flush=True)


def a2a_bench(args, w):
    """--pass a2a (see the module docstring)."""
    import numpy as np
    import torch

    import context_causal_attention_amd as cpa

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    rows = w.S // w.cp
    g_ = torch.Generator(device="cpu")
    g_.manual_seed(w.seed)
    x = torch.randn(rows, w.Hq, w.d, generator=g_, dtype=torch.float32).to(dt).to(dev)
    nbytes = x.numel() * x.element_size()
    groups = [int(t) for t in args.a2a_groups.split(",")]
    stream = torch.cuda.current_stream(dev)
    res = {}
    for g in groups:
        send = cpa.cp_a2a_pack(x, g)
        y = cpa.cp_a2a_unpack(send)
        back = torch.empty_like(x)
        calls = {"pack": lambda: cpa.cp_a2a_pack(x, g, send),
                 "unpack": lambda: cpa.cp_a2a_unpack(send, y),
                 "unpack_inverse": lambda: cpa.cp_a2a_unpack_inverse(y, g, send),
                 "pack_inverse": lambda: cpa.cp_a2a_pack_inverse(send, back)}
        for name, fn in calls.items():
            for _ in range(args.warmup):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            torch.cuda.synchronize()
            for a, b in ev:
                a.record(stream)
                fn()
                b.record(stream)
            torch.cuda.synchronize()
            ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
            res[f"g{g}_{name}"] = {"ms": round(ms, 5), "GB/s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}
            print(f"[bench] a2a g={g} {name}: {ms * 1e3:.1f} us, {2 * nbytes / (ms * 1e-3) / 1e9:.0f} GB/s",
                  file=sys.stderr, flush=True)
    # Context: a plain device copy (torch's copy kernel) of the same bytes.
    dst = torch.empty_like(x)
    for _ in range(args.warmup):
        dst.copy_(x)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        dst.copy_(x)
        b.record(stream)
    torch.cuda.synchronize()
    copy_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    rates = [v["GB/s"] for v in res.values()]
    value = float(np.mean(rates))
    dominant = min(res, key=lambda k: res[k]["GB/s"])
    ms_dom = res[dominant]["ms"]
    out = {
        "metric": "head exchange layout (all-to-all level of hierarchical CP): GB/s read + written per call",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(float(np.mean([v["ms"] for v in res.values()])), 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "a2a", "rows": rows, "heads": w.Hq, "d": w.d, "groups": groups,
                   "step": "one call on one rank's query shard [S/cp, Hq, d]"},
        "a2a": res,
        "plain_copy_same_bytes": {"ms": round(copy_ms, 5), "GB/s": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(2 * nbytes / (ms_dom * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(2 * nbytes / (ms_dom * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "traffic": stored_traffic("a2a", w.name),
                     "kernel": f"rows_kernel of the slowest call ({dominant}); achieved = algorithmic bytes "
                               f"(the shard read once and written once, {2 * nbytes} B) / mean call time from HIP "
                               "events on the launch stream; traffic = calibrated FETCH_SIZE + WRITE_SIZE bytes "
                               "per dispatch, mean over the calls"},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def rotate_bench(args, w):
    """--pass rotate (see the module docstring)."""
    import numpy as np
    import torch

    import context_causal_attention_amd as cpa
    import seeded_inputs as si

    dev = torch.device("cuda:0")
    full = si.make_qkv(w.B, w.Hq, w.Hkv, w.S, w.d, w.dtype, seed=w.seed)
    q, k, v = full
    cu = si.workload_cu_seqlens(w)
    ranks = list(range(w.cp)) if args.ranks == "all" else [int(x) for x in args.ranks.split(",")]
    if cu is None:
        allp = cpa.cp_unshard_zigzag(w.S, w.cp)
        idx = {r: (cpa.cp_shard_zigzag(w.S, w.cp, r), None) for r in ranks}
    else:
        vmode = {"stream": cpa.CP_STREAM, "per_doc": cpa.CP_PER_DOC, "whole_doc": cpa.CP_WHOLE_DOC}[args.varlen_mode]
        every = [cpa.cp_varlen_index(cu, w.cp, r, vmode) for r in range(w.cp)]
        allp = np.concatenate([e[0] for e in every])
        idx = {r: every[r] for r in ranks}
    ai = torch.from_numpy(allp.astype(np.int64))
    k_all = k.index_select(2, ai).to(dev)
    v_all = v.index_select(2, ai).to(dev)
    copy_stream = torch.cuda.Stream(device=dev)
    kinds = ["fused", "steps_in_place", "steps_staged", "steps_staged_in_line"]
    plans, pairs = {}, {}
    for r in ranks:
        pos, lo = idx[r]
        q_loc = q.index_select(2, torch.from_numpy(pos.astype(np.int64))).to(dev)
        a = (q_loc, k_all, v_all, w.cp, r, pos, lo, allp)
        plans[r] = {
            "fused": cpa.RingFwdPlan(*a, scale=w.scale),
            "steps_in_place": cpa.RingFwdStepwisePlan(*a, scale=w.scale, staged=False),
            "steps_staged": cpa.RingFwdStepwisePlan(*a, scale=w.scale, staged=True, copy_stream=copy_stream),
            "steps_staged_in_line": cpa.RingFwdStepwisePlan(*a, scale=w.scale, staged=True,
                                                            copy_stream=torch.cuda.current_stream(dev)),
        }
        pairs[r] = cpa.cp_pairs(pos, lo, allp)
    # The copies alone: the (cp - 1) shards of K and V a rank receives, as
    # plain device copies of the same bytes on the copy stream.
    R = w.S // w.cp
    src_k = [k_all[:, :, s * R:(s + 1) * R] for s in range(w.cp)]
    src_v = [v_all[:, :, s * R:(s + 1) * R] for s in range(w.cp)]
    slot = [torch.empty_like(src_k[0]) for _ in range(4)]
    stream = torch.cuda.current_stream(dev)
    # The LSE merge alone (cp_attn_merge): one rank's fp32 partial (O, LSE)
    # merged into an accumulator of the same size, as an unfused ring step
    # would after its partial forward.
    mrows = w.B * w.Hq * R
    gm = torch.Generator(device="cpu")
    gm.manual_seed(w.seed)
    m_part = (torch.randn(mrows, w.d, generator=gm).to(dev), torch.randn(mrows, generator=gm).to(dev))
    m_acc = (torch.randn(mrows, w.d, generator=gm).to(dev), torch.randn(mrows, generator=gm).to(dev))
    merge_bytes = mrows * (3 * w.d * 4 + 3 * 4)
    extra = ["copies", "merge"]

    def copies():
        copy_stream.wait_stream(stream)
        with torch.cuda.stream(copy_stream):
            for t in range(1, w.cp):
                slot[2 * (t & 1)].copy_(src_k[t])
                slot[2 * (t & 1) + 1].copy_(src_v[t])
        stream.wait_stream(copy_stream)

    def step(ev=None):
        for r in ranks:
            for kd in kinds + extra:
                if ev is not None:
                    ev[kd][r][0].record(stream)
                if kd == "copies":
                    copies()
                elif kd == "merge":
                    cpa.cp_attn_merge(m_acc[0], m_acc[1], m_part[0], m_part[1])
                else:
                    plans[r][kd].run()
                if ev is not None:
                    ev[kd][r][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [{kd: {r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in ranks}
            for kd in kinds + extra} for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_ in range(args.steps):
        step(evs[s_])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {kd: {r: float(np.mean([evs[s_][kd][r][0].elapsed_time(evs[s_][kd][r][1]) for s_ in range(args.steps)]))
               for r in ranks} for kd in kinds + extra}
    fl = {r: FLOPS_PER_PAIR_HEAD_DIM["fwd"] * w.d * w.Hq * w.B * pairs[r] for r in ranks}
    tot = sum(fl.values())

    def rate(kd):
        return round(tot / (sum(ms[kd].values()) * 1e-3) / 1e12, 3)

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    staged = sum(ms["steps_staged"].values())
    inplace = sum(ms["steps_in_place"].values())
    shard_bytes = 2 * w.B * w.Hkv * R * w.d * (2 if w.dtype == "bf16" else 4)
    copy_ms = sum(ms["copies"].values()) / len(ranks)
    merge_ms = sum(ms["merge"].values()) / len(ranks)
    for kd in kinds + extra:
        print(f"[bench] {kd} per-rank ms: " + ", ".join(f"{r}:{ms[kd][r]:.3f}" for r in ranks),
              file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, full, idx[ranks[0]], allp, cu, args.cpu_seconds, ranks[0], False)
    ach = tot / (staged * 1e-3) / 1e12
    out = {
        "metric": "ring forward as separate steps with rotating K/V copies: TFLOP/s per virtual rank",
        "value": rate("steps_staged"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "rotate", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "S": w.S,
                   "cp": w.cp, "ranks": ranks,
                   "step": "per rank, one after another: the fused ring, the steps in place, the steps with "
                           "staged copies on a second stream, the same in line, the copies alone and one LSE "
                           "merge of a rank-sized partial alone; value is the staged, overlapped rate"},
        "pct_peak": round(100 * rate("steps_staged") / peak, 2),
        "rotate": {
            "TFLOP/s": {kd: rate(kd) for kd in kinds},
            "per_rank_ms": {kd: {str(r): round(x, 4) for r, x in ms[kd].items()} for kd in kinds + extra},
            "copy_bytes_per_rank": shard_bytes * (w.cp - 1),
            "copies_alone_GB/s": round(shard_bytes * (w.cp - 1) / (copy_ms * 1e-3) / 1e9, 1),
            "staged_over_in_place": round(staged / inplace, 4),
            "exposed_copy_ms_per_rank": round((staged - inplace) / len(ranks), 4),
            "merge_alone": {"rows": mrows, "bytes": merge_bytes, "ms": round(merge_ms, 5),
                            "GB/s": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1), "peak_GB/s": PEAK_HBM_GBS},
        },
        "roofline": {"bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ach / peak, 4), "traffic": None,
                     "kernel": "cp_attn_ring_fwd_stepwise launch with staging (per step fwd_bf16_kernel over one "
                               "shard, merging in its epilogue; copies on a second stream); achieved = algorithmic flops per "
                               "launch / mean launch time from HIP events on the launch stream"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, full, idx_r, allp, cu, target_s, rank_id, bwd):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload,
    one query head at a time until ~target_s have passed: the forward
    (attention_fwd) over all of one virtual rank's rows, or for --pass fwdbwd
    the backward (attention_bwd, which runs its own forward) over every 16th
    of those rows; flops counted like the GPU's value (4*d per pair for the
    forward, 8*d more for the backward), from the exact pair count of the rows
    sampled."""
    import numpy as np
    import oracle as orc
    import context_causal_attention_amd as cpa

    pos, lo = idx_r
    q, k, v = full[:3]
    blas = None
    try:
        from threadpoolctl import threadpool_info
        np.dot(np.ones((2, 2)), np.ones((2, 2)))  # loads the BLAS library so that it is listed
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(int(i.get("num_threads", 1)) for i in infos)
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in infos)
    except Exception:
        cores = len(os.sched_getaffinity(0))
    g = w.Hq // w.Hkv
    stride = 16 if bwd else 1
    rows = pos[::stride]
    pairs = cpa.cp_pairs(rows, None if lo is None else lo[::stride], allp)
    per_pair = FLOPS_PER_PAIR_HEAD_DIM["fwd"] + (FLOPS_PER_PAIR_HEAD_DIM["bwd"] if bwd else 0.0)
    t0 = time.perf_counter()
    done = 0
    while done < w.Hq:
        h = done
        qh = q[:, h:h + 1].double().numpy()
        kh = k[:, h // g:h // g + 1].double().numpy()
        vh = v[:, h // g:h // g + 1].double().numpy()
        if bwd:
            do = full[3][:, h:h + 1].double().numpy()[:, :, rows]
            orc.attention_bwd(qh, kh, vh, do, w.scale, cu_seqlens=cu, rows=rows)
        else:
            orc.attention_fwd(qh, kh, vh, w.scale, cu_seqlens=cu, rows=rows)
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    fl = per_pair * w.d * done * pairs
    what = (f"forward+backward (attention_bwd) of every {stride}th row" if bwd else "forward of the rows")
    return {"value": round(fl / el / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "blas": blas, "kind": "oracle",
            "sample": f"{w.name}: {what} of virtual rank {rank_id}, {done} of {w.Hq} query heads, "
                      f"fp64 numpy, {el:.1f}s"}


if __name__ == "__main__":
    main()
