"""Benchmark of the dense flash-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fa_fwd call on the causal GQA prefill workload of the gfx950
prefill page's headline row (B=1, Hq=128, Hkv=8, Sq=Sk=8192, D=128, bf16,
inputs N(0,1), scale 1/sqrt(128)), with Q/K/V already resident in HBM.
`value` is useful TFLOP/s: 4*D per admissible (query, key) pair, causal
pairs only.  Before any figure is printed the same run checks sampled output
rows against the CPU oracle.  The Sq=1 split-KV decode (B1/Hq8/Hkv2/D128,
L = 65536, NaN-poisoned tail) is timed in the same run and reported as GB/s
of algorithmic bytes in the "decode" object.

One JSON line is printed.  Besides the throughput it carries
  roofline      the prefill kernel's average launch time (HIP events on the
                stream it runs on) against the bf16 dense MFMA peak, plus the
                HBM traffic measured by hardware counters when the stored
                counter summary still matches the kernel source;
  cpu_baseline  the CPU oracle timed on this host over a bounded sample of
                the same workload (whole query heads).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak
METRIC = "bf16 causal FA prefill TFLOP/s @Hq128/Hkv8/D128/Sq8192; % MFMA peak"
PAGE_TFLOPS = 948.0              # prefill page, "Measured": persistent shipped default (MI355X)
CALIB_BYTES = 256 << 20          # calibration copy: reads and writes 256 MiB
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_headline_traffic.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_l65536_traffic.json")
KERNEL_SOURCES = ["flash_attention_forward_fwd_amd/csrc/fa_prefill.hip",
                  "flash_attention_forward_fwd_amd/csrc/fa_common.h",
                  "flash_attention_forward_fwd_amd/csrc/fa_internal.h"]
DECODE_SOURCES = ["flash_attention_forward_fwd_amd/csrc/fa_decode.hip",
                  "flash_attention_forward_fwd_amd/csrc/fa_common.h",
                  "flash_attention_forward_fwd_amd/csrc/fa_internal.h"]


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that an edit of comments alone keeps the stored counter readings valid."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(path=TRAFFIC_FILE, sources=None):
    """HBM bytes per launch from a committed counter summary, or None when it
    is absent or was taken on a different kernel source."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def dev(bits, dtype):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).cuda()


def host_bits(t):
    import numpy as np
    import torch
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_sampled_rows(q, k, v, out_bits, s, rng, heads=2, rows=24):
    """Sampled rows of the output against the oracle; raises on a miss."""
    import numpy as np

    import oracle
    qf, kf, vf = oracle.widen(q, s.dtype), oracle.widen(k, s.dtype), oracle.widen(v, s.dtype)
    worst = 0.0
    for h in sorted(set(rng.integers(0, s.Hq, heads).tolist()) | {s.Hq - 1}):
        rr = np.unique(np.concatenate([[0, s.Sq - 1], rng.integers(0, s.Sq, rows)]))
        ref = oracle.attention_rows_ref(qf, kf, vf, s.causal, s.scale, 0, h, rr)
        got = oracle.widen(out_bits[0, h, rr], s.dtype)
        err = np.abs(got - ref)
        frac = float(np.max(err / (1e-2 + 1e-2 * np.abs(ref))))
        if not np.all(np.isfinite(got)) or frac > 1.0:
            raise SystemExit(f"parity check failed on head {h}: worst fraction {frac}")
        worst = max(worst, frac)
    return worst


def cpu_baseline(q, k, v, s, heads):
    """Time the oracle (as it stands) over `heads` whole query heads."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    qf = oracle.widen(q[:, :heads], s.dtype)
    gqa = s.Hq // s.Hkv
    nkv = (heads + gqa - 1) // gqa
    kf, vf = oracle.widen(k[:, :nkv], s.dtype), oracle.widen(v[:, :nkv], s.dtype)
    # keep the GQA mapping of the full workload: head h reads kv head h // gqa
    import numpy as np
    kk = np.repeat(kf, gqa, axis=1)[:, :heads]
    vv = np.repeat(vf, gqa, axis=1)[:, :heads]
    t0 = time.perf_counter()
    oracle.attention_ref(qf, kk, vv, s.causal, s.scale)
    dt = time.perf_counter() - t0
    flop = 4 * s.D * s.B * heads * s.admissible_pairs_per_head()
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {s.Hq} query heads (B=1, Sq=Sk={s.Sq}, D={s.D}, causal), "
                      f"{dt:.1f} s of float64 NumPy on {os.cpu_count()} visible CPUs",
            "seconds": dt}


def bench_decode(fa, torch, steps, warmup):
    """Sq=1 decode at capacity 65536, L=65536, NaN tail: GB/s of algorithmic
    bytes, cold (rotating over more caches than the 256 MB MALL holds) and warm."""
    import numpy as np

    import oracle
    import workloads as wl
    B, Hq, Hkv, D, cap = 1, 8, 2, 128, 65536
    L = cap
    copies = 9  # 9 x 64 MiB of K+V > 2 x the 256 MB last-level cache
    kb = wl.normal_bits((B, cap, Hkv, D), 5001, "bf16")
    vb = wl.normal_bits((B, cap, Hkv, D), 5002, "bf16")
    qb = wl.normal_bits((B, Hq, D), 5003, "bf16")
    kcs = [dev(kb, torch.bfloat16) for _ in range(copies)]
    vcs = [dev(vb, torch.bfloat16) for _ in range(copies)]
    q = dev(qb, torch.bfloat16)
    vl = torch.tensor([L], dtype=torch.int32, device="cuda")
    ws = fa.DecodeWorkspace(B, Hq, Hkv, D, cap)
    out = torch.empty_like(q)
    scale = 1 / math.sqrt(D)
    fa.decode(q, kcs[0], vcs[0], vl, scale=scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.decode_ref(oracle.widen(qb, "bf16"), oracle.widen(kb, "bf16"),
                            oracle.widen(vb, "bf16"), [L], scale)
    got = oracle.widen(host_bits(out), "bf16")
    frac = float(np.max(np.abs(got - ref) / (1e-2 + 1e-2 * np.abs(ref))))
    if not np.all(np.isfinite(got)) or frac > 1.0:
        raise SystemExit(f"decode parity check failed: worst fraction {frac}")
    nbytes = 2 * L * Hkv * D * 2 + 2 * Hq * D * 2 + 4 * B
    res = {}
    stream = torch.cuda.current_stream()
    for mode in ("cold", "warm"):
        for i in range(warmup):
            j = i % copies if mode == "cold" else 0
            fa.decode(q, kcs[j], vcs[j], vl, scale=scale, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            j = i % copies if mode == "cold" else 0
            fa.decode(q, kcs[j], vcs[j], vl, scale=scale, out=out, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        res[mode] = {"us_per_call": us, "GB_s": nbytes / (us * 1e-6) / 1e9}
    return {"metric": "bf16 Sq=1 split-KV decode GB/s @B1/Hq8/Hkv2/D128/L65536, NaN tail",
            "value": res["cold"]["GB_s"], "unit": "GB/s", "frac_of_hbm_peak":
            res["cold"]["GB_s"] / HBM_PEAK_GBS, "us_per_call": res["cold"]["us_per_call"],
            "warm": res["warm"], "algorithmic_bytes": nbytes, "parity_worst_frac": frac,
            "traffic": stored_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-heads", type=int, default=24,
                    help="query heads the CPU oracle is timed on (0: no CPU baseline)")
    ap.add_argument("--decode", type=int, default=1, help="also time decode (1) or not (0)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import flash_attention_forward_fwd_amd as fa
    import workloads as wl

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    fa.lib()
    s = wl.HEADLINE
    q, k, v = wl.prefill_inputs(s)
    tq, tk, tv = dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    out = torch.empty_like(tq)
    fa.fwd(tq, tk, tv, causal=True, scale=s.scale, out=out)
    torch.cuda.synchronize()
    worst = check_sampled_rows(q, k, v, host_bits(out), s, np.random.default_rng(11))

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fa.fwd(tq, tk, tv, causal=True, scale=s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        fa.fwd(tq, tk, tv, causal=True, scale=s.scale, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_kernel = e0.elapsed_time(e1) / args.steps
    flop = s.useful_flop()
    value = flop / (ms_step * 1e-3) / 1e12
    achieved = flop / (ms_kernel * 1e-3) / 1e12
    plan = fa.fwd_plan(s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, s.causal)

    # A plain device copy of known size after the timed region: hardware
    # counter passes over this script read its FETCH_SIZE / WRITE_SIZE to
    # scale the attention kernel's counters to bytes.
    calib_src = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device="cuda")
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    dec = bench_decode(fa, torch, max(args.steps, 20), args.warmup) if args.decode else None
    cpu = cpu_baseline(q, k, v, s, args.cpu_sample_heads) if args.cpu_sample_heads > 0 else None

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": round(value / PAGE_TFLOPS, 4), "dtype": "bf16",
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": s.name, "B": s.B, "Hq": s.Hq, "Hkv": s.Hkv, "Sq": s.Sq,
                   "Sk": s.Sk, "D": s.D, "causal": s.causal, "scale": s.scale,
                   "useful_flop": flop, "persistent": plan["persistent"],
                   "hkv_major": plan["hkv_major"], "grid": plan["grid"]},
        "frac_of_mfma_peak": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(),
                     "kernel": "prefill_kernel<128, bf16, causal>",
                     "avg_launch_ms": round(ms_kernel, 4),
                     "algorithmic_flop_per_launch": flop},
        "parity": {"sampled_rows_worst_frac_of_bound": round(worst, 4)},
        "decode": dec,
        "cpu_baseline": cpu,
    }
    if cpu:
        cpu.pop("seconds", None)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
