"""Benchmark of the dense flash-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one fa_fwd call on the causal GQA prefill workload of the gfx950
prefill page's headline row (B=1, Hq=128, Hkv=8, Sq=Sk=8192, D=128, bf16,
inputs N(0,1), scale 1/sqrt(128)), with Q/K/V already resident in HBM.
`value` is useful TFLOP/s: 4*D per admissible (query, key) pair, causal
pairs only.  The Sq=1 split-KV decode (B1/Hq8/Hkv2/D128, L = 65536 valid
tokens in a cache of 65536 + 128 whose last 128 rows hold bf16 quiet NaN)
is timed in the same run and reported as GB/s of algorithmic bytes in the
"decode" object (with the same call through a page table and a 4-token
causal step), and the packed varlen forward on a ragged batch (16 sequences
of 256..8192 tokens, Hq32/Hkv8/D128, causal) in the "varlen" object.  The
"configs" object times every other prefill workload of the pages (the tiny
case, MHA causal / non-causal / fp16, batched GQA at D128 and D64, the
ragged 1000 x 3000 case, the Sq sweep) and decode latency per token at
capacity 128 and at short lengths in a 65536-token cache.

One JSON line is printed.  Besides the throughput it carries
  roofline      the prefill kernel's average launch time (HIP events on the
                stream it runs on) against the bf16 dense MFMA peak, plus the
                HBM traffic measured by hardware counters when the stored
                counter summary still matches the kernel source;
  cpu_baseline  the CPU oracle timed on this host over a bounded sample of
                the same workload (whole query heads);
  parity        the GPU outputs of that sample, of the decode call and of
                sampled varlen rows against the same oracle (the CPU leg is
                the only part of this script that runs the oracle; with
                --cpu-sample-heads 0 both objects are null).
The line is printed only if every parity check passes.
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
PEAK_SCLK_MHZ = 2400             # shader clock the published matrix peak assumes
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


class ClockSampler:
    """Samples the GPU's current shader and memory clocks (the amdgpu driver's
    pp_dpm_sclk / pp_dpm_mclk files, the level marked '*') from a thread while
    a timed region runs.  Dense MFMA work is power-limited, so the clock it
    holds moves the result from box to box; this records it beside the
    figure.  Reads files only, no GPU call."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.files = {}
        for name in ("sclk", "mclk"):
            found = sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{name}"))
            if found:
                self.files[name] = found[0]
        self.period = period_s
        self.samples = {name: [] for name in self.files}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self, path):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def _run(self):
        while not self._stop.is_set():
            for name, path in self.files.items():
                v = self._read(path)
                if v is not None:
                    self.samples[name].append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.files:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.files:
            self._thread.join()

    def summary(self):
        if not any(self.samples.values()):
            return None
        out = {}
        for name, v in self.samples.items():
            if v:
                v = sorted(v)
                out[f"{name}_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1],
                                      "samples": len(v)}
        return out


def clock_context(summary, achieved_tflops):
    """The sampled clocks plus the matrix peak at the median shader clock held
    during the timed region (the published peak assumes 2400 MHz) and the
    kernel's fraction of it.  Context only: the roofline keeps the published
    peak."""
    if not summary or "sclk_mhz" not in summary:
        return summary
    mhz = summary["sclk_mhz"]["median"]
    if mhz <= 0:
        return summary
    peak = MFMA_BF16_PEAK_TFLOPS * mhz / PEAK_SCLK_MHZ
    summary["mfma_peak_at_median_sclk_tflops"] = round(peak, 1)
    summary["frac_at_median_sclk"] = round(achieved_tflops / peak, 4)
    return summary


def dev(bits, dtype):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).cuda()


def host_bits(t):
    import numpy as np
    import torch
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def worst_frac(got, ref):
    """Largest |got - ref| / (1e-2 + 1e-2 |ref|); inf if got is not finite."""
    import numpy as np
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref) / (1e-2 + 1e-2 * np.abs(ref)))) if got.size else 0.0


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(prefill, decode, varlen, heads, backward=None):
    """The CPU oracle, as it stands, on this host.

    Times it over `heads` whole query heads of the prefill workload (the CPU
    baseline) and compares the GPU output of those heads with its result; also
    runs it on the decode call and on sampled rows of the varlen batch and
    compares those GPU outputs.  Raises SystemExit on any parity miss."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v, out_bits, s = prefill
    qf = oracle.widen(q[:, :heads], s.dtype)
    gqa = s.Hq // s.Hkv
    nkv = (heads + gqa - 1) // gqa
    kf, vf = oracle.widen(k[:, :nkv], s.dtype), oracle.widen(v[:, :nkv], s.dtype)
    # keep the GQA mapping of the full workload: head h reads kv head h // gqa
    kk = np.repeat(kf, gqa, axis=1)[:, :heads]
    vv = np.repeat(vf, gqa, axis=1)[:, :heads]
    t0 = time.perf_counter()
    ref = oracle.attention_ref(qf, kk, vv, s.causal, s.scale)
    dt = time.perf_counter() - t0
    parity = {"prefill_heads": heads,
              "prefill_worst_frac": worst_frac(oracle.widen(out_bits[:, :heads], s.dtype), ref)}
    flop = 4 * s.D * s.B * heads * s.admissible_pairs_per_head()
    base = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} of {s.Hq} query heads (B=1, Sq=Sk={s.Sq}, D={s.D}, causal), "
                      f"{dt:.1f} s of float64 NumPy",
            "blas_threads": int(threads), "cpu_model": cpu_model()}
    if decode is not None:
        qb, kb, vb, L, scale, dout = decode
        t0 = time.perf_counter()
        dref = oracle.decode_ref(oracle.widen(qb, "bf16"), oracle.widen(kb, "bf16"),
                                 oracle.widen(vb, "bf16"), [L], scale)
        base["decode_seconds_per_token"] = round(time.perf_counter() - t0, 4)
        parity["decode_worst_frac"] = worst_frac(oracle.widen(dout, "bf16"), dref)
    if varlen is not None:
        vq, vk, vv_, vout, vs = varlen
        rng = np.random.default_rng(13)
        worst = 0.0
        qw, kw, vw = (oracle.widen(x, vs.dtype) for x in (vq, vk, vv_))
        cu_q, cu_k = vs.cu_q, vs.cu_k
        for b in sorted(set(rng.integers(0, vs.B, 3).tolist())):
            q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
            h = int(rng.integers(0, vs.Hq))
            rows = np.unique(np.concatenate([[0, q1 - q0 - 1], rng.integers(0, q1 - q0, 16)]))
            r = oracle.attention_rows_ref(qw[q0:q1].transpose(1, 0, 2)[None],
                                          kw[k0:k1].transpose(1, 0, 2)[None],
                                          vw[k0:k1].transpose(1, 0, 2)[None],
                                          vs.causal, vs.scale, 0, h, rows)
            worst = max(worst, worst_frac(oracle.widen(vout[q0 + rows, h], vs.dtype), r))
        parity["varlen_sampled_worst_frac"] = worst
    if backward is not None:
        # sampled dQ rows of the backward against the oracle (bound scaled by
        # the sample's largest gradient, as in the backward tests)
        g, dq_bits = backward
        gf = oracle.widen(g, s.dtype)
        rng = np.random.default_rng(17)
        worst = 0.0
        for h in (0, s.Hq // 2 + 3, s.Hq - 1):
            rows = np.unique(np.concatenate([[0, s.Sq - 1], rng.integers(0, s.Sq, 6)]))
            qh = oracle.widen(q[:, h:h + 1], s.dtype)
            hk = h // gqa
            kh, vh = oracle.widen(k[:, hk:hk + 1], s.dtype), oracle.widen(v[:, hk:hk + 1], s.dtype)
            r = oracle.attention_bwd_dq_rows_ref(qh, kh, vh, gf[:, h:h + 1], s.causal, s.scale, 0,
                                                 0, rows)
            got = oracle.widen(dq_bits[0, h, rows], s.dtype)
            bound = 1e-2 * np.max(np.abs(r)) + 1e-2 * np.abs(r) + 1e-12
            worst = max(worst, float(np.max(np.abs(got - r) / bound)) if np.all(np.isfinite(got))
                        else float("inf"))
        parity["backward_dq_sampled_worst_frac"] = worst
    bad = {key: val for key, val in parity.items() if key.endswith("frac") and not val <= 1.0}
    if bad:
        raise SystemExit(f"parity check failed: {bad}")
    for key in list(parity):
        if key.endswith("frac"):
            parity[key] = round(parity[key], 4)
    return base, parity


def timed_calls(torch, calls, n, warmup):
    """Mean time (us) per call of `calls` (zero-argument callables, used in
    rotation), kernel-side: HIP events on the current stream around n calls."""
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def decode_call(fa, torch, q, kc, vc, vl, out, ws, scale, causal=False):
    """fa_decode / fa_decode_multi with its arguments marshalled once, so that a
    timed loop costs one foreign call per launch."""
    lib = fa.lib()
    stream = torch.cuda.current_stream().cuda_stream
    B, cap, Hkv, D = kc.shape
    if q.dim() == 3:
        Hq = q.shape[1]
        fn, args = lib.fa_decode, (q.data_ptr(), kc.data_ptr(), vc.data_ptr(), vl.data_ptr(), cap,
                                   out.data_ptr(), B, Hq, Hkv, D, int(causal), scale, 0, ws.ptr,
                                   ws.nbytes, stream)
    else:
        Sq, Hq = q.shape[1], q.shape[2]
        fn, args = lib.fa_decode_multi, (q.data_ptr(), kc.data_ptr(), vc.data_ptr(), vl.data_ptr(),
                                         cap, out.data_ptr(), B, Sq, Hq, Hkv, D, int(causal), scale,
                                         0, ws.ptr, ws.nbytes, stream)

    def call():
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"decode failed: {st}")
    return call


def bench_decode(fa, torch, steps, warmup):
    """Sq=1 decode over L=65536 valid tokens of a cache with room for 128 more
    whose unused rows hold bf16 quiet NaN: GB/s of algorithmic bytes, cold
    (rotating over more caches than the 256 MB MALL holds) and warm."""
    import numpy as np

    import workloads as wl
    B, Hq, Hkv, D = 1, 8, 2, 128
    L = 65536
    cap = L + 128
    copies = 9  # 9 x 64 MiB of K+V > 2 x the 256 MB last-level cache
    kb = np.full((B, cap, Hkv, D), wl.BF16_QNAN, dtype=np.uint16)
    vb = kb.copy()
    kb[:, :L] = wl.normal_bits((B, L, Hkv, D), 5001, "bf16")
    vb[:, :L] = wl.normal_bits((B, L, Hkv, D), 5002, "bf16")
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
    first = host_bits(out)
    nbytes = 2 * L * Hkv * D * 2 + 2 * Hq * D * 2 + 4 * B
    res = {}
    stream = torch.cuda.current_stream()
    calls = [decode_call(fa, torch, q, kcs[j], vcs[j], vl, out, ws, scale) for j in range(copies)]
    for mode in ("cold", "warm"):
        us = timed_calls(torch, calls if mode == "cold" else calls[:1], steps, warmup)
        res[mode] = {"us_per_call": us, "GB_s": nbytes / (us * 1e-6) / 1e9}
    # the same caches read as pools of 128-token pages through a page table
    # (identity mapping), cold
    P = 128
    kps = [kc.view(cap // P, P, Hkv, D) for kc in kcs]
    vps = [vc.view(cap // P, P, Hkv, D) for vc in vcs]
    table = torch.arange(cap // P, dtype=torch.int32, device="cuda").view(1, cap // P)
    lib = fa.lib()
    st = torch.cuda.current_stream().cuda_stream

    def paged_call(j):
        args = (q.data_ptr(), kps[j].data_ptr(), vps[j].data_ptr(), table.data_ptr(), vl.data_ptr(),
                P, cap // P, cap // P, out.data_ptr(), B, Hq, Hkv, D, 0, scale, 0, ws.ptr,
                ws.nbytes, st)
        return lambda: lib.fa_decode_paged(*args)
    us = timed_calls(torch, [paged_call(j) for j in range(copies)], steps, warmup)
    res["paged"] = {"page_size": P, "us_per_call": us, "GB_s": nbytes / (us * 1e-6) / 1e9}
    # a multi-token step: 4 query tokens at the end of the same caches, causal
    Sq = 4
    q4 = dev(wl.normal_bits((B, Sq, Hq, D), 5004, "bf16"), torch.bfloat16)
    out4 = torch.empty_like(q4)
    ws4 = fa.DecodeWorkspace(B, Hq, Hkv, D, cap, Sq=Sq)
    calls4 = [decode_call(fa, torch, q4, kcs[j], vcs[j], vl, out4, ws4, scale, causal=True)
              for j in range(copies)]
    us = timed_calls(torch, calls4, steps, warmup)
    nb4 = 2 * L * Hkv * D * 2 + 2 * Sq * Hq * D * 2 + 4 * B
    res["multi"] = {"query_tokens": Sq, "causal": True, "us_per_call": us,
                    "GB_s": nb4 / (us * 1e-6) / 1e9}
    return {"metric": "bf16 Sq=1 split-KV decode GB/s @B1/Hq8/Hkv2/D128/L65536, NaN tail "
                      "(cache of 65536 + 128 tokens)",
            "value": res["cold"]["GB_s"], "unit": "GB/s", "frac_of_hbm_peak":
            res["cold"]["GB_s"] / HBM_PEAK_GBS, "us_per_call": res["cold"]["us_per_call"],
            "warm": res["warm"], "paged_cold": res["paged"], "multi_token_cold": res["multi"],
            "algorithmic_bytes": nbytes,
            "traffic": stored_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)}, \
        (qb, kb, vb, L, scale, first)


def fwd_call(fa, torch, s):
    """fa_fwd on seeded N(0,1) inputs of workload `s` with its arguments
    marshalled once; returns (call, tensors to keep alive)."""
    import workloads as wl
    q, k, v = wl.prefill_inputs(s)
    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float16
    tq, tk, tv = dev(q, tdt), dev(k, tdt), dev(v, tdt)
    out = torch.empty_like(tq)
    lib = fa.lib()
    args = (tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), s.B, s.Hq, s.Hkv, s.Sq,
            s.Sk, s.D, int(s.causal), s.scale, 0 if s.dtype == "bf16" else 1,
            torch.cuda.current_stream().cuda_stream)

    def call():
        st = lib.fa_fwd(*args)
        if st != 0:
            raise RuntimeError(f"fa_fwd failed: {st}")
    return call, (tq, tk, tv, out)


def bench_configs(fa, torch):
    """Every other prefill workload of the pages (kernel-side time, HIP events
    around back-to-back calls; about 0.1 s of calls each) and decode latency
    per token over 128 successive valid lengths, at capacity 128 and inside a
    65536-token cache."""
    import workloads as wl
    out = {}
    for s in (wl.TINY, wl.MHA_CAUSAL, wl.MHA_FULL, wl.MHA_FP16, wl.GQA_D128, wl.GQA_D64,
              wl.RAGGED_D128, wl.RAGGED_D64) + wl.SWEEP:
        call, keep = fwd_call(fa, torch, s)
        first = timed_calls(torch, [call], 3, 2)
        n = int(min(2000, max(20, 1e5 / max(first, 1.0))))
        us = timed_calls(torch, [call], n, 3)
        flop = s.useful_flop()
        tf = flop / (us * 1e-6) / 1e12
        plan = fa.fwd_plan(s.B, s.Hq, s.Hkv, s.Sq, s.Sk, s.D, s.causal)
        out[s.name] = {"ms": round(us / 1e3, 5), "tflops": round(tf, 1),
                       "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                       "dtype": s.dtype, "causal": s.causal, "useful_flop": flop, "calls": n,
                       "schedule": {key: plan[key] for key in ("work_items", "grid", "persistent",
                                                               "hkv_major", "xcd_map",
                                                               "split_tiles", "queue")}}
        del keep
    B, Hq, Hkv, D = 1, 8, 2, 128
    scale = 1 / math.sqrt(D)
    for cap in (128, 65536):
        kb = wl.normal_bits((B, cap, Hkv, D), 5101, "bf16")
        vb = wl.normal_bits((B, cap, Hkv, D), 5102, "bf16")
        kc, vc = dev(kb, torch.bfloat16), dev(vb, torch.bfloat16)
        q = dev(wl.normal_bits((B, Hq, D), 5103, "bf16"), torch.bfloat16)
        o = torch.empty_like(q)
        ws = fa.DecodeWorkspace(B, Hq, Hkv, D, cap)
        lens = [torch.tensor([L], dtype=torch.int32, device="cuda") for L in range(1, 129)]
        calls = [decode_call(fa, torch, q, kc, vc, vl, o, ws, scale) for vl in lens]
        us = timed_calls(torch, calls, 128 * 8, 128)
        name = f"decode_b1_hq8_hkv2_d128_cap{cap}_len1to128"
        out[name] = {"us_per_token": round(us, 3), "valid_lengths": "1..128, one call each",
                     "calls": 128 * 8}
        del kc, vc
    return out


def bench_varlen(fa, torch, steps, warmup):
    """The packed varlen forward on a ragged batch (16 causal sequences of
    256..8192 tokens, Hq32/Hkv8/D128, bf16): useful TFLOP/s."""
    import workloads as wl
    s = wl.VARLEN
    q, k, v = wl.varlen_inputs(s)
    tq, tk, tv = dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16)
    cq = torch.tensor(s.cu_q, dtype=torch.int32, device="cuda")
    ck = torch.tensor(s.cu_k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(tq)
    mq, mk = max(s.lens_q), max(s.lens_k)

    def call():
        fa.fwd_varlen(tq, tk, tv, cq, ck, mq, mk, causal=s.causal, scale=s.scale, out=out)

    call()
    torch.cuda.synchronize()
    first = host_bits(out)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = s.useful_flop()
    tf = flop / (ms * 1e-3) / 1e12
    return {"metric": "bf16 causal packed-varlen prefill TFLOP/s @16 seqs of 256..8192 tokens, "
                      "Hq32/Hkv8/D128",
            "value": round(tf, 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
            "ms_per_call": round(ms, 4),
            "config": {"workload": s.name, "B": s.B, "total_tokens": int(sum(s.lens_q)),
                       "max_seqlen": mq, "Hq": s.Hq, "Hkv": s.Hkv, "D": s.D,
                       "causal": s.causal, "useful_flop": flop}}, \
        (q, k, v, first, s)


def bench_backward(fa, torch, q, k, v, tq, tk, tv, s, steps, warmup):
    """The backward pass at the headline shape for a seeded N(0,1) output
    gradient: useful TFLOP/s at 10*D per admissible pair (the five products
    S, dP, dV, dK, dQ of 2*D each)."""
    import workloads as wl
    g = wl.normal_bits((s.B, s.Hq, s.Sq, s.D), s.seed_base + 3, s.dtype)
    tg = dev(g, torch.bfloat16)
    o, lse = fa.fwd(tq, tk, tv, causal=s.causal, scale=s.scale, return_lse=True)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tg, lse, causal=s.causal, scale=s.scale)
    torch.cuda.synchronize()
    first = host_bits(dq)
    for _ in range(warmup):
        fa.bwd(tq, tk, tv, o, tg, lse, causal=s.causal, scale=s.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fa.bwd(tq, tk, tv, o, tg, lse, causal=s.causal, scale=s.scale, dq=dq, dk=dk, dv=dv)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 10 * s.D * s.B * s.Hq * s.admissible_pairs_per_head()
    tf = flop / (ms * 1e-3) / 1e12
    return {"metric": "bf16 causal FA backward TFLOP/s @Hq128/Hkv8/D128/Sq8192 (10*D per pair)",
            "value": round(tf, 2), "unit": "TFLOP/s",
            "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "ms_per_call": round(ms, 3),
            "useful_flop": flop}, (g, first)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-heads", type=int, default=24,
                    help="query heads the CPU oracle is timed on (0: no CPU baseline)")
    ap.add_argument("--decode", type=int, default=1, help="also time decode (1) or not (0)")
    ap.add_argument("--varlen", type=int, default=1,
                    help="also time the packed varlen forward (1) or not (0)")
    ap.add_argument("--backward", type=int, default=1,
                    help="also time the backward pass (1) or not (0)")
    ap.add_argument("--configs", type=int, default=1,
                    help="also time the other workloads of the pages (1) or not (0)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(heads shard across GPUs with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

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
    out_bits = host_bits(out)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fa.fwd(tq, tk, tv, causal=True, scale=s.scale, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clocks:
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

    dec, dec_data = (bench_decode(fa, torch, max(args.steps, 20), args.warmup) if args.decode
                     else (None, None))
    vl, vl_data = (bench_varlen(fa, torch, max(args.steps // 5, 5), min(args.warmup, 2))
                   if args.varlen else (None, None))
    bw, bw_data = (bench_backward(fa, torch, q, k, v, tq, tk, tv, s, 3, 1) if args.backward
                   else (None, None))
    cfgs = bench_configs(fa, torch) if args.configs else None
    cpu = parity = None
    if args.cpu_sample_heads > 0:
        cpu, parity = cpu_leg((q, k, v, out_bits, s), dec_data, vl_data, args.cpu_sample_heads,
                              bw_data)

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
        "clocks_during_prefill": clock_context(clocks.summary(), achieved),
        "parity": parity,
        "decode": dec,
        "varlen": vl,
        "backward": bw,
        "configs": cfgs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
