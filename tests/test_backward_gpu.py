"""GPU parity of the backward pass (fa_bwd through the C ABI) against the CPU
float64 oracle's dQ, dK, dV.

Bound: gradients are not O(1) like attention outputs, so the absolute part of
the bound scales with the tensor's largest magnitude:
|gpu - oracle| <= 1e-2 max|oracle| + 1e-2 |oracle| elementwise, per tensor.
The GPU computes P and dS in fp32 and rounds them to the input type before
each product (relative 2^-9 for bf16), and takes D = rowsum(dO * O) from the
forward's rounded O, which this bound covers.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu


def _fa():
    import flash_attention_forward_fwd_amd as fa
    return fa


def grad_parity(got, ref, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    if ref.size == 0:
        return 0.0
    bound = 1e-2 * float(np.max(np.abs(ref))) + 1e-2 * np.abs(ref) + 1e-12
    frac = float(np.max(np.abs(got - ref) / bound))
    assert frac <= 1.0, f"{what}: bound exceeded, worst fraction {frac}"
    return frac


def run_bwd(q, k, v, g, causal, scale, dtype):
    fa = _fa()
    tq, tk, tv, tg = (to_dev(x, dtype) for x in (q, k, v, g))
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale, return_lse=True)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, tg, lse, causal=causal, scale=scale)
    return [oracle.widen(bits_of(x), dtype) for x in (dq, dk, dv)]


CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype
    (1, 2, 1, 256, 256, 64, True, "bf16"),
    (1, 4, 2, 300, 300, 128, True, "bf16"),
    (2, 4, 1, 257, 700, 64, True, "bf16"),      # bottom-right, ragged
    (1, 2, 2, 129, 65, 128, False, "bf16"),
    (1, 8, 2, 700, 300, 128, True, "bf16"),     # Sq > Sk: rows without keys
    (1, 3, 3, 511, 513, 128, False, "fp16"),
    (1, 2, 1, 1, 77, 128, True, "bf16"),        # one query row
    (1, 2, 1, 1000, 1, 64, True, "bf16"),       # one key
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_backward_parity(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = case
    q = wl.normal_bits((B, Hq, Sq, D), 1100 + Sq, dtype)
    k = wl.normal_bits((B, Hkv, Sk, D), 1101 + Sq, dtype)
    v = wl.normal_bits((B, Hkv, Sk, D), 1102 + Sq, dtype)
    g = wl.normal_bits((B, Hq, Sq, D), 1103 + Sq, dtype)
    scale = 1 / math.sqrt(D)
    got = run_bwd(q, k, v, g, causal, scale, dtype)
    ref = oracle.attention_bwd_ref(*(oracle.widen(x, dtype) for x in (q, k, v, g)), causal, scale)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        grad_parity(a, r, f"{name} {case}")


@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_backward_negative_and_zero_scale(scale):
    dtype, B, Hq, Hkv, S, D = "bf16", 1, 4, 2, 200, 128
    q = wl.normal_bits((B, Hq, S, D), 1201, dtype)
    k = wl.normal_bits((B, Hkv, S, D), 1202, dtype)
    v = wl.normal_bits((B, Hkv, S, D), 1203, dtype)
    g = wl.normal_bits((B, Hq, S, D), 1204, dtype)
    got = run_bwd(q, k, v, g, True, scale, dtype)
    ref = oracle.attention_bwd_ref(*(oracle.widen(x, dtype) for x in (q, k, v, g)), True, scale)
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        grad_parity(a, r, f"{name} scale={scale}")
    if scale == 0.0:
        assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)


def test_backward_is_deterministic():
    dtype, B, Hq, Hkv, S, D = "bf16", 1, 8, 2, 384, 128
    q, k, v, g = (wl.normal_bits(sh, 1300 + i, dtype) for i, sh in
                  enumerate([(B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D), (B, Hq, S, D)]))
    a = run_bwd(q, k, v, g, True, 0.09, dtype)
    b = run_bwd(q, k, v, g, True, 0.09, dtype)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_many_tiles_gqa4():
    # 2048 rows and keys: 16 dq blocks, 16 dk/dv blocks, a 4-head GQA group
    dtype, B, Hq, Hkv, S, D = "bf16", 1, 4, 1, 2048, 128
    q, k, v, g = (wl.normal_bits(sh, 1400 + i, dtype) for i, sh in
                  enumerate([(B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D), (B, Hq, S, D)]))
    got = run_bwd(q, k, v, g, True, 1 / math.sqrt(D), dtype)
    ref = oracle.attention_bwd_ref(*(oracle.widen(x, dtype) for x in (q, k, v, g)), True,
                                   1 / math.sqrt(D))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        grad_parity(a, r, f"{name} S=2048 gqa4")


@pytest.mark.parametrize("case", [(1, 8, 1, 4096, 4096, 128, True),
                                  (1, 16, 2, 1000, 4500, 64, True),
                                  (1, 8, 1, 4096, 4096, 128, False)],
                         ids=["s4096_gqa8_causal", "sq1000_sk4500_gqa8_d64", "s4096_gqa8_full"])
def test_backward_long_keys_gqa8(case):
    # dK / dV summed over an 8-head GQA group and over 4096+ keys: 32+ dk/dv
    # key blocks, each accumulating the contributions of every query block
    # and of all 8 query heads of its kv head (the full oracle backward,
    # a few seconds of float64 on the host)
    B, Hq, Hkv, Sq, Sk, D, causal = case
    dtype = "bf16"
    print(f"\n[backward] {case}", flush=True)
    q, k, v, g = (wl.normal_bits(sh, 1500 + i, dtype) for i, sh in
                  enumerate([(B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D), (B, Hq, Sq, D)]))
    scale = 1 / math.sqrt(D)
    got = run_bwd(q, k, v, g, causal, scale, dtype)
    ref = oracle.attention_bwd_ref(*(oracle.widen(x, dtype) for x in (q, k, v, g)), causal, scale)
    fr = [grad_parity(a, r, f"{name} {case}") for name, a, r in zip(("dq", "dk", "dv"), got, ref)]
    print(f"  worst fraction of bound dq {fr[0]:.3f} dk {fr[1]:.3f} dv {fr[2]:.3f}", flush=True)
