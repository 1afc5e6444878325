"""GPU parity of the packed variable-length forward (fa_fwd_varlen through the
C ABI) against the CPU float64 oracle, plus its layout and bitwise semantics.

Bound: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise on bf16/fp16 outputs.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bits_of, parity, to_dev

pytestmark = pytest.mark.gpu

CANARY = 0x3C3C  # storage bits pre-filled into rows that no sequence owns


def _fa():
    import flash_attention_forward_fwd_amd as fa
    return fa


def offsets(lens, start=0):
    return np.concatenate([[start], start + np.cumsum(lens)]).astype(np.int64)


def packed_inputs(total_q, total_k, Hq, Hkv, D, dtype, seed):
    q = wl.normal_bits((total_q, Hq, D), seed, dtype)
    k = wl.normal_bits((total_k, Hkv, D), seed + 1, dtype)
    v = wl.normal_bits((total_k, Hkv, D), seed + 2, dtype)
    return q, k, v


def run_varlen(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale, dtype, lse=False):
    import torch
    fa = _fa()
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out = to_dev(np.full(q.shape, CANARY, dtype=np.uint16), dtype)
    cq = torch.tensor(np.asarray(cu_q), dtype=torch.int32, device="cuda")
    ck = torch.tensor(np.asarray(cu_k), dtype=torch.int32, device="cuda")
    res = fa.fwd_varlen(tq, tk, tv, cq, ck, max_q, max_k, causal=causal, scale=scale, out=out,
                        return_lse=lse)
    if lse:
        return bits_of(res[0]), res[1].cpu().numpy().astype(np.float64)
    return bits_of(res)


def owned_rows(cu_q, total_q):
    own = np.zeros(total_q, dtype=bool)
    for b in range(len(cu_q) - 1):
        own[cu_q[b]:cu_q[b + 1]] = True
    return own


CASES = [
    # lens_q, lens_k (None = same), Hq, Hkv, D, causal, dtype, extra max_seqlen_q
    ([300, 0, 1, 513, 256, 77], None, 4, 2, 128, True, "bf16", 0),
    ([100, 700, 257], [300, 200, 1000], 8, 2, 64, True, "bf16", 0),   # Sq > Sk in one
    ([129, 65, 1000], [65, 513, 3], 3, 3, 128, False, "fp16", 0),
    ([5, 64, 33, 1, 60, 17, 64, 2, 40, 9, 63, 30], None, 2, 1, 64, True, "bf16", 0),
    ([200, 31], [500, 90], 4, 1, 128, True, "bf16", 300),            # max above every length
    # 70 sequences (more than one 64-wide ballot of the schedule table), kv-head-major order
    (list(np.random.default_rng(771).integers(0, 601, 70)), None, 8, 2, 64, True, "bf16", 0),
    # more sequences than the schedule table holds: the plain order with empty items skipped
    (list(np.random.default_rng(772).integers(0, 4, 4100)), None, 2, 1, 64, True, "bf16", 0),
    # Hkv a multiple of 8 on a persistent launch: whole kv heads dealt to the XCDs, through
    # the compacted list and through the plain order
    ([300, 0, 1, 513, 256, 77, 700, 1000], None, 16, 8, 64, True, "bf16", 0),
    (list(np.random.default_rng(773).integers(0, 4, 4100)), None, 8, 8, 64, True, "bf16", 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{len(c[0])}-{str(c[0][:3])}" for c in CASES])
def test_varlen_parity(case):
    lens_q, lens_k, Hq, Hkv, D, causal, dtype, extra = case
    lens_k = lens_q if lens_k is None else lens_k
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    q, k, v = packed_inputs(int(cu_q[-1]), int(cu_k[-1]), Hq, Hkv, D, dtype, 700 + len(lens_q))
    scale = 1 / math.sqrt(D)
    got = run_varlen(q, k, v, cu_q, cu_k, max(lens_q) + extra, max(lens_k), causal, scale, dtype)
    ref = oracle.varlen_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                            oracle.widen(v, dtype), cu_q, cu_k, causal, scale)
    parity(oracle.widen(got, dtype), ref, f"varlen {case}")


def test_varlen_rows_outside_every_sequence_are_untouched():
    dtype, Hq, Hkv, D = "bf16", 2, 1, 128
    cu_q, cu_k = np.array([50, 150, 400]), np.array([0, 120, 300])
    q, k, v = packed_inputs(480, 300, Hq, Hkv, D, dtype, 731)
    got, lse = run_varlen(q, k, v, cu_q, cu_k, 250, 180, True, 0.1, dtype, lse=True)
    own = owned_rows(cu_q, 480)
    assert np.all(got[~own] == CANARY)
    ref, ref_lse = oracle.varlen_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                                     oracle.widen(v, dtype), cu_q, cu_k, True, 0.1, True)
    parity(oracle.widen(got[own], dtype), ref[own], "varlen with uncovered rows")
    fin = np.isfinite(ref_lse[:, own])
    np.testing.assert_allclose(lse[:, own][fin], ref_lse[:, own][fin], rtol=1e-4, atol=1e-3)


def test_varlen_lse_matches_oracle():
    dtype, Hq, Hkv, D = "bf16", 4, 2, 64
    lens_q, lens_k = [300, 1, 129], [200, 700, 129]
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    q, k, v = packed_inputs(int(cu_q[-1]), int(cu_k[-1]), Hq, Hkv, D, dtype, 741)
    o_bits, lse = run_varlen(q, k, v, cu_q, cu_k, 300, 700, True, 0.125, dtype, lse=True)
    _, ref = oracle.varlen_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), cu_q, cu_k, True, 0.125, True)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.isneginf(lse[~fin]))
    np.testing.assert_allclose(lse[fin], ref[fin], rtol=1e-4, atol=1e-3)
    assert np.array_equal(o_bits, run_varlen(q, k, v, cu_q, cu_k, 300, 700, True, 0.125, dtype))


@pytest.mark.parametrize("causal", [True, False])
def test_equal_length_varlen_is_the_dense_kernel_bitwise(causal):
    # same arithmetic, other layout: B sequences of one length packed token-major
    # give exactly the bits of the dense [B, H, S, D] forward with one
    # workgroup per item (24 items: the automatic dense plan would split the
    # keys, which the varlen path never does)
    import torch
    fa = _fa()
    dtype, B, Hq, Hkv, Sq, Sk, D = "bf16", 3, 4, 2, 300, 520, 128
    qd = wl.normal_bits((B, Hq, Sq, D), 751, dtype)
    kd = wl.normal_bits((B, Hkv, Sk, D), 752, dtype)
    vd = wl.normal_bits((B, Hkv, Sk, D), 753, dtype)
    dense = bits_of(fa.fwd(to_dev(qd, dtype), to_dev(kd, dtype), to_dev(vd, dtype),
                           causal=causal, scale=0.09,
                           schedule=dict(persistent=0, hkv_major=0, xcd_map=0, split_tiles=0)))
    pack = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(-1, x.shape[1], D))
    got = run_varlen(pack(qd), pack(kd), pack(vd), np.arange(B + 1) * Sq, np.arange(B + 1) * Sk,
                     Sq, Sk, causal, 0.09, dtype)
    assert np.array_equal(got, pack(dense))
    del torch


def test_varlen_long_sequences_sampled_rows():
    # long ragged sequences: every row of a few sampled (sequence, head) pairs
    # is checked against the oracle row by row
    dtype, Hq, Hkv, D = "bf16", 16, 2, 128
    lens = [4096, 1000, 8192, 2049]
    cu = offsets(lens)
    q, k, v = packed_inputs(int(cu[-1]), int(cu[-1]), Hq, Hkv, D, dtype, 761)
    got = oracle.widen(run_varlen(q, k, v, cu, cu, max(lens), max(lens), True, 1 / math.sqrt(D),
                                  dtype), dtype)
    qf, kf, vf = oracle.widen(q, dtype), oracle.widen(k, dtype), oracle.widen(v, dtype)
    rng = np.random.default_rng(762)
    for b, h in [(0, 3), (1, 15), (2, 0), (2, 9), (3, 7)]:
        q0, q1 = int(cu[b]), int(cu[b + 1])
        qs = qf[q0:q1].transpose(1, 0, 2)[None]
        ks = kf[q0:q1].transpose(1, 0, 2)[None]
        vs = vf[q0:q1].transpose(1, 0, 2)[None]
        rows = np.unique(np.concatenate([[0, q1 - q0 - 1], rng.integers(0, q1 - q0, 24)]))
        ref = oracle.attention_rows_ref(qs, ks, vs, True, 1 / math.sqrt(D), 0, h, rows)
        parity(got[q0 + rows, h], ref, f"varlen long b={b} h={h}")


@pytest.mark.parametrize("k0", [24.0, 256.0], ids=["rescaled", "overflowed"])
def test_varlen_score_jump_in_mask_free_tile(k0):
    # as the dense test of the same name: in sequences 0 and 2 the key at
    # relative position 700 scores far above the rest for every row and sits
    # in a mask-free tile of the query blocks from row 1024 on; with k0 = 256
    # the exp overflows and the item runs again with the max-first softmax
    dtype, Hq, Hkv, D = "bf16", 4, 2, 128
    lens = [1536, 300, 1400]
    cu = offsets(lens)
    q, k, v = packed_inputs(int(cu[-1]), int(cu[-1]), Hq, Hkv, D, dtype, 771)
    qf, kf = oracle.widen(q, dtype).astype(np.float32), oracle.widen(k, dtype).astype(np.float32)
    qf[:, :, 0] = 8.0
    for b in (0, 2):
        kf[int(cu[b]) + 700, :, 0] = k0
    q, k = wl.to_bits(qf, dtype), wl.to_bits(kf, dtype)
    scale = 1 / math.sqrt(D)
    got = run_varlen(q, k, v, cu, cu, max(lens), max(lens), True, scale, dtype)
    ref = oracle.varlen_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                            oracle.widen(v, dtype), cu, cu, True, scale)
    parity(oracle.widen(got, dtype), ref, f"varlen score jump k0={k0}")


def test_varlen_empty_batch_and_empty_queries():
    import torch
    fa = _fa()
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((10, 1, 64), dtype=torch.bfloat16, device="cuda")
    cu0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert fa.fwd_varlen(q, k, k, cu0, cu0, 0, 0).shape == (0, 2, 64)
    cu = torch.tensor([0, 0, 0], dtype=torch.int32, device="cuda")
    cuk = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda")
    assert fa.fwd_varlen(q, k, k, cu, cuk, 0, 6, causal=True).shape == (0, 2, 64)
