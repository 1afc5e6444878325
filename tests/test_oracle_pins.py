"""Pins for the CPU oracle: it is checked against things other than itself.

Each test states which property of the definition it pins.  Nothing here
needs a GPU.  See oracle/attention.py for the definition being pinned.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------
# widening of storage bits (pinned to fixed bit patterns and to torch's casts)
# ----------------------------------------------------------------------------
def test_widen_fixed_bit_patterns():
    bf = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x3FC0, 0x4049],
                  dtype=np.uint16)
    got = oracle.widen(bf, "bf16")
    want = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 1.5, 3.140625]
    assert got.tolist() == want
    assert math.copysign(1.0, got[3]) == -1.0
    fp = np.array([0x3C00, 0xC000, 0x0001, 0x7BFF, 0x3555], dtype=np.uint16)
    got = oracle.widen(fp, "fp16")
    assert got.tolist() == [1.0, -2.0, 2.0 ** -24, 65504.0, 0.333251953125]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_generator_rounding_matches_torch_cast(dtype):
    x = np.random.default_rng(7).standard_normal(50000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 65519.0]  # ties and near-overflow
    bits = wl.to_bits(x, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    want = torch.from_numpy(x).to(tdt).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.widen(bits, dtype), want)


# ----------------------------------------------------------------------------
# brute force on tiny shapes: pure-Python loops with math.exp
# ----------------------------------------------------------------------------
def brute(q, k, v, causal, scale):
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    o = np.zeros((B, Hq, Sq, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                keys = [j for j in range(Sk) if (not causal) or j <= i + Sk - Sq]
                if not keys:
                    continue
                s = {}
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[b, h, i, d]) * float(k[b, h // g, j, d])
                    s[j] = scale * acc
                mx = max(s.values())
                w = {j: math.exp(s[j] - mx) for j in keys}
                den = sum(w.values())
                for e in range(v.shape[3]):
                    o[b, h, i, e] = sum(w[j] * float(v[b, h // g, j, e]) for j in keys) / den
    return o


TINY_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 1, 1, 5, 5, 3, True),
    (2, 4, 2, 7, 7, 8, True),
    (1, 4, 1, 6, 13, 4, True),    # ragged, bottom-right
    (1, 2, 2, 17, 9, 5, True),    # Sq > Sk: first rows have no key
    (2, 2, 1, 9, 11, 8, False),
    (1, 3, 3, 1, 16, 8, True),    # single row
]


@pytest.mark.parametrize("case", TINY_CASES)
def test_brute_force_tiny(case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = rnd((B, Hq, Sq, D), 1), rnd((B, Hkv, Sk, D), 2), rnd((B, Hkv, Sk, D), 3)
    scale = 0.7 / math.sqrt(D)
    got = oracle.attention_ref(q, k, v, causal, scale, row_chunk=4)
    want = brute(q, k, v, causal, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# an independent library routine: torch's float64 CPU attention
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("case", [(2, 4, 2, 40, 40, 16, True), (1, 6, 3, 23, 71, 32, True),
                                  (1, 2, 1, 64, 48, 64, False), (2, 8, 1, 33, 33, 128, True)])
def test_against_torch_sdpa_float64(case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = rnd((B, Hq, Sq, D), 11), rnd((B, Hkv, Sk, D), 12), rnd((B, Hkv, Sk, D), 13)
    scale = 1.0 / math.sqrt(D)
    got = oracle.attention_ref(q, k, v, causal, scale)
    g = Hq // Hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Sk)[None, :]
    mask = (j <= i + (Sk - Sq)) if causal else torch.ones(Sq, Sk, dtype=torch.bool)
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                            scale=scale).numpy()
    rows_ok = mask.any(dim=1).numpy()
    np.testing.assert_allclose(got[:, :, rows_ok], want[:, :, rows_ok], rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Sq,Sk", [(37, 37), (20, 50)])
def test_identical_keys_give_prefix_mean(Sq, Sk):
    D = 8
    q = rnd((1, 2, Sq, D), 21)
    krow = rnd((D,), 22)
    k = np.broadcast_to(krow, (1, 1, Sk, D)).copy()
    v = rnd((1, 1, Sk, D), 23)
    got = oracle.attention_ref(q, k, v, True, 0.3)
    csum = np.cumsum(v[0, 0], axis=0)
    for i in range(Sq):
        last = i + Sk - Sq
        want = csum[last] / (last + 1)
        np.testing.assert_allclose(got[0, :, i], np.broadcast_to(want, (2, D)), atol=1e-12)
    # non-causal: the plain mean of all rows
    got = oracle.attention_ref(q, k, v, False, 0.3)
    np.testing.assert_allclose(got[0, 0], np.broadcast_to(v[0, 0].mean(0), (Sq, D)), atol=1e-12)


def test_one_hot_dominant_key():
    # query i points along axis i; only key j*(i) <= i has a component there,
    # so s_{i,j*} = 60 and every other admissible score is 0 (gap 60 nats)
    S = 64
    rng = np.random.default_rng(31)
    jstars = [(i * 5 + 3) % (i + 1) for i in range(S)]
    qa = 60.0 * np.eye(S)
    ka = np.zeros((S, S))
    for i, js in enumerate(jstars):
        ka[js, i] = 1.0
    vv = rng.standard_normal((1, 1, S, 8))
    got = oracle.attention_ref(qa[None, None], ka[None, None], vv, True, 1.0)
    for i, js in enumerate(jstars):
        np.testing.assert_allclose(got[0, 0, i], vv[0, 0, js], atol=1e-12)


def test_causal_row0_is_v0_exactly():
    q, k, v = rnd((2, 4, 19, 8), 41), rnd((2, 2, 19, 8), 42), rnd((2, 2, 19, 8), 43)
    got = oracle.attention_ref(q, k, v, True, 0.5)
    for h in range(4):
        assert np.array_equal(got[:, h, 0], v[:, h // 2, 0])


def test_probability_rows_sum_to_one_and_constant_v():
    q, k = rnd((9, 8), 51), rnd((30, 8), 52)
    allowed = oracle.admissible_mask(9, 30, True)
    p = oracle.probs_ref(q, k, allowed, 0.4)
    assert np.all(p >= 0)
    assert np.all(p[~allowed] == 0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    v = np.ones((1, 1, 30, 4))
    o = oracle.attention_ref(q[None, None], k[None, None], v, True, 0.4)
    np.testing.assert_allclose(o, 1.0, atol=1e-15)


def test_rows_without_keys_are_zero():
    q, k, v = rnd((1, 1, 10, 4), 61), rnd((1, 1, 4, 4), 62), rnd((1, 1, 4, 4), 63)
    o = oracle.attention_ref(q, k, v, True, 1.0)
    # j <= i + (4 - 10): rows 0..5 admit nothing
    assert np.all(o[0, 0, :6] == 0)
    assert np.all(np.any(o[0, 0, 6:] != 0, axis=1))


def test_scale_enters_as_temperature():
    # scale -> 0 turns every admissible row into the uniform mean of V
    q, k, v = rnd((1, 1, 12, 4), 71), rnd((1, 1, 12, 4), 72), rnd((1, 1, 12, 4), 73)
    o = oracle.attention_ref(q, k, v, True, 0.0)
    csum = np.cumsum(v[0, 0], axis=0) / np.arange(1, 13)[:, None]
    np.testing.assert_allclose(o[0, 0], csum, atol=1e-12)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_gqa_equals_mha_with_repeated_heads():
    B, Hq, Hkv, S, D = 2, 8, 2, 21, 16
    q, k, v = rnd((B, Hq, S, D), 81), rnd((B, Hkv, S, D), 82), rnd((B, Hkv, S, D), 83)
    g = oracle.attention_ref(q, k, v, True, 0.25)
    m = oracle.attention_ref(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1),
                             True, 0.25)
    assert np.array_equal(g, m)
    # and the grouping is contiguous (head h reads kv head h // 4), not strided
    wrong = oracle.attention_ref(q, np.tile(k, (1, Hq // Hkv, 1, 1)),
                                 np.tile(v, (1, Hq // Hkv, 1, 1)), True, 0.25)
    assert not np.allclose(g, wrong)


def test_rows_subset_matches_full():
    q, k, v = rnd((1, 4, 50, 8), 91), rnd((1, 2, 70, 8), 92), rnd((1, 2, 70, 8), 93)
    full = oracle.attention_ref(q, k, v, True, 0.3)
    rows = [0, 3, 17, 49]
    for h in range(4):
        np.testing.assert_array_equal(oracle.attention_rows_ref(q, k, v, True, 0.3, 0, h, rows),
                                      full[0, h, rows])


def test_decode_equals_last_prefill_row_and_ignores_tail():
    B, Hq, Hkv, D, cap = 2, 8, 2, 16, 40
    rng = np.random.default_rng(101)
    kc = rng.standard_normal((B, cap, Hkv, D))
    vc = rng.standard_normal((B, cap, Hkv, D))
    q = rng.standard_normal((B, Hq, D))
    L = np.array([17, 40])
    kc_nan, vc_nan = kc.copy(), vc.copy()
    kc_nan[0, 17:] = np.nan
    vc_nan[0, 17:] = np.nan
    got = oracle.decode_ref(q, kc_nan, vc_nan, L, 0.2)
    assert np.all(np.isfinite(got))
    for b in range(B):
        Lb = int(L[b])
        kk = np.transpose(kc[b:b + 1, :Lb], (0, 2, 1, 3))  # [1, Hkv, L, D]
        vv = np.transpose(vc[b:b + 1, :Lb], (0, 2, 1, 3))
        # non-causal prefill over L keys with one query row
        pre = oracle.attention_ref(q[b:b + 1, :, None, :], kk, vv, False, 0.2)[0, :, 0]
        np.testing.assert_allclose(got[b], pre, atol=1e-13)
        # last row of a causal prefill whose queries are arbitrary but end with q
        qq = rng.standard_normal((1, Hq, Lb, D))
        qq[0, :, -1] = q[b]
        pre2 = oracle.attention_ref(qq, kk, vv, True, 0.2)[0, :, -1]
        np.testing.assert_allclose(got[b], pre2, atol=1e-13)


def test_decode_valid_len_clamped():
    rng = np.random.default_rng(111)
    kc, vc = rng.standard_normal((1, 8, 1, 4)), rng.standard_normal((1, 8, 1, 4))
    q = rng.standard_normal((1, 2, 4))
    assert np.all(oracle.decode_ref(q, kc, vc, [0], 1.0) == 0)
    assert np.all(oracle.decode_ref(q, kc, vc, [-5], 1.0) == 0)
    np.testing.assert_array_equal(oracle.decode_ref(q, kc, vc, [99], 1.0),
                                  oracle.decode_ref(q, kc, vc, [8], 1.0))


def test_split_merge_identity():
    rng = np.random.default_rng(121)
    R, S, D = 5, 97, 8
    q, k, v = rng.standard_normal((R, D)), rng.standard_normal((S, D)), rng.standard_normal((S, D))
    full = oracle.probs_ref(q, k, np.ones((R, S), bool), 0.9) @ v
    for trial in range(20):
        cuts = np.sort(rng.integers(0, S + 1, size=rng.integers(1, 9)))
        edges = [0] + cuts.tolist() + [S]      # repeated cuts give empty chunks
        parts = [oracle.partial_ref(q, k[a:b], v[a:b], 0.9) for a, b in zip(edges[:-1], edges[1:])]
        np.testing.assert_allclose(oracle.merge_ref(parts), full, atol=1e-13)
    empty = [oracle.partial_ref(q, k[:0], v[:0], 0.9)] * 3
    assert np.all(oracle.merge_ref(empty) == 0)


def test_lse_against_brute_force_and_torch():
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 7, 11, 4
    q, k = rnd((B, Hq, Sq, D), 131), rnd((B, Hkv, Sk, D), 132)
    got = oracle.lse_ref(q, k, True, 0.6)
    for h in range(Hq):
        for i in range(Sq):
            keys = [j for j in range(Sk) if j <= i + Sk - Sq]
            want = math.log(sum(math.exp(0.6 * float(np.dot(q[0, h, i], k[0, 0, j])))
                                for j in keys))
            assert abs(got[0, h, i] - want) < 1e-12
    s = 0.6 * torch.from_numpy(q[0]) @ torch.from_numpy(k[0, 0]).T
    mask = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + (Sk - Sq)
    want = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1).numpy()
    np.testing.assert_allclose(got[0], want, atol=1e-12)
    # empty rows are -inf
    q2, k2 = rnd((1, 1, 6, 4), 133), rnd((1, 1, 2, 4), 134)
    l2 = oracle.lse_ref(q2, k2, True, 1.0)
    assert np.all(np.isneginf(l2[0, 0, :4])) and np.all(np.isfinite(l2[0, 0, 4:]))


# ----------------------------------------------------------------------------
# packed variable-length batches
# ----------------------------------------------------------------------------
def _pack(x):
    """[B, H, S, D] -> [B*S, H, D] (sequences back to back)."""
    B, H, S, D = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * S, H, D)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_is_the_dense_batch(causal):
    B, Hq, Hkv, Sq, Sk, D = 3, 4, 2, 9, 13, 8
    q, k, v = rnd((B, Hq, Sq, D), 141), rnd((B, Hkv, Sk, D), 142), rnd((B, Hkv, Sk, D), 143)
    cu_q, cu_k = np.arange(B + 1) * Sq, np.arange(B + 1) * Sk
    got, lse = oracle.varlen_ref(_pack(q), _pack(k), _pack(v), cu_q, cu_k, causal, 0.4, True)
    np.testing.assert_allclose(got, _pack(oracle.attention_ref(q, k, v, causal, 0.4)), atol=1e-12)
    want_lse = oracle.lse_ref(q, k, causal, 0.4)  # [B, Hq, Sq]
    np.testing.assert_allclose(lse, want_lse.transpose(1, 0, 2).reshape(Hq, B * Sq), atol=1e-12)


def test_varlen_ragged_against_brute_force():
    # lengths 3/0/5 queries against 4/2/6 keys, rows 8..9 belong to no sequence
    Hq, Hkv, D = 2, 1, 3
    cu_q, cu_k = np.array([0, 3, 3, 8]), np.array([0, 4, 6, 12])
    q, k, v = rnd((10, Hq, D), 144), rnd((12, Hkv, D), 145), rnd((12, Hkv, D), 146)
    for causal in (False, True):
        got = oracle.varlen_ref(q, k, v, cu_q, cu_k, causal, 0.7)
        for b in range(3):
            q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
            want = brute(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                         v[k0:k1].transpose(1, 0, 2)[None], causal, 0.7)[0].transpose(1, 0, 2)
            np.testing.assert_allclose(got[q0:q1], want, atol=1e-12)
        assert np.all(np.isnan(got[8:]))


def test_varlen_sequences_do_not_mix():
    Hq, Hkv, D = 2, 2, 4
    cu_q, cu_k = np.array([0, 5, 12]), np.array([0, 7, 10])
    q, k, v = rnd((12, Hq, D), 147), rnd((10, Hkv, D), 148), rnd((10, Hkv, D), 149)
    base = oracle.varlen_ref(q, k, v, cu_q, cu_k, True, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[7:] += 3.0
    v2[7:] -= 2.0
    other = oracle.varlen_ref(q, k2, v2, cu_q, cu_k, True, 0.5)
    np.testing.assert_array_equal(base[:5], other[:5])   # sequence 0 untouched
    assert not np.allclose(base[5:], other[5:])           # sequence 1 sees its own keys
    # swapping the two sequences swaps the outputs
    qs = np.concatenate([q[5:], q[:5]])
    ks, vs = np.concatenate([k[7:], k[:7]]), np.concatenate([v[7:], v[:7]])
    sw = oracle.varlen_ref(qs, ks, vs, np.array([0, 7, 12]), np.array([0, 3, 10]), True, 0.5)
    np.testing.assert_allclose(sw[:7], base[5:], atol=1e-12)
    np.testing.assert_allclose(sw[7:], base[:5], atol=1e-12)


# ----------------------------------------------------------------------------
# the pages' own reproduction case (decode review): NaN tail, L = 1 -> V[0]
# ----------------------------------------------------------------------------
def test_golden_decode_nan_tail_case():
    g = json.load(open(os.path.join(GOLDEN, "decode_nan_tail.json")))
    s = wl.DecodeShape("golden", g["B"], g["Hq"], g["Hkv"], g["D"], g["capacity"])
    kc, vc = wl.decode_cache(s, g["valid_len"], tail_bits=g["tail_bits"])
    q = wl.decode_query(s, 77)
    kf, vf, qf = oracle.widen(kc, "bf16"), oracle.widen(vc, "bf16"), oracle.widen(q, "bf16")
    assert np.isnan(vf[0, g["valid_len"]:]).all()
    o = oracle.decode_ref(qf, kf, vf, [g["valid_len"]], s.scale)
    gqa = g["Hq"] // g["Hkv"]
    for h in range(g["Hq"]):
        assert np.array_equal(o[0, h], vf[0, 0, h // gqa])


# ----------------------------------------------------------------------------
# the pins catch plausible mistakes planted in the oracle
# ----------------------------------------------------------------------------
MUTATIONS = [
    ("j <= (rows[:, None] + (Sk - Sq))", "j <= rows[:, None]"),          # top-left causal
    ("j <= (rows[:, None] + (Sk - Sq))", "j < (rows[:, None] + (Sk - Sq))"),  # off by one
    ("s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),                # dropped scale
    ("hk = h // gqa", "hk = h % Hkv"),                                   # strided GQA
    ("    if not causal:\n        return np.ones", "    if causal:\n        return np.ones"),  # mask off
    ("den = w.sum(axis=1, keepdims=True)", "den = w.sum(axis=0, keepdims=True)"),  # wrong axis
    ("out[b, h, rows] = p @ v[b, hk]", "out[b, h, rows] = p @ k[b, hk]"),  # wrong operand
    ("return np.where(empty, 0.0, w / np.where(empty, 1.0, den))", "return w"),  # no normaliser
]


def _mutant(src_from, src_to):
    path = os.path.join(os.path.dirname(oracle.__file__), "attention.py")
    src = open(path).read()
    assert src_from in src, src_from
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(src_from, src_to, 1), "oracle_mutant", "exec"), ns)
    return ns


def _pins_pass(ns):
    """A compact rerun of the brute-force and closed-form pins on a mutant."""
    try:
        for case in TINY_CASES[:5]:
            B, Hq, Hkv, Sq, Sk, D, causal = case
            q, k, v = rnd((B, Hq, Sq, D), 1), rnd((B, Hkv, Sk, D), 2), rnd((B, Hkv, Sk, D), 3)
            scale = 0.7 / math.sqrt(D)
            got = ns["attention_ref"](q, k, v, causal, scale, row_chunk=4)
            if not np.allclose(got, brute(q, k, v, causal, scale), atol=1e-12, rtol=0):
                return False
        return True
    except Exception:
        return False


def test_unmutated_oracle_passes_compact_pins():
    assert _pins_pass(_mutant("", ""))


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m[1][:30] for m in MUTATIONS])
def test_planted_mistake_is_caught(mutation):
    assert not _pins_pass(_mutant(*mutation))


VARLEN_MUTATIONS = [
    ("k0, k1 = int(cu_k[b]), int(cu_k[b + 1])", "k0, k1 = int(cu_q[b]), int(cu_q[b + 1])"),
    ("qs = q[q0:q1].transpose(1, 0, 2)[None]",
     "qs = q[q0:q1].reshape(1, q.shape[1], q1 - q0, -1)"),             # token/head mix-up
    ("vs = v[k0:k1].transpose(1, 0, 2)[None]", "vs = k[k0:k1].transpose(1, 0, 2)[None]"),
    ("for b in range(len(cu_q) - 1):", "for b in range(len(cu_q) - 2):"),  # last sequence lost
]


def _varlen_pins_pass(ns):
    """The ragged brute-force pin, rerun on a mutant."""
    try:
        Hq, Hkv, D = 2, 1, 3
        cu_q, cu_k = np.array([0, 3, 3, 8]), np.array([0, 4, 6, 12])
        q, k, v = rnd((8, Hq, D), 144), rnd((12, Hkv, D), 145), rnd((12, Hkv, D), 146)
        for causal in (False, True):
            got = ns["varlen_ref"](q, k, v, cu_q, cu_k, causal, 0.7)
            for b in range(3):
                q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
                want = brute(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                             v[k0:k1].transpose(1, 0, 2)[None], causal, 0.7)[0].transpose(1, 0, 2)
                if not np.allclose(got[q0:q1], want, atol=1e-12, rtol=0):
                    return False
        return True
    except Exception:
        return False


def test_unmutated_varlen_oracle_passes_its_pin():
    assert _varlen_pins_pass(_mutant("", ""))


@pytest.mark.parametrize("mutation", VARLEN_MUTATIONS, ids=[m[1][:30] for m in VARLEN_MUTATIONS])
def test_planted_varlen_mistake_is_caught(mutation):
    assert not _varlen_pins_pass(_mutant(*mutation))


# ----------------------------------------------------------------------------
# paged decode cache
# ----------------------------------------------------------------------------
def test_paged_decode_against_brute_force():
    # token t of batch b: row t % P of page table[b, t // P]; every step spelled out
    B, Hq, Hkv, D, P, pps, npages = 2, 4, 2, 3, 4, 3, 7
    q = rnd((B, Hq, D), 151)
    kp, vp = rnd((npages, P, Hkv, D), 152), rnd((npages, P, Hkv, D), 153)
    table = np.array([[5, 0, 3], [2, 6, 1]])
    L = [10, 5]
    got = oracle.decode_paged_ref(q, kp, vp, table, L, 0.8)
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            toks = [(table[b][t // P], t % P) for t in range(L[b])]
            s = [0.8 * sum(float(q[b, h, d]) * float(kp[pg, r, hk, d]) for d in range(D))
                 for pg, r in toks]
            mx = max(s)
            w = [math.exp(x - mx) for x in s]
            for e in range(D):
                want = sum(wi * float(vp[pg, r, hk, e]) for wi, (pg, r) in zip(w, toks)) / sum(w)
                assert abs(got[b, h, e] - want) < 1e-12


def test_paged_decode_identity_and_shuffled_pools_match_contiguous():
    B, Hq, Hkv, D, P, pps = 2, 8, 2, 16, 32, 4
    cap = P * pps
    q = rnd((B, Hq, D), 154)
    kc, vc = rnd((B, cap, Hkv, D), 155), rnd((B, cap, Hkv, D), 156)
    L = [cap - 7, 33]
    want = oracle.decode_ref(q, kc, vc, L, 0.3)
    # identity: batch b's pages are pool pages b*pps .. b*pps+pps-1
    kp, vp = kc.reshape(B * pps, P, Hkv, D), vc.reshape(B * pps, P, Hkv, D)
    ident = np.arange(B * pps).reshape(B, pps)
    np.testing.assert_allclose(oracle.decode_paged_ref(q, kp, vp, ident, L, 0.3), want, atol=1e-12)
    # the same pages shuffled inside a larger pool, unused pages NaN
    perm = np.random.default_rng(157).permutation(3 * B * pps)[:B * pps]
    kbig = np.full((3 * B * pps, P, Hkv, D), np.nan)
    vbig = np.full((3 * B * pps, P, Hkv, D), np.nan)
    kbig[perm], vbig[perm] = kp, vp
    got = oracle.decode_paged_ref(q, kbig, vbig, perm.reshape(B, pps), L, 0.3)
    np.testing.assert_allclose(got, want, atol=1e-12)


# ----------------------------------------------------------------------------
# multi-token decode
# ----------------------------------------------------------------------------
def test_multi_token_decode_is_the_last_rows_of_causal_prefill():
    # Sq new tokens at the end of L: the last Sq rows of causal self-attention
    # over the L tokens, whose queries are the new tokens' queries
    B, Hq, Hkv, D, cap, Sq = 2, 4, 2, 6, 40, 5
    kc, vc = rnd((B, cap, Hkv, D), 161), rnd((B, cap, Hkv, D), 162)
    L = [37, 9]
    qn = rnd((B, Sq, Hq, D), 163)
    got = oracle.decode_multi_ref(qn, kc, vc, L, True, 0.45)
    for b in range(B):
        qfull = rnd((1, Hq, L[b], D), 164 + b)
        qfull[0, :, L[b] - Sq:] = qn[b].transpose(1, 0, 2)
        full = oracle.attention_ref(qfull, kc[b:b + 1, :L[b]].transpose(0, 2, 1, 3),
                                    vc[b:b + 1, :L[b]].transpose(0, 2, 1, 3), True, 0.45)
        np.testing.assert_allclose(got[b], full[0, :, L[b] - Sq:].transpose(1, 0, 2), atol=1e-12)
    # without the mask every token sees all L keys: each token is a plain decode
    got_nc = oracle.decode_multi_ref(qn, kc, vc, L, False, 0.45)
    for t in range(Sq):
        np.testing.assert_allclose(got_nc[:, t], oracle.decode_ref(qn[:, t], kc, vc, L, 0.45),
                                   atol=1e-12)


def test_multi_token_decode_brute_force_and_short_sequences():
    B, Hq, Hkv, D, cap, Sq = 1, 2, 1, 3, 8, 4
    kc, vc = rnd((B, cap, Hkv, D), 171), rnd((B, cap, Hkv, D), 172)
    qn = rnd((B, Sq, Hq, D), 173)
    for L in (6, 2, 0):
        got = oracle.decode_multi_ref(qn, kc, vc, [L], True, 0.9)
        for t in range(Sq):
            keys = list(range(0, L - Sq + t + 1))
            for h in range(Hq):
                if not keys:
                    assert np.all(got[0, t, h] == 0.0)
                    continue
                s = [0.9 * float(np.dot(qn[0, t, h], kc[0, j, 0])) for j in keys]
                w = [math.exp(x - max(s)) for x in s]
                want = sum(wi * vc[0, j, 0] for wi, j in zip(w, keys)) / sum(w)
                np.testing.assert_allclose(got[0, t, h], want, atol=1e-12)


# ----------------------------------------------------------------------------
# backward pass
# ----------------------------------------------------------------------------
BWD_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 2, 1, 5, 5, 4, True),
    (2, 2, 2, 4, 7, 3, True),     # bottom-right, Sq < Sk
    (1, 4, 2, 6, 3, 4, True),     # Sq > Sk: rows without keys
    (1, 2, 1, 5, 6, 4, False),
]


def _loss_and_grads(case, seed):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = rnd((B, Hq, Sq, D), seed), rnd((B, Hkv, Sk, D), seed + 1), rnd((B, Hkv, Sk, D), seed + 2)
    g = rnd((B, Hq, Sq, D), seed + 3)  # dO: the loss is sum(O * g)
    return q, k, v, g, causal


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_backward_against_finite_differences(case):
    q, k, v, g, causal = _loss_and_grads(case, 181)
    scale = 0.6
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, g, causal, scale)
    loss = lambda q_, k_, v_: float(np.sum(oracle.attention_ref(q_, k_, v_, causal, scale) * g))
    eps = 1e-6
    rng = np.random.default_rng(182)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_backward_against_torch_autograd_float64(case):
    q, k, v, g, causal = _loss_and_grads(case, 191)
    B, Hq, Hkv, Sq, Sk, D, _ = case
    scale = 0.45
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, g, causal, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * tq @ kk.transpose(-1, -2)
    mask = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + (Sk - Sq)
    if causal:
        s = s.masked_fill(~mask, -math.inf)
    p = torch.softmax(s, dim=-1).nan_to_num(0.0)  # rows without keys: 0
    (p @ vv * torch.tensor(g)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


BWD_MUTATIONS = [
    ("ds = p * (dp - dr)", "ds = p * dp"),                               # dropped D term
    ("dv[b, hk] += p.T @ do[b, h]", "dv[b, hk] += p @ do[b, h]"),        # transposed P
    ("dq[b, h] = scale * (ds @ k[b, hk])", "dq[b, h] = (ds @ k[b, hk])"),  # dropped scale
    ("dk[b, hk] += scale * (ds.T @ q[b, h])", "dk[b, hk] = scale * (ds.T @ q[b, h])"),  # GQA sum lost
]


def _bwd_pins_pass(ns):
    """Finite differences of sum(O * g) on two tiny cases, rerun on a mutant."""
    try:
        for case in (BWD_CASES[0], (1, 4, 2, 5, 5, 3, True)):
            q, k, v, g, causal = _loss_and_grads(case, 201)
            dq, dk, dv = ns["attention_bwd_ref"](q, k, v, g, causal, 0.6)
            loss = lambda q_, k_, v_: float(np.sum(ns["attention_ref"](q_, k_, v_, causal, 0.6) * g))
            for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
                it = np.nditer(x, flags=["multi_index"])
                for _ in it:
                    idx = it.multi_index
                    xp, xm = x.copy(), x.copy()
                    xp[idx] += 1e-6
                    xm[idx] -= 1e-6
                    args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
                    args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
                    fd = (loss(*args_p) - loss(*args_m)) / 2e-6
                    if abs(fd - grad[idx]) > 1e-6 * max(1.0, abs(fd)):
                        return False
        return True
    except Exception:
        return False


def test_unmutated_backward_oracle_passes_its_pin():
    assert _bwd_pins_pass(_mutant("", ""))


@pytest.mark.parametrize("mutation", BWD_MUTATIONS, ids=[m[1][:30] for m in BWD_MUTATIONS])
def test_planted_backward_mistake_is_caught(mutation):
    assert not _bwd_pins_pass(_mutant(*mutation))


def test_backward_dq_rows_match_the_full_backward():
    q, k, v, g, causal = _loss_and_grads((2, 4, 2, 9, 12, 5, True), 211)
    dq, _, _ = oracle.attention_bwd_ref(q, k, v, g, causal, 0.5)
    rows = [0, 3, 8]
    for b in range(2):
        for h in range(4):
            got = oracle.attention_bwd_dq_rows_ref(q, k, v, g, causal, 0.5, b, h, rows)
            np.testing.assert_allclose(got, dq[b, h, rows], atol=1e-12)
