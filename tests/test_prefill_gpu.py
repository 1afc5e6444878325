"""GPU parity of the dense forward (fa_fwd through the C ABI) against the
CPU float64 oracle, plus the bitwise mask semantics.

Bound: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise on bf16/fp16 outputs.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bits_of, parity, to_dev

pytestmark = pytest.mark.gpu


def _fa():
    import flash_attention_forward_fwd_amd as fa
    return fa


def run_fwd(q, k, v, causal, scale, dtype, lse=False):
    fa = _fa()
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    if lse:
        o, l = fa.fwd(tq, tk, tv, causal=causal, scale=scale, return_lse=True)
        return bits_of(o), l.cpu().numpy().astype(np.float64)
    return bits_of(fa.fwd(tq, tk, tv, causal=causal, scale=scale))


def shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed, magnitude=1.0):
    q = wl.normal_bits((B, Hq, Sq, D), seed, dtype, magnitude)
    k = wl.normal_bits((B, Hkv, Sk, D), seed + 1, dtype, magnitude)
    v = wl.normal_bits((B, Hkv, Sk, D), seed + 2, dtype)
    return q, k, v


# ----------------------------------------------------------------------------
# full-output parity at sizes the oracle finishes in seconds: several tiles,
# ragged tails, GQA, Sq != Sk both ways, both dtypes and head dims
# ----------------------------------------------------------------------------
SMALL = [
    # B, Hq, Hkv, Sq, Sk, D, causal, dtype
    (1, 2, 1, 256, 256, 64, True, "bf16"),       # the tiny causal GQA workload
    (1, 4, 2, 300, 300, 128, True, "bf16"),
    (2, 4, 1, 257, 700, 64, True, "bf16"),       # bottom-right, ragged
    (1, 2, 2, 129, 65, 128, False, "bf16"),
    (1, 8, 2, 700, 300, 128, True, "bf16"),      # Sq > Sk: 400 rows without keys
    (1, 3, 3, 511, 513, 128, False, "fp16"),
    (2, 4, 4, 333, 333, 64, True, "fp16"),
    (1, 16, 1, 65, 1000, 128, True, "bf16"),     # gqa 16
    (1, 2, 1, 1, 77, 128, True, "bf16"),         # one query row
    (1, 2, 1, 1000, 1, 64, True, "bf16"),        # one key
]


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_small_full_parity(case):
    B, Hq, Hkv, Sq, Sk, D, causal, dtype = case
    print(f"\n[prefill] {case}", flush=True)
    q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=200 + 10 * SMALL.index(case))
    scale = 1.0 / math.sqrt(D)
    got = oracle.widen(run_fwd(q, k, v, causal, scale, dtype), dtype)
    ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), causal, scale)
    st = parity(got, ref, str(case))
    print(f"  {st}", flush=True)
    if causal and Sq > Sk:
        assert np.all(got[:, :, :Sq - Sk] == 0)


def test_tiny_config_exact_workload():
    s = wl.TINY
    print(f"\n[prefill] {s.name}", flush=True)
    q, k, v = wl.prefill_inputs(s)
    got = oracle.widen(run_fwd(q, k, v, s.causal, s.scale, s.dtype), s.dtype)
    ref = oracle.attention_ref(oracle.widen(q, s.dtype), oracle.widen(k, s.dtype),
                               oracle.widen(v, s.dtype), s.causal, s.scale)
    parity(got, ref, s.name)


# ----------------------------------------------------------------------------
# the pages' workloads at full size, checked on sampled rows (the oracle
# computes each sampled row on its own), in the launch configuration the
# benchmark times
# ----------------------------------------------------------------------------
def sample_rows(Sq, rng, n=48):
    fixed = {0, 1, 31, 32, 63, 64, 255, 256, 257, Sq - 1, Sq - 2, Sq // 2}
    rows = sorted({r for r in fixed if 0 <= r < Sq} | set(rng.integers(0, Sq, n).tolist()))
    return np.array(rows)


FULL = [wl.MHA_CAUSAL, wl.MHA_FULL, wl.MHA_FP16, wl.GQA_D128, wl.GQA_D64, wl.RAGGED_D128,
        wl.RAGGED_D64, wl.HEADLINE] + list(wl.SWEEP)


@pytest.mark.parametrize("s", FULL, ids=[s.name for s in FULL])
def test_workload_sampled_parity(s):
    print(f"\n[prefill] {s.name}", flush=True)
    q, k, v = wl.prefill_inputs(s)
    got_bits = run_fwd(q, k, v, s.causal, s.scale, s.dtype)
    rng = np.random.default_rng(s.seed_base + 7)
    qf, kf, vf = oracle.widen(q, s.dtype), oracle.widen(k, s.dtype), oracle.widen(v, s.dtype)
    heads = sorted({0, s.Hq - 1} | set(rng.integers(0, s.Hq, 3).tolist()))
    worst = 0.0
    for b in sorted({0, s.B - 1}):
        for h in heads:
            rows = sample_rows(s.Sq, rng)
            ref = oracle.attention_rows_ref(qf, kf, vf, s.causal, s.scale, b, h, rows)
            got = oracle.widen(got_bits[b, h, rows], s.dtype)
            worst = max(worst, parity(got, ref, f"{s.name} b{b} h{h}")["worst_frac_of_bound"])
    # every output is finite
    assert np.all(np.isfinite(oracle.widen(got_bits, s.dtype)))
    print(f"  worst fraction of bound {worst:.3f}", flush=True)


# ----------------------------------------------------------------------------
# degenerate and special cases
# ----------------------------------------------------------------------------
def test_empty_keys_give_zero_and_empty_queries_are_noop():
    fa = _fa()
    import torch
    q = torch.randn(1, 2, 70, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 1, 0, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, float("nan"))
    for causal in (False, True):
        fa.fwd(q, k, k, causal=causal, out=o)
        torch.cuda.synchronize()
        assert bool((o == 0).all())
    q0 = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.bfloat16)
    k1 = torch.randn(1, 1, 5, 64, device="cuda").to(torch.bfloat16)
    assert fa.fwd(q0, k1, k1, causal=True).shape == (1, 2, 0, 64)


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.37])
def test_zero_and_negative_scale(scale):
    dtype = "bf16"
    q, k, v = shape_inputs(1, 2, 1, 200, 260, 128, dtype, seed=91)
    got = oracle.widen(run_fwd(q, k, v, True, scale, dtype), dtype)
    ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), True, scale)
    parity(got, ref, f"scale={scale}")


@pytest.mark.parametrize("magnitude", [8.0, 64.0])
def test_large_magnitude_inputs_stay_finite(magnitude):
    dtype = "bf16"
    q, k, v = shape_inputs(1, 2, 2, 300, 300, 128, dtype, seed=92, magnitude=magnitude)
    got = oracle.widen(run_fwd(q, k, v, True, 1 / math.sqrt(128), dtype), dtype)
    assert np.all(np.isfinite(got))
    ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), True, 1 / math.sqrt(128))
    parity(got, ref, f"magnitude={magnitude}")


def test_identical_keys_prefix_mean():
    dtype = "bf16"
    B, H, S, D = 1, 2, 520, 128
    q = wl.normal_bits((B, H, S, D), 93, dtype)
    krow = wl.normal_bits((D,), 94, dtype)
    k = np.broadcast_to(krow, (B, 1, S, D)).copy()
    v = wl.normal_bits((B, 1, S, D), 95, dtype)
    got = oracle.widen(run_fwd(q, k, v, True, 0.1, dtype), dtype)
    vf = oracle.widen(v, dtype)[0, 0]
    pref = np.cumsum(vf, axis=0) / np.arange(1, S + 1)[:, None]
    parity(got[0, 0], pref, "prefix mean")
    parity(got[0, 1], pref, "prefix mean")


def test_causal_row0_equals_v0_bitwise():
    dtype = "bf16"
    q, k, v = shape_inputs(2, 4, 2, 300, 300, 128, dtype, seed=96)
    got = run_fwd(q, k, v, True, 0.088, dtype)
    for h in range(4):
        assert np.array_equal(got[:, h, 0], v[:, h // 2, 0])


def test_dominant_key_in_late_tile():
    # row i's dominant key sits in the last KV tile it can see: the running max
    # must be raised late and the accumulator rescaled
    dtype = "bf16"
    S, D = 512, 128
    rng = np.random.default_rng(97)
    qf = rng.standard_normal((1, 1, S, D)).astype(np.float32) * 0.05
    kf = rng.standard_normal((1, 1, S, D)).astype(np.float32) * 0.05
    qf[0, 0, :, 0] = 4.0
    kf[0, 0, S - 1, 0] = 4.0   # dominant for the last row only ...
    kf[0, 0, ::64, 1] = 3.0    # ... and a ladder of rising keys, one per tile
    qf[0, 0, :, 1] = np.linspace(0.5, 3.0, S)
    q, k = wl.to_bits(qf, dtype), wl.to_bits(kf, dtype)
    v = wl.normal_bits((1, 1, S, D), 98, dtype)
    got = oracle.widen(run_fwd(q, k, v, True, 1.0, dtype), dtype)
    ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), True, 1.0)
    parity(got, ref, "late dominant key")


def test_max_rising_below_rescale_threshold():
    # one "ladder" key per 64-key tile whose score rises by 4 log2 units per
    # tile: a row's running max keeps rising by less than the kernel's rescale
    # threshold, so the exp2 reference lags the true max on some tiles (p > 1)
    # and moves on others; every row mixes several ladder keys with weights
    # 2^-4, 2^-8, ...
    dtype = "bf16"
    S, D = 520, 128
    rng = np.random.default_rng(100)
    qf = rng.standard_normal((1, 2, S, D)).astype(np.float32) * 0.05
    kf = rng.standard_normal((1, 1, S, D)).astype(np.float32) * 0.05
    qf[0, :, :, 1] = 1.0
    kf[0, 0, ::64, 1] = 4.0 * math.log(2.0) * np.arange(0, S, 64) / 64
    q, k = wl.to_bits(qf, dtype), wl.to_bits(kf, dtype)
    v = wl.normal_bits((1, 1, S, D), 101, dtype)
    for causal in (True, False):
        got = oracle.widen(run_fwd(q, k, v, causal, 1.0, dtype), dtype)
        ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                                   oracle.widen(v, dtype), causal, 1.0)
        parity(got, ref, f"rising max below threshold, causal={causal}")


def test_lse_matches_oracle():
    dtype = "bf16"
    for (B, Hq, Hkv, Sq, Sk, D, causal) in [(1, 4, 2, 300, 300, 128, True),
                                            (2, 2, 1, 700, 200, 64, True),
                                            (1, 2, 2, 129, 513, 128, False)]:
        q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=99 + Sq)
        scale = 1 / math.sqrt(D)
        o_bits, lse = run_fwd(q, k, v, causal, scale, dtype, lse=True)
        ref = oracle.lse_ref(oracle.widen(q, dtype), oracle.widen(k, dtype), causal, scale)
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.all(np.isneginf(lse[~fin]))
        np.testing.assert_allclose(lse[fin], ref[fin], rtol=1e-4, atol=1e-3)
        o_plain = run_fwd(q, k, v, causal, scale, dtype)
        assert np.array_equal(o_bits, o_plain)


# ----------------------------------------------------------------------------
# bitwise semantics: determinism, GQA == MHA, masked-region independence,
# guard bands around every buffer
# ----------------------------------------------------------------------------
def test_deterministic_and_gqa_equals_mha_bitwise():
    dtype = "bf16"
    B, Hq, Hkv, S, D = 1, 8, 2, 600, 128
    q, k, v = shape_inputs(B, Hq, Hkv, S, S, D, dtype, seed=101)
    a = run_fwd(q, k, v, True, 0.088, dtype)
    b = run_fwd(q, k, v, True, 0.088, dtype)
    assert np.array_equal(a, b)
    mha = run_fwd(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), True,
                  0.088, dtype)
    assert np.array_equal(a, mha)


def test_causal_outputs_ignore_future_keys_bitwise():
    dtype = "bf16"
    B, H, Sq, Sk, D = 1, 2, 500, 700, 128
    q, k, v = shape_inputs(B, H, H, Sq, Sk, D, dtype, seed=102)
    a = run_fwd(q, k, v, True, 0.088, dtype)
    j0 = 450
    k2, v2 = k.copy(), v.copy()
    k2[:, :, j0:] = wl.normal_bits(k2[:, :, j0:].shape, 103, dtype, 3.0)
    v2[:, :, j0:] = wl.normal_bits(v2[:, :, j0:].shape, 104, dtype, 3.0)
    b = run_fwd(q, k2, v2, True, 0.088, dtype)
    keep = j0 - (Sk - Sq)  # rows i < keep see no key >= j0
    assert np.array_equal(a[:, :, :keep], b[:, :, :keep])
    assert not np.array_equal(a[:, :, keep:], b[:, :, keep:])


def test_guard_bands_untouched_and_unread():
    import torch
    fa = _fa()
    dtype = "bf16"
    B, Hq, Hkv, Sq, Sk, D = 1, 4, 2, 333, 517, 128
    q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=105)
    G = 4096  # guard elements on each side
    nan = np.uint16(wl.BF16_QNAN)

    def guarded(bits):
        flat = np.full(bits.size + 2 * G, nan, dtype=np.uint16)
        flat[G:G + bits.size] = bits.ravel()
        return to_dev(flat, dtype)

    gq, gk, gv = guarded(q), guarded(k), guarded(v)
    canary = np.full(q.size + 2 * G, 0x1234, dtype=np.uint16)
    go = to_dev(canary, dtype)
    view = lambda t, shp: t[G:G + int(np.prod(shp))].view(shp)
    fa.fwd(view(gq, q.shape), view(gk, k.shape), view(gv, v.shape), causal=True,
           out=view(go, q.shape))
    torch.cuda.synchronize()
    out = bits_of(go)
    assert np.all(out[:G] == 0x1234) and np.all(out[G + q.size:] == 0x1234)
    got = oracle.widen(out[G:G + q.size].reshape(q.shape), dtype)
    assert np.all(np.isfinite(got))
    plain = run_fwd(q, k, v, True, 1 / math.sqrt(D), dtype)
    assert np.array_equal(out[G:G + q.size].reshape(q.shape), plain)


@pytest.mark.parametrize("k0", [24.0, 256.0], ids=["rescaled", "overflowed"])
def test_score_jump_in_mask_free_tile(k0):
    # key 700 scores far above every other key for every row (q[:, 0] = 8,
    # k[700, 0] = k0) and sits in a mask-free tile of the query blocks that
    # start at rows 1024 and 1280.  With k0 = 24 its exp against the running
    # reference is about 2^19 (above 2^tau but finite: the row's reference
    # moves by a power of two); with k0 = 256 the exp overflows and the item
    # is computed again with the max-first softmax.  Every schedule matches
    # the oracle; the grid, the queue-driven and the snake-order persistent
    # launches (whole items all) give the same bits (the automatic plan here, and the split launch
    # with 4-tile parts whose middle parts reach the mask-free steps, cut
    # items' keys into parts, whose merge rounds differently).
    fa = _fa()
    dtype = "bf16"
    B, Hq, Hkv, S, D = 1, 4, 2, 1536, 128
    rng = np.random.default_rng(131)
    qf = rng.standard_normal((B, Hq, S, D)).astype(np.float32)
    kf = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    qf[..., 0] = 8.0
    kf[:, :, 700, 0] = k0
    q, k = wl.to_bits(qf, dtype), wl.to_bits(kf, dtype)
    v = wl.normal_bits((B, Hkv, S, D), 132, dtype)
    scale = 1 / math.sqrt(D)
    ref = oracle.attention_ref(oracle.widen(q, dtype), oracle.widen(k, dtype),
                               oracle.widen(v, dtype), True, scale)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    outs = []
    for sched in (None, dict(persistent=0, hkv_major=0, xcd_map=0, queue=0),
                  dict(persistent=1, hkv_major=0, xcd_map=0, queue=1),
                  dict(persistent=0, hkv_major=0, xcd_map=0, split_tiles=4),
                  dict(persistent=1, hkv_major=0, xcd_map=0, queue=0)):
        print(f"\n[score jump] k0={k0} schedule={sched}", flush=True)
        if sched is None:
            o = bits_of(fa.fwd(tq, tk, tv, causal=True, scale=scale))
        else:
            o = bits_of(fa.fwd(tq, tk, tv, causal=True, scale=scale, schedule=sched))
        parity(oracle.widen(o, dtype), ref, f"k0={k0} schedule={sched}")
        outs.append(o)
    assert np.array_equal(outs[1], outs[2])
    assert np.array_equal(outs[1], outs[4])


def test_persistent_and_grid_launches_agree_bitwise():
    # the same items computed by the persistent launch, in both orders, with
    # and without the XCD dealing of (batch, kv head) units, and by one
    # workgroup per item (in both orders) give identical bits (fa_fwd_planned)
    fa = _fa()
    dtype = "bf16"
    B, Hq, Hkv, S = 2, 32, 4, 1024
    assert fa.fwd_plan(B, Hq, Hkv, S, S, 128, True)["xcd_map"] == 1
    q, k, v = shape_inputs(B, Hq, Hkv, S, S, 128, dtype, seed=106)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    outs = [run_fwd(q, k, v, True, 0.088, dtype)]  # the automatic plan
    for pers, hkv, xcd, queue in ((0, 0, 0, 0), (0, 1, 0, 0), (1, 0, 0, 0), (1, 1, 0, 0),
                                  (1, 0, 1, 0), (1, 1, 1, 0), (1, 0, 0, 1), (1, 1, 0, 1),
                                  (1, 1, 1, 1)):
        sched = dict(persistent=pers, hkv_major=hkv, xcd_map=xcd, queue=queue)
        outs.append(bits_of(fa.fwd(tq, tk, tv, causal=True, scale=0.088, schedule=sched)))
    # the key-split launch with parts of up to 8 tiles: every item here has at
    # most 1024 / 128 = 8 tiles, so each part is a whole item -- the split
    # launch's own mapping of workgroups to items, with nothing to merge
    sched = dict(persistent=0, hkv_major=0, xcd_map=0, split_tiles=8)
    outs.append(bits_of(fa.fwd(tq, tk, tv, causal=True, scale=0.088, schedule=sched)))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)


# B, Hq, Hkv, Sq, Sk, D, causal, dtype, tiles per part
SPLITS = [
    (1, 4, 2, 700, 300, 128, True, "bf16", 1),    # Sq > Sk: rows without keys; 1 tile a part
    (2, 4, 1, 257, 700, 64, True, "bf16", 1),     # bottom-right ragged, 6 parts an item
    (1, 3, 3, 511, 513, 128, False, "fp16", 2),   # 5 tiles (one key in the last) in 3 parts
    (1, 16, 1, 65, 1000, 128, True, "bf16", 3),   # 8 tiles cut 2 + 3 + 3
    (1, 2, 1, 300, 2000, 128, False, "bf16", 5),  # 16 tiles in 4 parts, ragged key tail
]


@pytest.mark.parametrize("case", SPLITS, ids=[str(c) for c in SPLITS])
def test_key_split_matches_oracle_and_repeats_bitwise(case):
    # each item's keys cut into parts summed by separate workgroups and merged
    # by the last part: O and LSE against the oracle, the same bits on a
    # second call, and within rounding of the unsplit launch
    B, Hq, Hkv, Sq, Sk, D, causal, dtype, T = case
    print(f"\n[prefill split] {case}", flush=True)
    fa = _fa()
    q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=400 + 10 * SPLITS.index(case))
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    scale = 1.0 / math.sqrt(D)
    sched = dict(persistent=0, hkv_major=0, xcd_map=0, split_tiles=T)
    o1, l1 = fa.fwd(tq, tk, tv, causal=causal, scale=scale, return_lse=True, schedule=sched)
    o2, l2 = fa.fwd(tq, tk, tv, causal=causal, scale=scale, return_lse=True, schedule=sched)
    a, b = bits_of(o1), bits_of(o2)
    assert np.array_equal(a, b)
    assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32))
    qf, kf, vf = oracle.widen(q, dtype), oracle.widen(k, dtype), oracle.widen(v, dtype)
    got = oracle.widen(a, dtype)
    ref_o = oracle.attention_ref(qf, kf, vf, causal, scale)
    st = parity(got, ref_o, str(case))
    print(f"  {st}", flush=True)
    ref = oracle.lse_ref(qf, kf, causal, scale)
    lse = l1.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.isneginf(lse[~fin]))
    np.testing.assert_allclose(lse[fin], ref[fin], rtol=1e-4, atol=1e-3)
    if causal and Sq > Sk:
        assert np.all(got[:, :, :Sq - Sk] == 0)
    plain = oracle.widen(bits_of(fa.fwd(tq, tk, tv, causal=causal, scale=scale,
                                        schedule=dict(persistent=0, hkv_major=0, xcd_map=0))),
                         dtype)
    # the split changes rounding only (each part's own reference max rounds
    # exp2 and the packed P differently; the merge adds in another order):
    # its worst error against the oracle stays within twice the unsplit
    # launch's, plus half a bf16 unit at 1
    e_split = float(np.max(np.abs(got - ref_o)))
    e_plain = float(np.max(np.abs(plain - ref_o)))
    print(f"  max |err| split {e_split:.2e}, unsplit {e_plain:.2e}", flush=True)
    assert e_split <= 2 * e_plain + 2.0 ** -8


def test_key_split_workspace_reused_across_shapes():
    # split launches of different shapes and part counts in a row on one
    # stream share the workspace: each leaves its counters at zero, so the
    # first shape gives the same bits again afterwards
    fa = _fa()
    dtype = "bf16"
    runs = []
    for (B, Hq, Hkv, Sq, Sk, D, T) in ((1, 16, 1, 65, 1000, 128, 3), (2, 4, 2, 300, 1500, 64, 1),
                                       (1, 16, 1, 65, 1000, 128, 3)):
        q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, D, dtype, seed=450 + Sk)
        tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
        sched = dict(persistent=0, hkv_major=0, xcd_map=0, split_tiles=T)
        runs.append(bits_of(fa.fwd(tq, tk, tv, causal=True, scale=0.1, schedule=sched)))
    assert np.array_equal(runs[0], runs[2])


def test_work_queue_counters_reset_between_launches():
    # persistent launches that deal items from the work queue, of different
    # shapes and list splits in a row on one stream: each leaves its counters
    # at zero, so repeating the first shape gives the same bits, and every
    # item is computed exactly once (against the static schedule)
    fa = _fa()
    dtype = "bf16"
    shapes = [(2, 32, 4, 1024, 1024, True), (1, 96, 8, 600, 900, True), (2, 32, 4, 1024, 1024, True),
              (4, 32, 8, 512, 512, False)]
    runs = []
    for i, (B, Hq, Hkv, Sq, Sk, causal) in enumerate(shapes):
        assert fa.fwd_plan(B, Hq, Hkv, Sq, Sk, 128, causal)["persistent"] == 1
        q, k, v = shape_inputs(B, Hq, Hkv, Sq, Sk, 128, dtype, seed=470 + 10 * (i % 2))
        tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
        got = bits_of(fa.fwd(tq, tk, tv, causal=causal, scale=0.09,
                             schedule=dict(persistent=1, hkv_major=i % 2, xcd_map=0, queue=1)))
        static = bits_of(fa.fwd(tq, tk, tv, causal=causal, scale=0.09,
                                schedule=dict(persistent=1, hkv_major=0, xcd_map=0, queue=0)))
        assert np.array_equal(got, static), shapes[i]
        runs.append(got)
    assert np.array_equal(runs[0], runs[2])


def test_planned_rejects_schedules_that_do_not_fit():
    import torch
    fa = _fa()
    q = torch.zeros((1, 8, 256, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 256, 64), dtype=torch.bfloat16, device="cuda")
    # 8 items: no persistent grid of 256 workgroups, and B * Hkv = 2
    with pytest.raises(fa.FaError):
        fa.fwd(q, k, k, schedule=dict(persistent=1, hkv_major=0, xcd_map=1))
    with pytest.raises(fa.FaError):
        fa.fwd(q, k, k, schedule=dict(persistent=2, hkv_major=0, xcd_map=0))
    with pytest.raises(fa.FaError):  # a work queue needs a persistent grid
        fa.fwd(q, k, k, schedule=dict(persistent=0, hkv_major=0, xcd_map=0, queue=1))
