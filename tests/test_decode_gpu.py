"""GPU parity of Sq=1 decode (fa_decode through the C ABI) against the CPU
float64 oracle, with the unused cache tail poisoned by bf16 quiet NaN, and
the bitwise valid-length semantics.

Bound: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bits_of, parity, to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fa():
    import flash_attention_forward_fwd_amd as fa
    return fa


class DecodeRig:
    """Device cache + valid length + workspace reused across calls, as a
    serving loop would hold them."""

    def __init__(self, B, Hq, Hkv, D, cap, dtype="bf16", tail=wl.BF16_QNAN):
        import torch
        fa = _fa()
        self.B, self.Hq, self.Hkv, self.D, self.cap, self.dtype = B, Hq, Hkv, D, cap, dtype
        fill = np.full((B, cap, Hkv, D), tail, dtype=np.uint16)
        self.kc = to_dev(fill, dtype)
        self.vc = to_dev(fill, dtype)
        self.vl = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.ws = fa.DecodeWorkspace(B, Hq, Hkv, D, cap)

    def write(self, b, t0, kbits, vbits):
        n = kbits.shape[0]
        self.kc[b, t0:t0 + n] = to_dev(kbits, self.dtype)
        self.vc[b, t0:t0 + n] = to_dev(vbits, self.dtype)

    def set_len(self, lens):
        import torch
        self.vl.copy_(torch.tensor(lens, dtype=torch.int32))

    def run(self, qbits, causal=False, scale=None):
        fa = _fa()
        q = to_dev(qbits, self.dtype)
        return bits_of(fa.decode(q, self.kc, self.vc, self.vl, causal=causal, scale=scale,
                                 workspace=self.ws))

    def host_cache(self):
        return bits_of(self.kc), bits_of(self.vc)


def oracle_decode(rig, qbits, lens, scale):
    kb, vb = rig.host_cache()
    return oracle.decode_ref(oracle.widen(qbits, rig.dtype), oracle.widen(kb, rig.dtype),
                             oracle.widen(vb, rig.dtype), lens, scale)


# ----------------------------------------------------------------------------
# the pages' reproduction: capacity 128, L = 1, V tail = 0x7fc0 -> O = V[0]
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_golden_nan_tail_single_token(causal):
    g = json.load(open(os.path.join(GOLDEN, "decode_nan_tail.json")))
    rig = DecodeRig(g["B"], g["Hq"], g["Hkv"], g["D"], g["capacity"], tail=g["tail_bits"])
    k0 = wl.normal_bits((1, g["Hkv"], g["D"]), 11, "bf16")
    v0 = wl.normal_bits((1, g["Hkv"], g["D"]), 12, "bf16")
    rig.write(0, 0, k0, v0)
    rig.set_len([g["valid_len"]])
    q = wl.normal_bits((1, g["Hq"], g["D"]), 13, "bf16")
    out = rig.run(q, causal=causal)
    gqa = g["Hq"] // g["Hkv"]
    for h in range(g["Hq"]):
        assert np.array_equal(out[0, h], v0[0, h // gqa]), h


# ----------------------------------------------------------------------------
# incremental decode: 128 sequential appends per sequence, every step checked
# ----------------------------------------------------------------------------
SEQUENCES = [
    # (name, capacity, first valid length)
    ("cap128_from_empty", 128, 0),
    ("cap65536_from_empty", 65536, 0),
    ("cap65536_prefilled_to_65408", 65536, 65536 - 128),
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_append_sequence(seq):
    name, cap, L0 = seq
    s = wl.DecodeShape(name, 1, 8, 2, 128, cap)
    print(f"\n[decode] {name}", flush=True)
    rig = DecodeRig(s.B, s.Hq, s.Hkv, s.D, cap)
    kall = wl.normal_bits((cap, s.Hkv, s.D), 5001, "bf16")
    vall = wl.normal_bits((cap, s.Hkv, s.D), 5002, "bf16")
    if L0:
        rig.write(0, 0, kall[:L0], vall[:L0])
    kf_all, vf_all = oracle.widen(kall, "bf16"), oracle.widen(vall, "bf16")
    worst = 0.0
    for step in range(128):
        L = L0 + step + 1
        rig.write(0, L - 1, kall[L - 1:L], vall[L - 1:L])
        rig.set_len([L])
        q = wl.normal_bits((1, s.Hq, s.D), 5000 + step, "bf16")
        out = oracle.widen(rig.run(q, causal=bool(step % 2)), "bf16")
        ref = oracle.decode_ref(oracle.widen(q, "bf16"), kf_all[None, :L], vf_all[None, :L], [L],
                                s.scale)
        worst = max(worst, parity(out, ref, f"{name} L={L}")["worst_frac_of_bound"])
    print(f"  128 appends ok, worst fraction of bound {worst:.3f}", flush=True)


# ----------------------------------------------------------------------------
# bitwise valid-length semantics
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("cap", [128, 4096, 65536])
def test_tail_contents_never_matter_bitwise(cap):
    B, Hq, Hkv, D = 1, 8, 2, 128
    valid = wl.normal_bits((cap, Hkv, D), 21, "bf16"), wl.normal_bits((cap, Hkv, D), 22, "bf16")
    junk = wl.normal_bits((cap, Hkv, D), 23, "bf16", 50.0)
    q = wl.normal_bits((B, Hq, D), 24, "bf16")
    for L in sorted({1, 31, 32, 33, cap // 3, cap - 1, cap}):
        outs = []
        for tail in ("nan", "zero", "junk"):
            rig = DecodeRig(B, Hq, Hkv, D, cap, tail={"nan": wl.BF16_QNAN, "zero": 0,
                                                      "junk": 0}[tail])
            if tail == "junk":
                rig.write(0, 0, junk, junk)
            rig.write(0, 0, valid[0][:L], valid[1][:L])
            rig.set_len([L])
            outs.append(rig.run(q))
        assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2]), L
        assert np.all(np.isfinite(oracle.widen(outs[0], "bf16")))


def test_causal_equals_unmasked_and_repeat_calls_bitwise():
    rig = DecodeRig(1, 8, 2, 128, 4096)
    k = wl.normal_bits((3000, 2, 128), 31, "bf16")
    v = wl.normal_bits((3000, 2, 128), 32, "bf16")
    rig.write(0, 0, k, v)
    rig.set_len([3000])
    q = wl.normal_bits((1, 8, 128), 33, "bf16")
    a = rig.run(q, causal=False)
    b = rig.run(q, causal=True)
    c = rig.run(q, causal=False)  # workspace reused: the run flags were lowered
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_length_zero_negative_and_clamped():
    rig = DecodeRig(3, 8, 2, 128, 256)
    k = wl.normal_bits((256, 2, 128), 41, "bf16")
    v = wl.normal_bits((256, 2, 128), 42, "bf16")
    for b in range(3):
        rig.write(b, 0, k, v)
    q = wl.normal_bits((3, 8, 128), 43, "bf16")
    rig.set_len([0, -7, 9999])
    out = rig.run(q)
    assert np.all(out[0] == 0) and np.all(out[1] == 0)
    rig.set_len([0, 0, 256])
    assert np.array_equal(rig.run(q)[2], out[2])
    ref = oracle_decode(rig, q, [0, 0, 256], 1 / np.sqrt(128))
    parity(oracle.widen(out, "bf16")[2], ref[2], "clamped")


@pytest.mark.parametrize("cfg", [
    # B, Hq, Hkv, D, cap, dtype, lens
    (2, 8, 2, 128, 3000, "bf16", [1234, 2999]),
    (1, 32, 1, 128, 2048, "bf16", [2048]),       # 32 heads share one kv head
    (1, 64, 1, 64, 1024, "bf16", [777]),         # two head groups per kv head
    (2, 4, 4, 64, 700, "fp16", [1, 650]),
    (1, 8, 2, 128, 65536, "bf16", [40000]),
    (8, 8, 2, 128, 8192, "bf16", [8192, 1, 33, 4000, 8191, 0, 6000, 129]),  # 4-column mergers
    (4, 32, 2, 64, 4096, "fp16", [4096, 2500, 31, 3000]),  # 32 columns per unit
    (32, 8, 2, 128, 2048, "bf16", [2048 - 7 * b for b in range(32)]),  # no split: one run per unit
], ids=lambda c: str(c))
def test_decode_shapes(cfg):
    B, Hq, Hkv, D, cap, dtype, lens = cfg
    print(f"\n[decode] {cfg}", flush=True)
    nan = wl.BF16_QNAN if dtype == "bf16" else wl.FP16_QNAN
    rig = DecodeRig(B, Hq, Hkv, D, cap, dtype=dtype, tail=nan)
    for b in range(B):
        k = wl.normal_bits((lens[b], Hkv, D), 51 + b, dtype)
        v = wl.normal_bits((lens[b], Hkv, D), 61 + b, dtype)
        rig.write(b, 0, k, v)
    rig.set_len(lens)
    q = wl.normal_bits((B, Hq, D), 71, dtype)
    out = oracle.widen(rig.run(q), dtype)
    ref = oracle_decode(rig, q, lens, 1 / np.sqrt(D))
    parity(out, ref, str(cfg))


def test_run_flags_lowered_across_lengths():
    """One workspace over calls whose valid lengths (and so split runs and
    merger flags) differ from call to call; every output matches the oracle,
    so no call sees a flag left raised by an earlier one."""
    cap = 65536
    rig = DecodeRig(1, 8, 2, 128, cap)
    k = wl.normal_bits((cap, 2, 128), 81, "bf16")
    v = wl.normal_bits((cap, 2, 128), 82, "bf16")
    rig.write(0, 0, k, v)
    q = wl.normal_bits((1, 8, 128), 83, "bf16")
    for L in (65536, 3000, 65536, 100, 40000, 129, 65500):
        print(f"\n[decode flags] L={L}", flush=True)
        rig.set_len([L])
        out = oracle.widen(rig.run(q), "bf16")
        ref = oracle_decode(rig, q, [L], 1 / np.sqrt(128))
        parity(out, ref, f"L={L}")


def test_workspace_reused_across_shapes():
    """One workspace, sized for the larger of two shapes, used by fa_decode for
    a long single-batch cache and then for a smaller two-batch cache: the
    second call's flags must not fall on the first call's records."""
    import torch
    fa = _fa()
    lib = fa.lib()
    shapes = [(1, 8, 2, 128, 65536, [65536], 700), (2, 8, 2, 128, 4096, [3000, 17], 720)]
    need = max(fa.decode_workspace_bytes(B, Hq, Hkv, D, cap) for B, Hq, Hkv, D, cap, _, _ in shapes)
    buf = torch.zeros(need + 256, dtype=torch.uint8, device="cuda")
    ws = buf.data_ptr() + (-buf.data_ptr()) % 256
    for B, Hq, Hkv, D, cap, lens, seed in shapes:
        print(f"\n[decode reuse] B={B} cap={cap} lens={lens}", flush=True)
        rig = DecodeRig(B, Hq, Hkv, D, cap)
        for b, L in enumerate(lens):
            rig.write(b, 0, wl.normal_bits((L, Hkv, D), seed + 2 * b, "bf16"),
                      wl.normal_bits((L, Hkv, D), seed + 2 * b + 1, "bf16"))
        rig.set_len(lens)
        qb = wl.normal_bits((B, Hq, D), seed + 50, "bf16")
        q = to_dev(qb, "bf16")
        out = torch.empty_like(q)
        st = lib.fa_decode(q.data_ptr(), rig.kc.data_ptr(), rig.vc.data_ptr(), rig.vl.data_ptr(),
                           cap, out.data_ptr(), B, Hq, Hkv, D, 0, 1 / np.sqrt(D), 0, ws, need,
                           torch.cuda.current_stream().cuda_stream)
        assert st == 0
        ref = oracle_decode(rig, qb, lens, 1 / np.sqrt(D))
        parity(oracle.widen(bits_of(out), "bf16"), ref, f"reuse lens={lens}")
