"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic. It only names the workload shapes
and produces the raw storage bits (bf16 / fp16 as uint16) that both sides
consume: the oracle widens those bits to float64 itself, the HIP side views
them as device tensors. Neither side imports the other; both import this.

Workload shapes follow the pages' experiments:
  * dense prefill, bf16/fp16, head_dim 64/128, MHA or GQA -- page "Dense
    flash-attention prefill (gfx950 / MI355X)", intro and "Measured" table
    (B=1, Hq=128, Hkv=8, D=128, causal, Sq=8192 is its headline row);
  * Sq=1 decode, B1/Hq8/Hkv2/D128 bf16 over a contiguous token-major cache
    with a device valid length -- page "hip-kernel-provider: enable minimal
    single-token attention decode", PR description.
Values are i.i.d. N(0,1) drawn in float32 and rounded to the storage type
with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
DTYPES = (BF16, FP16)

# bf16 quiet NaN used to poison the unused tail of a decode cache (page
# "hip-kernel-provider ...", review reproduction: unused V filled with 0x7fc0).
BF16_QNAN = 0x7FC0
FP16_QNAN = 0x7E00


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), return uint16 bits.

    NaN inputs map to a quiet NaN. This is storage conversion only.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_QNAN
    return r


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE fp16 (numpy's cast is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP16:
        return f32_to_fp16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def normal_bits(shape, seed: int, dtype: str, magnitude: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, magnitude^2) values in the storage type, as uint16 bits."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if magnitude != 1.0:
        x *= np.float32(magnitude)
    return to_bits(x, dtype)


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    dtype: str = BF16
    seed_base: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def admissible_pairs_per_head(self) -> int:
        """|{(i, j)}| with j <= i + (Sk - Sq) (causal) or all pairs."""
        if not self.causal:
            return self.Sq * self.Sk
        off = self.Sk - self.Sq
        tot = 0
        # row i admits min(Sk, max(0, i + off + 1)) keys
        for i in range(self.Sq):
            tot += min(self.Sk, max(0, i + off + 1))
        return tot

    def useful_flop(self) -> int:
        """4 * D per admissible (query, key) pair, summed over B and Hq.

        Non-causal form 4*B*H*Sq*Sk*D is the one printed on the tessera PR page
        ("perf ladders" commit); causal counts unmasked pairs only.
        """
        return 4 * self.D * self.B * self.Hq * self.admissible_pairs_per_head()

    def algorithmic_bytes(self) -> int:
        e = 2
        return e * self.D * (2 * self.B * self.Hq * self.Sq + 2 * self.B * self.Hkv * self.Sk)


def prefill_inputs(s: PrefillShape, magnitude: float = 1.0):
    """(q, k, v) uint16 bit arrays, q:[B,Hq,Sq,D], k,v:[B,Hkv,Sk,D]."""
    q = normal_bits((s.B, s.Hq, s.Sq, s.D), s.seed_base + 0, s.dtype, magnitude)
    k = normal_bits((s.B, s.Hkv, s.Sk, s.D), s.seed_base + 1, s.dtype, magnitude)
    v = normal_bits((s.B, s.Hkv, s.Sk, s.D), s.seed_base + 2, s.dtype, magnitude)
    return q, k, v


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    capacity: int
    dtype: str = BF16
    seed_base: int = 5000

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


def decode_cache(s: DecodeShape, valid: int, tail_bits: int | None = BF16_QNAN,
                 seed: int | None = None):
    """A token-major cache [B, capacity, Hkv, D] whose first `valid` tokens are
    N(0,1) and whose tail holds `tail_bits` (NaN by default; None = N(0,1) too).
    Returns (kcache, vcache) uint16."""
    seed = s.seed_base if seed is None else seed
    shape = (s.B, s.capacity, s.Hkv, s.D)
    k = normal_bits(shape, seed + 1, s.dtype)
    v = normal_bits(shape, seed + 2, s.dtype)
    if tail_bits is not None:
        k[:, valid:] = tail_bits
        v[:, valid:] = tail_bits
    return k, v


def decode_query(s: DecodeShape, seed: int) -> np.ndarray:
    return normal_bits((s.B, s.Hq, s.D), seed, s.dtype)


def admissible_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """Number of (query, key) pairs the mask admits for one head of one
    sequence: row i admits min(Sk, max(0, i + Sk - Sq + 1)) keys when causal."""
    if not causal:
        return Sq * Sk
    i = np.arange(Sq, dtype=np.int64)
    return int(np.minimum(Sk, np.maximum(0, i + (Sk - Sq) + 1)).sum())


def ragged_lengths(n: int, lo: int, hi: int, seed: int) -> tuple:
    """n sequence lengths drawn uniformly from [lo, hi] (seeded)."""
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, n))


@dataclasses.dataclass(frozen=True)
class VarlenShape:
    """A batch of sequences packed along the token axis ([total, H, D]),
    sequence b owning rows cu[b] .. cu[b+1]-1 (the packed varlen path with
    cu_seqlens_q / cu_seqlens_k of the prefill page's follow-ups)."""
    name: str
    lens_q: tuple
    lens_k: tuple
    Hq: int
    Hkv: int
    D: int
    causal: bool
    dtype: str = BF16
    seed_base: int = 6000

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens_q)]).astype(np.int64)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lens_k)]).astype(np.int64)

    @property
    def B(self) -> int:
        return len(self.lens_q)

    def useful_flop(self) -> int:
        """4 * D * Hq per admissible pair, summed over the sequences."""
        return 4 * self.D * self.Hq * sum(admissible_pairs(a, b, self.causal)
                                          for a, b in zip(self.lens_q, self.lens_k))

    def algorithmic_bytes(self) -> int:
        e = 2
        return e * self.D * (2 * self.Hq * sum(self.lens_q) + 2 * self.Hkv * sum(self.lens_k))


def varlen_inputs(s: VarlenShape):
    """(q, k, v) uint16 bit arrays, q:[total_q,Hq,D], k,v:[total_k,Hkv,D]."""
    tq, tk = int(sum(s.lens_q)), int(sum(s.lens_k))
    q = normal_bits((tq, s.Hq, s.D), s.seed_base + 0, s.dtype)
    k = normal_bits((tk, s.Hkv, s.D), s.seed_base + 1, s.dtype)
    v = normal_bits((tk, s.Hkv, s.D), s.seed_base + 2, s.dtype)
    return q, k, v


# The pages' workloads, as sizes.  seed_base = 1000 * config number.
TINY = PrefillShape("tiny_causal_gqa_b1_hq2_hkv1_s256_d64", 1, 2, 1, 256, 256, 64, True,
                    seed_base=1000)
MHA_CAUSAL = PrefillShape("mha_causal_b1_h16_s2048_d128", 1, 16, 16, 2048, 2048, 128, True,
                          seed_base=2000)
MHA_FULL = PrefillShape("mha_noncausal_b1_h16_s2048_d128", 1, 16, 16, 2048, 2048, 128, False,
                        seed_base=2000)
MHA_FP16 = PrefillShape("mha_causal_fp16_b1_h16_s2048_d128", 1, 16, 16, 2048, 2048, 128, True,
                        dtype=FP16, seed_base=2000)
GQA_D128 = PrefillShape("gqa_causal_b4_hq32_hkv8_s4096_d128", 4, 32, 8, 4096, 4096, 128, True,
                        seed_base=3000)
GQA_D64 = PrefillShape("gqa_causal_b4_hq32_hkv8_s4096_d64", 4, 32, 8, 4096, 4096, 64, True,
                       seed_base=3000)
RAGGED_D128 = PrefillShape("ragged_causal_b4_hq32_hkv8_sq1000_sk3000_d128", 4, 32, 8, 1000, 3000,
                           128, True, seed_base=3100)
RAGGED_D64 = PrefillShape("ragged_causal_b4_hq32_hkv8_sq1000_sk3000_d64", 4, 32, 8, 1000, 3000,
                          64, True, seed_base=3100)
HEADLINE = PrefillShape("causal_gqa_b1_hq128_hkv8_s8192_d128", 1, 128, 8, 8192, 8192, 128, True,
                        seed_base=4000)
SWEEP = tuple(PrefillShape(f"causal_gqa_b1_hq128_hkv8_s{s}_d128", 1, 128, 8, s, s, 128, True,
                           seed_base=4000 + s) for s in (256, 512, 2048))

DECODE_SMALL = DecodeShape("decode_b1_hq8_hkv2_d128_cap128", 1, 8, 2, 128, 128)
DECODE_LARGE = DecodeShape("decode_b1_hq8_hkv2_d128_cap65536", 1, 8, 2, 128, 65536)

# a ragged batch for the packed varlen path: 16 sequences of 256..8192 tokens
_VARLEN_LENS = ragged_lengths(16, 256, 8192, 6000)
VARLEN = VarlenShape("varlen_causal_b16_len256to8192_hq32_hkv8_d128", _VARLEN_LENS, _VARLEN_LENS,
                     32, 8, 128, True, seed_base=6000)

PREFILL_CONFIGS = (TINY, MHA_CAUSAL, MHA_FULL, MHA_FP16, GQA_D128, GQA_D64, RAGGED_D128,
                   RAGGED_D64, HEADLINE) + SWEEP
