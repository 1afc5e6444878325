"""Plain CPU float64 oracle for dense attention forward and Sq=1 decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library: it widens the
raw storage bits itself and computes the textbook definition, slowly, in
float64 with NumPy.

What it computes (the plain definition the tiled method reaches exactly, up
to rounding order):

  For every batch b, query head h (kv head hk = floor(h / (Hq/Hkv))) and
  query row i, the admissible key set is
      A(i) = { j in [0, Sk) : not causal  or  j <= i + (Sk - Sq) }
  (bottom-right aligned causal mask -- page "hip-kernel-provider: enable
  minimal single-token attention decode", PR description: "bottom-right
  causal"; tessera PR page, flash_attn commit: "causal/ragged mask").
      s_ij = scale * sum_d q[b,h,i,d] * k[b,hk,j,d]
      p_ij = exp(s_ij - max_{j' in A(i)} s_ij') / sum_{j in A(i)} exp(...)
      o[b,h,i,:] = sum_{j in A(i)} p_ij * v[b,hk,j,:]
  and o = 0 when A(i) is empty (the pages are silent on that case).
  That is softmax(scale * Q K^T + mask) V -- the forward pass both the gfx950
  prefill page (parity against scaled-dot-product attention, "Measured") and
  the tessera page (S = scale*Q@K^T, online softmax, O += P@V) compute.

  Decode is the Sq = 1 case over the first L tokens of a token-major cache
  [B, capacity, Hkv, D]; L is clamped to [0, capacity] and the cache tail
  past L is never read (decode PR page: device valid length, contiguous
  token-major KV; review: the unused tail is outside the logical sequence).

Packed variable-length batches (varlen_ref) apply the same definition to
each sequence of the batch separately; a paged decode cache
(decode_paged_ref) is gathered into the contiguous one first.

Pins: every function here is checked in tests/test_oracle_pins.py against
brute force on tiny inputs, closed forms (identical keys -> prefix mean of V,
one dominant key -> that V row, causal row 0 -> V[0], probability rows sum
to 1), torch's float64 CPU attention as an independent library routine,
GQA == MHA with repeated kv heads, decode == last causal prefill row, and the
split/merge identity.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP16 = "fp16"


# ----------------------------------------------------------------------------
# storage bits -> float64 (exact: every bf16 / fp16 value is a float64 value)
# ----------------------------------------------------------------------------
def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 storage bits of bf16 or fp16 -> float64, exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# mask
# ----------------------------------------------------------------------------
def admissible_mask(Sq: int, Sk: int, causal: bool, rows=None) -> np.ndarray:
    """Boolean [len(rows), Sk]: True where key j is admissible for query i.

    Bottom-right aligned causal: j <= i + (Sk - Sq)."""
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    j = np.arange(Sk)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Sk), dtype=bool)
    return j <= (rows[:, None] + (Sk - Sq))


# ----------------------------------------------------------------------------
# softmax(scale * q k^T + mask) and its product with v
# ----------------------------------------------------------------------------
def probs_ref(q_rows: np.ndarray, k: np.ndarray, allowed: np.ndarray, scale: float) -> np.ndarray:
    """P for one head: q_rows [R, D], k [Sk, D], allowed [R, Sk] -> P [R, Sk].

    Rows with no admissible key are all zero."""
    s = scale * (q_rows @ k.T)
    s = np.where(allowed, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True, initial=-np.inf)  # also for Sk = 0
    empty = ~allowed.any(axis=1, keepdims=True)
    m = np.where(empty, 0.0, m)
    w = np.where(allowed, np.exp(s - m), 0.0)
    den = w.sum(axis=1, keepdims=True)
    return np.where(empty, 0.0, w / np.where(empty, 1.0, den))


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                  row_chunk: int = 1024) -> np.ndarray:
    """Full output O [B, Hq, Sq, D] (float64) of softmax(scale Q K^T + mask) V.

    q: [B, Hq, Sq, D]; k, v: [B, Hkv, Sk, D]; all float64."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    gqa = Hq // Hkv
    out = np.zeros((B, Hq, Sq, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // gqa
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                allowed = admissible_mask(Sq, Sk, causal, rows)
                p = probs_ref(q[b, h, rows], k[b, hk], allowed, scale)
                out[b, h, rows] = p @ v[b, hk]
    return out


def attention_rows_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                       b: int, h: int, rows) -> np.ndarray:
    """The same definition for selected rows of one (b, h): [len(rows), D].

    Used to check sampled outputs at sizes where the full oracle is too slow."""
    Hq, Sq = q.shape[1], q.shape[2]
    Hkv, Sk = k.shape[1], k.shape[2]
    hk = h // (Hq // Hkv)
    rows = np.asarray(rows)
    allowed = admissible_mask(Sq, Sk, causal, rows)
    p = probs_ref(q[b, h, rows], k[b, hk], allowed, scale)
    return p @ v[b, hk]


# ----------------------------------------------------------------------------
# Sq = 1 decode over a contiguous token-major cache
# ----------------------------------------------------------------------------
def decode_ref(q: np.ndarray, kcache: np.ndarray, vcache: np.ndarray, valid_len, scale: float
               ) -> np.ndarray:
    """O [B, Hq, D] for q [B, Hq, D] over kcache, vcache [B, capacity, Hkv, D].

    Only the first L = clamp(valid_len[b], 0, capacity) tokens are read; the
    tail is sliced away before any arithmetic, so whatever it holds (NaN
    included) cannot matter.  Causal and unmasked decode coincide at Sq = 1
    (bottom-right alignment admits every j <= L - 1)."""
    B, Hq, D = q.shape
    cap, Hkv = kcache.shape[1], kcache.shape[2]
    gqa = Hq // Hkv
    valid_len = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), (B,))
    out = np.zeros((B, Hq, vcache.shape[3]), dtype=np.float64)
    for b in range(B):
        L = int(min(max(int(valid_len[b]), 0), cap))
        if L == 0:
            continue
        kk = kcache[b, :L]  # [L, Hkv, D]
        vv = vcache[b, :L]
        for h in range(Hq):
            hk = h // gqa
            allowed = np.ones((1, L), dtype=bool)
            p = probs_ref(q[b, h][None, :], kk[:, hk, :], allowed, scale)
            out[b, h] = (p @ vv[:, hk, :])[0]
    return out


def decode_multi_ref(q: np.ndarray, kcache: np.ndarray, vcache: np.ndarray, valid_len,
                     causal: bool, scale: float) -> np.ndarray:
    """O [B, Sq, Hq, D] for Sq query tokens per sequence, q [B, Sq, Hq, D],
    over kcache, vcache [B, capacity, Hkv, D] (multi-token decode, named as
    follow-up work on the decode PR page).

    Query token t sits at position L - Sq + t of its sequence, so with the
    bottom-right causal mask it sees keys j <= L - Sq + t: this is the
    definition above with Sq queries against Sk = L keys (only the first L
    cache rows are read).  Without the mask every token sees all L keys."""
    B, Sq, Hq, _ = q.shape
    cap = kcache.shape[1]
    valid_len = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), (B,))
    out = np.zeros((B, Sq, Hq, vcache.shape[3]), dtype=np.float64)
    for b in range(B):
        L = int(min(max(int(valid_len[b]), 0), cap))
        qs = q[b].transpose(1, 0, 2)[None]           # [1, Hq, Sq, D]
        ks = kcache[b, :L].transpose(1, 0, 2)[None]  # [1, Hkv, L, D]
        vs = vcache[b, :L].transpose(1, 0, 2)[None]
        out[b] = attention_ref(qs, ks, vs, causal, scale)[0].transpose(1, 0, 2)
    return out


def decode_paged_ref(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, page_table,
                     valid_len, scale: float, causal: bool = False) -> np.ndarray:
    """O [B, Hq, D] over a paged cache: pools [num_pages, page_size, Hkv, D]
    and page_table [B, pages_per_seq], token t of batch b being row
    t % page_size of page page_table[b, t // page_size] (the paged KV that the
    decode PR page leaves as follow-up work to its identity page table).

    The first L = clamp(valid_len[b], 0, pages_per_seq * page_size) tokens are
    gathered into a contiguous cache and decode_ref's definition applied
    (decode_multi_ref's for q [B, Sq, Hq, D]); rows past L, and pages no
    valid token maps to, are never read."""
    B = q.shape[0]
    P = k_pages.shape[1]
    page_table = np.asarray(page_table)
    cap = P * page_table.shape[1]
    valid_len = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), (B,))
    out = np.zeros(q.shape[:-1] + (v_pages.shape[3],), dtype=np.float64)
    for b in range(B):
        L = int(min(max(int(valid_len[b]), 0), cap))
        t = np.arange(L)
        pages, rows = page_table[b, t // P], t % P
        kk, vv = k_pages[pages, rows], v_pages[pages, rows]  # [L, Hkv, D]
        if q.ndim == 3:
            out[b] = decode_ref(q[b:b + 1], kk[None], vv[None], [L], scale)[0]
        else:
            out[b] = decode_multi_ref(q[b:b + 1], kk[None], vv[None], [L], causal, scale)[0]
    return out


# ----------------------------------------------------------------------------
# split-KV partials and their merge (the decode combine step)
# ----------------------------------------------------------------------------
def partial_ref(q_rows: np.ndarray, k_chunk: np.ndarray, v_chunk: np.ndarray, scale: float):
    """Unnormalised partial over one KV chunk: (m [R], l [R], acc [R, D]) with
    m = max_j s_ij, l = sum_j exp(s_ij - m), acc = sum_j exp(s_ij - m) v_j.
    An empty chunk gives m = -inf, l = 0, acc = 0."""
    R = q_rows.shape[0]
    if k_chunk.shape[0] == 0:
        return (np.full(R, -np.inf), np.zeros(R), np.zeros((R, v_chunk.shape[1])))
    s = scale * (q_rows @ k_chunk.T)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    return m, w.sum(axis=1), w @ v_chunk


def merge_ref(parts) -> np.ndarray:
    """Merge partials: M = max_s m_s; O = sum_s e^(m_s-M) acc_s / sum_s e^(m_s-M) l_s.

    Chunks with m_s = -inf contribute nothing; if every chunk is empty the
    result is 0."""
    ms = np.stack([p[0] for p in parts])          # [S, R]
    M = ms.max(axis=0)                            # [R]
    Msafe = np.where(np.isfinite(M), M, 0.0)
    num = 0.0
    den = 0.0
    for m, l, acc in parts:
        f = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - Msafe), 0.0)
        num = num + f[:, None] * acc
        den = den + f * l
    den = np.asarray(den)
    safe = den > 0
    return np.where(safe[:, None], num / np.where(safe, den, 1.0)[:, None], 0.0)


# ----------------------------------------------------------------------------
# log-sum-exp of each row's scores (natural log), -inf for an empty row
# ----------------------------------------------------------------------------
def lse_ref(q: np.ndarray, k: np.ndarray, causal: bool, scale: float) -> np.ndarray:
    """LSE [B, Hq, Sq] = log sum_{j in A(i)} exp(s_ij) in float64."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    gqa = Hq // Hkv
    out = np.full((B, Hq, Sq), -np.inf)
    allowed = admissible_mask(Sq, Sk, causal)
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // gqa].T)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1)
            ok = np.isfinite(m)
            ms = np.where(ok, m, 0.0)
            tot = np.where(allowed, np.exp(s - ms[:, None]), 0.0).sum(axis=1)
            out[b, h] = np.where(ok, ms + np.log(np.where(ok, tot, 1.0)), -np.inf)
    return out


# ----------------------------------------------------------------------------
# packed variable-length batches
# ----------------------------------------------------------------------------
def varlen_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k, causal: bool,
               scale: float, with_lse: bool = False):
    """Attention over sequences packed along the token axis (the packed varlen
    path with cu_seqlens_q / cu_seqlens_k named on the page "Dense
    flash-attention prefill (gfx950 / MI355X)", TODO / follow-ups).

    q: [total_q, Hq, D]; k, v: [total_k, Hkv, D]; cu_q, cu_k: int [B + 1],
    non-decreasing offsets.  Sequence b is plain attention of query rows
    cu_q[b] .. cu_q[b+1]-1 against key rows cu_k[b] .. cu_k[b+1]-1, with the
    bottom-right causal mask of its own two lengths.  Returns O
    [total_q, Hq, D] (float64) -- NaN in rows that belong to no sequence --
    and, with with_lse, LSE [Hq, total_q] (NaN likewise)."""
    total_q, Hq, _ = q.shape
    out = np.full((total_q, Hq, v.shape[2]), np.nan)
    lse = np.full((Hq, total_q), np.nan)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        qs = q[q0:q1].transpose(1, 0, 2)[None]  # [1, Hq, Sq_b, D]
        ks = k[k0:k1].transpose(1, 0, 2)[None]  # [1, Hkv, Sk_b, D]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        out[q0:q1] = attention_ref(qs, ks, vs, causal, scale)[0].transpose(1, 0, 2)
        if with_lse:
            lse[:, q0:q1] = lse_ref(qs, ks, causal, scale)[0]
    return (out, lse) if with_lse else out


# ----------------------------------------------------------------------------
# backward pass (gradients of O with respect to Q, K and V)
# ----------------------------------------------------------------------------
def attention_bwd_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, causal: bool,
                      scale: float):
    """(dQ, dK, dV) float64 for O = softmax(scale Q K^T + mask) V and an output
    gradient dO (tessera PR page, flash_attn backward commit: the textbook
    FA-2 backward -- a pre-pass for D = rowsum(O * dO), dK/dV per key tile,
    dQ per query tile -- whose plain matrix form is written out here).

    Per (b, h) with kv head hk = h // (Hq/Hkv), in the plain matrix form:
        P  = softmax(scale Q K^T + mask)          (rows without keys: 0)
        dV[hk] += P^T dO
        dP = dO V^T
        Dr = rowsum(dO * O)  (= rowsum(P * dP))
        dS = P * (dP - Dr)
        dQ = scale dS K,     dK[hk] += scale dS^T Q
    Query heads of one GQA group add into their kv head's dK and dV."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    gqa = Hq // Hkv
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    allowed = admissible_mask(Sq, Sk, causal)
    for b in range(B):
        for h in range(Hq):
            hk = h // gqa
            p = probs_ref(q[b, h], k[b, hk], allowed, scale)  # [Sq, Sk]
            o = p @ v[b, hk]
            dv[b, hk] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, hk].T
            dr = np.sum(do[b, h] * o, axis=1, keepdims=True)
            ds = p * (dp - dr)
            dq[b, h] = scale * (ds @ k[b, hk])
            dk[b, hk] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def attention_bwd_dq_rows_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                              causal: bool, scale: float, b: int, h: int, rows) -> np.ndarray:
    """dQ rows [len(rows), D] of one (b, h) by the same definition as
    attention_bwd_ref, for sizes where the full backward is too slow: a row
    of dQ needs only that row's P, dP and D."""
    Hq, Sq = q.shape[1], q.shape[2]
    Hkv, Sk = k.shape[1], k.shape[2]
    hk = h // (Hq // Hkv)
    rows = np.asarray(rows)
    allowed = admissible_mask(Sq, Sk, causal, rows)
    p = probs_ref(q[b, h, rows], k[b, hk], allowed, scale)  # [R, Sk]
    o = p @ v[b, hk]
    dp = do[b, h, rows] @ v[b, hk].T
    dr = np.sum(do[b, h, rows] * o, axis=1, keepdims=True)
    return scale * ((p * (dp - dr)) @ k[b, hk])
