// Dense attention forward (prefill) for gfx950.
//
// Computes O = softmax(scale * Q K^T + mask) V tile by tile with a running
// max / running sum, so no Sq x Sk score matrix is ever stored (tessera PR
// page, flash_attn forward commit: S = scale*Q@K^T, causal/ragged mask,
// online softmax, O += P@V).  Mask: key j is admissible for query i iff
// j <= i + (Sk - Sq) when causal (decode PR page: "bottom-right causal").
//
// Work decomposition (page "Dense flash-attention prefill (gfx950 / MI355X)"):
//  * a work item is (batch, query head, 256-row query block); a workgroup of
//    8 waves owns one item at a time, each wave 32 query rows;
//  * in persistent mode a grid of one workgroup per CU strides over the
//    items ("Persistent (grid-stride) mode"), ordered kv-head-major when
//    that still balances, so concurrently running items share K/V in L2;
//  * with fewer items than CUs, each item's key tiles may be cut into parts
//    run by separate workgroups, whose partial (O, max, sum) the last part
//    to start merges in the same launch (merge_parts);
//  * KV tiles of kPrefillBN keys (128; 64 as a build option) stream through
//    rings of two (three) row-padded LDS slots ("Baked-in levers": K rows
//    padded against bank conflicts, V pad), copied by 16-byte buffer loads
//    that write LDS directly;
//  * the two waves that share a SIMD run one phase apart (ping-pong): while
//    one issues the tile's MFMAs the other runs its softmax;
//  * below-diagonal tiles run mask-free, only tiles crossing the diagonal
//    or the end of the keys evaluate the mask ("diagonal-only causal
//    masking"); a wave skips tiles that are entirely masked for its rows.
//
// Per wave and KV tile, on the 32x32x16 matrix core:
//  * S^T = K Q^T: K (A operand) read from LDS, Q (B operand) resident in
//    VGPRs for the whole item.  The accumulator layout puts one query row
//    per lane (row = lane % 32) and 16 of the tile's keys per lane, so the
//    row max and row sum need only one exchange with lane ^ 32.
//  * exp2 online softmax: c = |scale| * log2(e) folded into one FMA per score,
//    p = exp2(s*c - m_ref) ("native exp2_fast"), where the reference m_ref
//    trails the running max by at most kRescaleTau, so the argument stays
//    <= kRescaleTau.
//  * O^T += V^T P^T: P is fed straight from the S accumulator registers as
//    the B operand.  The contraction over keys is permuted to the order in
//    which P already sits in registers, and V (A operand) is read from LDS
//    with the gfx950 transposing read in that same permuted order -- no
//    cross-lane relayout of P ("CK-1 transposed PV" describes the same
//    idea).  O^T keeps one query row per lane, so the rescale by
//    exp2(m_old - m_new) is lane-local; it runs only on tiles where some
//    row of the wave moves its reference max.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kKPad = 8;   // K LDS row = D + 8 elements (16-byte skew per row)
constexpr int kVPad = 32;  // V LDS row = D + 32 elements (64-byte skew per row)
// 1 KiB LDS-image pieces per wave per tile copy: the K image of a BN-key tile
// has BN (D + 8) / 512 pieces, the V image BN (D + 32) / 512; 4 waves share them
constexpr int kDmaSlots = (kPrefillBN * (128 + kVPad) / 512 + 3) / 4;

// The exp2 reference max of a row moves only when the row's running max
// exceeds it by more than kRescaleTau (log2 units), so p = exp2(s*c - m_ref)
// stays <= 2^kRescaleTau and the O accumulator is rescaled only on the rare
// tiles where some row of the wave jumps that far.  The final O / l and the
// LSE are exact for any reference, so this changes rounding only.
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 8.0f
#endif
constexpr float kRescaleTau = FA_RESCALE_TAU;
static_assert(kRescaleTau == (float)(int)kRescaleTau && kRescaleTau >= 1.f && kRescaleTau <= 64.f,
              "the rescale threshold is a whole number of octaves");
constexpr float pow2_whole(int n) {
  float r = 1.f;
  for (int i = 0; i < n; ++i) r *= 2.f;
  return r;
}
// 2^kRescaleTau: no p above it survives a tile
constexpr float kRescaleGate = pow2_whole((int)kRescaleTau);
// LDS operand reads run this many MFMAs ahead of their consumer in the
// steady-state M step (LDS latency under load exceeds two MFMAs)
#ifndef FA_LOOKAHEAD
#define FA_LOOKAHEAD 4
#endif
constexpr int kLookahead = FA_LOOKAHEAD;
// wave priority of the MFMA step (s_setprio; 0 = default) while the other
// wave of its SIMD runs the vector step
#ifndef FA_MFMA_SETPRIO
#define FA_MFMA_SETPRIO 0
#endif
constexpr int kMfmaPrio = FA_MFMA_SETPRIO;

// Work item -> (batch, query head, query block).  Query blocks are visited
// heaviest first (a causal block's cost grows with its index).
__device__ __forceinline__ void decode_item(const PrefillParams& p, int w, int& b, int& hq,
                                            int& qb) {
  if (p.hkv_major) {
    // kv head outermost, then query block (descending), batch, group member
    const int per_kv = p.gqa * p.nqb * p.B;
    const int hk = w / per_kv;
    int r = w - hk * per_kv;
    const int per_lvl = p.gqa * p.B;
    const int lvl = r / per_lvl;
    r -= lvl * per_lvl;
    b = r / p.gqa;
    const int g = r - b * p.gqa;
    qb = p.nqb - 1 - lvl;
    hq = hk * p.gqa + g;
  } else {
    const int per_lvl = p.Hq * p.B;
    const int lvl = w / per_lvl;
    const int r = w - lvl * per_lvl;
    qb = p.nqb - 1 - lvl;
    b = r / p.Hq;
    hq = r - b * p.Hq;
  }
}

// Item w of XCD x's list -> (batch, query head, query block).  The XCD owns
// the units u = (batch, kv head) = b * Hkv + hk with u % kXcds == x, its
// ui-th unit being ui * kXcds + x.  Its list runs unit-major (unit, query
// block descending, group member) when hkv_major, else block-major (query
// block descending, unit, group member).
__device__ __forceinline__ void xcd_item(const PrefillParams& p, int x, int w, int& b, int& hq,
                                         int& qb) {
  const int nu = p.B * p.Hkv / kXcds;  // units per XCD
  int ui, lvl;
  if (p.hkv_major) {
    const int per_unit = p.gqa * p.nqb;
    ui = w / per_unit;
    const int r = w - ui * per_unit;
    lvl = r / p.gqa;
    w = r - lvl * p.gqa;
  } else {
    const int per_lvl = nu * p.gqa;
    lvl = w / per_lvl;
    const int r = w - lvl * per_lvl;
    ui = r / p.gqa;
    w = r - ui * p.gqa;
  }
  const int u = ui * kXcds + x;
  b = u / p.Hkv;
  hq = (u - b * p.Hkv) * p.gqa + w;
  qb = p.nqb - 1 - lvl;
}

// Key tiles of query block qb of a dense item (all of them when not causal).
template <bool CAUSAL>
__device__ __forceinline__ int dense_block_tiles(const PrefillParams& p, int qb) {
  int kv_end = p.Sk;
  if (CAUSAL) kv_end = min(max(min(p.Sq, qb * kPrefillBM + kPrefillBM) + p.Sk - p.Sq, 0), p.Sk);
  return (kv_end + kPrefillBN - 1) / kPrefillBN;
}

// Split schedule: workgroup `bid` -> (work item w, part `part` of `nparts`,
// key tiles [t0, t1) of the item).  Items run in the query-block-major order
// of decode_item (block level descending, then batch and query head); an item
// of nt tiles has ceil(nt / split_tiles) parts (at least one) of near-equal
// tile counts, numbered consecutively.  The grid holds exactly the parts, so
// every workgroup finds one; one past the end gets nparts = 0.
template <bool CAUSAL>
__device__ __forceinline__ void split_part(const PrefillParams& p, int bid, int& w, int& part,
                                           int& nparts, int& t0, int& t1) {
  const int per_lvl = p.Hq * p.B, T = p.split_tiles;
  int r = bid;
  nparts = 0;
  for (int lvl = 0; lvl < p.nqb; ++lvl) {
    const int nt = dense_block_tiles<CAUSAL>(p, p.nqb - 1 - lvl);
    const int np = max(1, (nt + T - 1) / T);
    if (r < np * per_lvl) {
      const int i = r / np;
      part = r - i * np;
      nparts = np;
      w = lvl * per_lvl + i;
      t0 = part * nt / np;
      t1 = (part + 1) * nt / np;
      return;
    }
    r -= np * per_lvl;
  }
}

// bounded wait of an item's last part for the other parts' records (those
// parts have all started, so in practice the wait is a few microseconds)
constexpr int kSplitSpinLimit = 1 << 20;

// End of a split part (nparts > 1).  Each part took an arrival rank from
// the item's first counter when it started (the atomic's round trip hides
// behind the prologue loads).  Every part but the last to start stores its
// fp32 record -- O^T unnormalized against its reference max m, m and the row
// sum l (per wave and lane, in register order) -- waits until the stores are
// complete, counts itself in the item's second counter and returns false.
// The last part to start waits until that counter shows the other parts'
// records (those parts started before it, so they are running and will
// finish), zeroes both counters for the next launch, and forms the merged
// result in its registers:
//     M = max_s m_s,  O = sum_s 2^(m_s - M) O_s,  l = sum_s 2^(m_s - M) l_s
// summed in part order with the same fused multiply-adds for its own part as
// for the stored ones, so the bits do not depend on which part starts last.
// It returns true and the caller writes O / l (and the LSE from M and l).
template <int DTILES>
__device__ __forceinline__ bool merge_parts(const PrefillParams& p, int w, int part, int nparts,
                                            unsigned rank, unsigned* split_word,
                                            f32x16 (&oacc)[DTILES], float& m_run,
                                            float& l_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned* cnt = p.split_cnt + 2 * w;
  constexpr int OB = kPrefillWaves * DTILES * 4 * 1024;  // O bytes of a record
  constexpr int REC = OB + kPrefillWaves * 64 * 8;       // record bytes
  static_assert((size_t)REC == split_record_bytes(32 * DTILES), "record layout");
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      p.split_rec, (short)0, (int)gridDim.x * REC, kBufferFlags);
  const int first = (int)blockIdx.x - part;  // workgroup of part 0
  auto o_off = [&](int s, int dt, int a) {
    return (first + s) * REC + ((wave * DTILES + dt) * 4 + a) * 1024 + lane * 16;
  };
  auto ml_off = [&](int s) { return (first + s) * REC + OB + (wave * 64 + lane) * 8; };

  if ((int)rank < nparts - 1) {
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        st4_coherent(rs, o_off(part, dt, a),
                     f32x4{oacc[dt][4 * a], oacc[dt][4 * a + 1], oacc[dt][4 * a + 2],
                           oacc[dt][4 * a + 3]});
    st2_coherent(rs, ml_off(part), f32x2{m_run, l_tot});
    wait_vmem();
    __syncthreads();
    if (tid == 0) add_flag(cnt + 1, 1u);
    return false;
  }
  if (tid == 0) {
    unsigned seen = 0;
    for (int it = 0; it < kSplitSpinLimit && !seen; ++it) {
      seen = ld_flag(cnt + 1) >= (unsigned)(nparts - 1);
      if (!seen) __builtin_amdgcn_s_sleep(1);
    }
    split_word[1] = seen;
    st_flag(cnt, 0u);
    st_flag(cnt + 1, 0u);
  }
  __syncthreads();
  if (!split_word[1]) {  // records missing: make the failure visible
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = f32x16{} + nan;
    m_run = nan;
    l_tot = 1.f;
    return true;
  }
  float M = m_run;
  for (int s = 0; s < nparts; ++s)
    if (s != part) M = fmaxf(M, ld2_coherent(rs, ml_off(s))[0]);
  const float Mu = M == -__builtin_inff() ? 0.f : M;
  f32x16 acc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) acc[dt] = f32x16{};
  float l = 0.f;
  for (int s = 0; s < nparts; ++s) {
    f32x16 x[DTILES];
    float ms, ls;
    if (s == part) {
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) x[dt] = oacc[dt];
      ms = m_run;
      ls = l_tot;
    } else {
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x4 v = ld4_coherent(rs, o_off(s, dt, a));
#pragma unroll
          for (int i = 0; i < 4; ++i) x[dt][4 * a + i] = v[i];
        }
      const f32x2 ml = ld2_coherent(rs, ml_off(s));
      ms = ml[0];
      ls = ml[1];
    }
    const float f = fast_exp2(ms - Mu);
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = __builtin_fmaf(f, x[dt][r], acc[dt][r]);
    l = __builtin_fmaf(f, ls, l);
  }
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = acc[dt];
  m_run = Mu;
  l_tot = l;
  return true;
}

// Packed varlen schedule.  The work items are the non-empty (sequence, query
// head, query block) triples, in the dense order: block level descending (a
// causal block's cost grows with its index whatever sequence it belongs to),
// kv head outermost when kv-head-major.  Empty blocks of short sequences are
// left out, so the persistent round-robin sees a list of items of steadily
// falling cost, as in the dense case, instead of long and short sequences
// pinned to fixed workgroups (page "Dense flash-attention prefill (gfx950 /
// MI355X)", TODO / follow-ups: per-sequence load balance of the varlen path).
// Every wave derives an item from the per-sequence block counts in LDS.
constexpr int kVarlenMaxSeqs = 4096;  // batches up to this size use the table
// block levels up to which the item lookup uses a per-level table in LDS
// (binary search) instead of walking the levels from the top
constexpr int kVarlenMaxLevels = 960;

// sequences with more than L query blocks
__device__ __forceinline__ int seqs_above(const uint16_t* nqb, int B, int L, int lane) {
  int n = 0;
  for (int c = 0; c < B; c += 64) {
    const bool on = c + lane < B && nqb[c + lane] > L;
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(on));
  }
  return n;
}

// index of the j-th (from 0) sequence with more than L query blocks
__device__ __forceinline__ int nth_seq_above(const uint16_t* nqb, int B, int L, int j, int lane) {
  for (int c = 0; c < B; c += 64) {
    const bool on = c + lane < B && nqb[c + lane] > L;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(on);
    const int cnt = __builtin_popcountll(m);
    if (j < cnt) {
      // the lane whose bit is the j-th set bit has j set bits below it
      const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
      return c + __builtin_ctzll(__builtin_amdgcn_ballot_w64(on && below == j));
    }
    j -= cnt;
  }
  return 0;
}

// work item w of the compacted varlen list -> (sequence, query head, block).
// With the XCD map, w indexes XCD x's list, which holds the items of the kv
// heads hk with hk % kXcds == x (every kv head has the same items, so the
// XCDs' lists are alike) in the block-major order (block level descending,
// sequence, kv head, group member): sorted by cost, which the snake rounds
// balance best, while each kv head's K/V stays in one XCD's L2.
// `above` (LDS, or nullptr): above[L] = (sequence, block) pairs at levels >= L,
// above[nqb] = 0.  Level L holds the items r with above[L + 1] per <= r <
// above[L] per.
__device__ __forceinline__ void varlen_item(const PrefillParams& p, const uint16_t* nqb,
                                            const int* above, int total_blocks, int w, int lane,
                                            bool xmap, int x, int& b, int& hq, int& qb) {
  // items per (sequence, block)
  const int per = xmap ? p.Hq / kXcds : (p.hkv_major ? p.gqa : p.Hq);
  int r = w, hk = 0;
  if (p.hkv_major && !xmap) {
    const int per_kv = total_blocks * p.gqa;
    hk = w / per_kv;
    r = w - hk * per_kv;
  }
  int L = p.nqb - 1;
  if (above != nullptr) {
    // the last level L with above[L] per > r (above falls as L rises)
    int lo = 0, hi = p.nqb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (above[mid] * per > r) lo = mid;
      else hi = mid - 1;
    }
    L = lo;
    r -= above[L + 1] * per;
  } else {
    for (; L > 0; --L) {
      const int n = seqs_above(nqb, p.B, L, lane) * per;
      if (r < n) break;
      r -= n;
    }
  }
  const int j = r / per, m = r - j * per;
  b = nth_seq_above(nqb, p.B, L, j, lane);
  qb = L;
  if (xmap) {
    const int ui = m / p.gqa;  // the XCD's ui-th kv head
    hq = (ui * kXcds + x) * p.gqa + (m - ui * p.gqa);
  } else {
    hq = p.hkv_major ? hk * p.gqa + m : m;
  }
}

template <int D, int DT, bool CAUSAL, bool LSE, bool VARLEN, bool SPLIT, bool PF>
__global__ __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams p) {
  static_assert(!(SPLIT && VARLEN), "the key split is for the dense layout");
  static_assert(!(PF && (SPLIT || VARLEN)), "the prefetch and work queue are for dense launches");
  using E = Elt<DT>;
  constexpr int NT = kPrefillWaves * 64;
  constexpr int BM = kPrefillBM;
  constexpr int BN = kPrefillBN;
  // LDS ring depth: with 64-key tiles three slots (tile X is copied two
  // phases before the lead group reads it), with 128-key tiles two (copied in
  // the phase just before; three would not fit in LDS)
  constexpr int NBUF = BN == 64 ? 3 : 2;
  constexpr int NST = BN / 32;       // 32-key sub-tiles per tile
  constexpr int KST = D + kKPad;
  constexpr int VST = D + kVPad;
  constexpr int KTILE = BN * KST;    // elements per K buffer
  constexpr int VTILE = BN * VST;    // elements per V buffer
  constexpr int KSTEPS = D / 16;     // k-steps of the QK product
  constexpr int DTILES = D / 32;     // 32-wide column tiles of O
  constexpr int CH = D / 8;          // 16-byte chunks per K/V row
  static_assert(BN == 64 || BN == 128, "a tile is two or four 32-key sub-tiles");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[NBUF * KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[NBUF * VTILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31;   // query row inside the wave's 32 rows
  const int lh = lane >> 5;   // which half of the k (or key) slots this lane holds
  // LDS element offsets of this lane's operands inside a tile
  const int k_lane = li * KST + 8 * lh;
  const int ti = lane & 15;
  const int v_lane = (4 * lh + (ti >> 2)) * VST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);
  uint16_t* __restrict__ og = static_cast<uint16_t*>(p.o);
  const float c = p.c_log2;

  // varlen: query blocks per sequence, and the compacted item count
  __shared__ uint16_t nqb_tab[VARLEN ? kVarlenMaxSeqs : 1];
  __shared__ int lvl_above[VARLEN ? kVarlenMaxLevels + 1 : 1];
  int work_items = p.work_items, total_blocks = 0;
  const bool compact = VARLEN && p.B <= kVarlenMaxSeqs && p.nqb <= 0xFFFF;
  const bool lvl = compact && p.nqb <= kVarlenMaxLevels;
  if constexpr (VARLEN) {
    if (compact) {
      for (int i = tid; i < p.B; i += NT) {
        const int lo = min(max(p.cu_q[i], 0), p.total_q);
        const int hi = min(max(p.cu_q[i + 1], lo), p.total_q);
        nqb_tab[i] = (uint16_t)((min(hi - lo, p.Sq) + BM - 1) / BM);
      }
      __syncthreads();
      int t = 0;
      for (int i = lane; i < p.B; i += 64) t += nqb_tab[i];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
      total_blocks = uniform(t);
      work_items = total_blocks * p.Hq;
      if (lvl) {
        // above[L] = sum over sequences of max(0, blocks - L): a histogram of
        // the sequences' top levels, then two suffix sums (wave 0)
        for (int i = tid; i <= p.nqb; i += NT) lvl_above[i] = 0;
        __syncthreads();
        for (int i = tid; i < p.B; i += NT)
          if (nqb_tab[i] > 0) atomicAdd(&lvl_above[min((int)nqb_tab[i], p.nqb) - 1], 1);
        __syncthreads();
        if (wave == 0) {
          for (int pass = 0; pass < 2; ++pass) {
            int carry = 0;
            for (int base = ((p.nqb - 1) >> 6) << 6; base >= 0; base -= 64) {
              const int i = base + lane;
              int v = i < p.nqb ? lvl_above[i] : 0;
#pragma unroll
              for (int o = 1; o < 64; o <<= 1) {
                const int u = __shfl_down(v, o);
                v += lane + o < 64 ? u : 0;
              }
              v += carry;
              if (i < p.nqb) lvl_above[i] = v;
              carry = __shfl(v, 0);
            }
          }
        }
        __syncthreads();
      }
    }
  }

  // The workgroups that stride over one item list: the whole grid, or with
  // the XCD map the grid's workgroups on one XCD (workgroup i runs on XCD
  // i % kXcds), which stride over the items of that XCD's units only (the
  // host sets the map only for a persistent grid of a multiple of kXcds).
  const bool xmap = p.xcd_map && p.persistent;
  const int xcd = xmap ? (int)blockIdx.x % kXcds : 0;
  const int NP = xmap ? (int)gridDim.x / kXcds : (int)gridDim.x;
  const int cta = xmap ? (int)blockIdx.x / kXcds : (int)blockIdx.x;
  const int list_items = xmap ? work_items / kXcds : work_items;
  // split launches: this workgroup's part of its item, key tiles [t0, t1),
  // and its arrival rank among the item's parts (through LDS)
  int part = 0, nparts = 1, t0 = 0, t1 = 0;
  __shared__ unsigned split_word[SPLIT ? 2 : 1];

  // Where an item's rows and keys live: its sequence has Sq query rows and Sk
  // keys, row strides QRS / KRS elements.  Dense: [B, H, S, D] tensors.
  // Varlen: packed [total, H, D] tensors whose sequence b spans rows
  // [cu[b], cu[b + 1]), with offsets clamped to [0, total] and lengths to the
  // declared maxima (p.Sq, p.Sk), so no index leaves the tensors whatever the
  // offsets hold.  False for a varlen query block past its sequence's end.
  struct ItemLoc {
    int b, hq, q0, Sq, Sk, q_lo, QRS, KRS;
    long long qbase, kvbase;
  };
  auto locate = [&](int w, ItemLoc& L) -> bool {
    int b, hq, qb;
    if (compact)
      varlen_item(p, nqb_tab, lvl ? lvl_above : nullptr, total_blocks, w, lane, xmap, xcd, b, hq,
                  qb);
    else if (xmap) xcd_item(p, xcd, w, b, hq, qb);
    else decode_item(p, w, b, hq, qb);
    const int hk = hq / p.gqa;
    L.b = b;
    L.hq = hq;
    L.q0 = qb * BM;
    L.Sq = p.Sq;
    L.Sk = p.Sk;
    L.q_lo = 0;
    L.QRS = D;
    L.KRS = D;
    if constexpr (VARLEN) {
      int q_lo = min(max(p.cu_q[b], 0), p.total_q);
      const int q_hi = min(max(p.cu_q[b + 1], q_lo), p.total_q);
      const int k_lo = min(max(p.cu_k[b], 0), p.total_k);
      const int k_hi = min(max(p.cu_k[b + 1], k_lo), p.total_k);
      L.Sq = uniform(min(q_hi - q_lo, p.Sq));
      L.Sk = uniform(min(k_hi - k_lo, p.Sk));
      q_lo = uniform(q_lo);
      L.q_lo = q_lo;
      L.QRS = p.Hq * D;
      L.KRS = p.Hkv * D;
      L.qbase = (long long)q_lo * L.QRS + (long long)hq * D;
      L.kvbase = (long long)uniform(k_lo) * L.KRS + (long long)hk * D;
      return L.q0 < L.Sq;
    } else {
      L.qbase = (long long)b * p.q_bstride + (long long)hq * L.Sq * D;
      L.kvbase = (long long)b * p.kv_bstride + (long long)hk * L.Sk * D;
      return true;
    }
  };
  // Q rows of this wave as the B operand, lane holding q[row][16kk + 8lh ..
  // +7], as raw bits: buffer loads from a range that ends after the item's
  // last row, so rows past it read zeros without a branch, and nothing waits
  // for the loads here (the sign of the scale is folded in by fold_q once
  // they have landed)
  u32x4 qr[KSTEPS];
  auto load_q = [&](const ItemLoc& L) {
    const int rows = min(BM, L.Sq - L.q0);
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(qg + L.qbase + (long long)L.q0 * L.QRS), (short)0,
        ((rows - 1) * L.QRS + D) * 2, kBufferFlags);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qr[kk] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     qrs, ((wave * 32 + li) * L.QRS + 16 * kk + 8 * lh) * 2, 0, 0));
  };
  auto fold_q = [&]() {
    if (p.q_sign != 1) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        qr[kk] = p.q_sign < 0 ? (qr[kk] ^ 0x80008000u) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // Cross-item prefetch (the PF instances: persistent grids with the work
  // queue, two-slot rings): in its last
  // phases an item loads the next item's Q and copies its first K/V tile,
  // each wave group into the ring slot it would fill with the item's own
  // tile ntiles, so the next item starts without a prologue.  The ring numbering carries
  // on across items: tile t of an item sits in slot (t + ring) % NBUF.
  constexpr bool kPrefetch = PF && NBUF == 2;
  bool have_pf = false;  // this item's Q and tile 0 were loaded by the one before
  int ring = 0;
  // Work queue (persistent launches with the prefetch): a workgroup's first
  // two items are list positions cta and NP + cta (no atomic before the
  // first item); each later item is list position 2 NP + t for a ticket t
  // taken from the list's counter.  The ticket for the
  // item after next is taken in an item's final phase, so the next item is
  // known (and prefetched) a whole item ahead and the atomic's latency hides
  // behind the item's end.  Items are dealt in list order (heaviest first
  // within each kv head), each to the first workgroup that is free, which
  // also evens out XCDs that run at different speeds.  The queue state lives
  // in LDS, not in registers, which the tile loop needs every one of:
  // q_item[r & 1] holds round r's item, q_tick the ticket thread 0 took in
  // the last item (kEmpty if that item ran no phase and took none).
  const bool qmode = kPrefetch && p.persistent && p.queue != nullptr;
  __shared__ unsigned q_item[2], q_tick;
  constexpr unsigned kEmpty = 0xFFFFFFFFu, kNoTicket = 0x3FFFFFFFu;
  auto qctr = [&]() { return p.queue + (xmap ? xcd : 0); };
  // An item whose straight-line softmax overflowed runs again in the next
  // round (`again`) with the max-first softmax in every phase; such a round
  // takes no new item (qround counts the rounds that do).
  __shared__ int redo_item;  // r + 1 when round r's item must run again
  if (tid == 0) redo_item = 0;
  bool again = false;
  int w_again = 0, qround = 0;
  for (int round = 0;; ++round) {
    int w;
    const bool safe = again;
    if (again) {
      w = w_again;
      again = false;
    } else if (qmode) {
      const int round = qround++;
      w = round == 0 ? cta : uniform((int)q_item[round & 1]);
      if (tid == 0) {
        unsigned nxt = NP + cta;
        if (round > 0) {
          unsigned t = q_tick;
          if (t == kEmpty) t = add_flag(qctr(), 1u);
          nxt = 2 * NP + min(t, kNoTicket);
        }
        q_item[(round + 1) & 1] = nxt;
        q_tick = kEmpty;
      }
      __syncthreads();
      if (w >= list_items) break;
    } else if (p.persistent) {
      const int round = qround++;
      if (round * NP >= list_items) break;
      // snake order: even rounds ascend, odd rounds descend, so every CTA
      // pairs a heavy item with a light one
      w = round * NP + ((round & 1) ? (NP - 1 - cta) : cta);
      if (w >= list_items) continue;
    } else {
      if (qround++ > 0) break;
      w = blockIdx.x;
      if constexpr (SPLIT) {
        split_part<CAUSAL>(p, blockIdx.x, w, part, nparts, t0, t1);
        if (nparts == 0) break;
      }
      if (w >= work_items) break;
    }
    ItemLoc L;
    if (!locate(w, L)) continue;  // query block past the end of this sequence
    const int b = L.b, hq = L.hq, q0 = L.q0, QRS = L.QRS, KRS = L.KRS;
    int Sq = L.Sq, Sk = L.Sk;
    const int q_lo = L.q_lo;
    const long long qbase = L.qbase;
    long long kvbase = L.kvbase;
    const int rw0 = q0 + wave * 32;  // first row of this wave
    const int row = rw0 + li;        // this lane's query row
    int kv_off = Sk - Sq;  // bottom-right causal offset

    // keys [0, kv_end) are streamed for the item; this wave needs [0, wave_end)
    int kv_end = Sk, wave_end = Sk;
    if (CAUSAL) {
      kv_end = min(max(min(Sq, q0 + BM) + kv_off, 0), Sk);
      wave_end = min(max(min(Sq, rw0 + 32) + kv_off, 0), Sk);
    }
    if (rw0 >= Sq) wave_end = 0;
    if constexpr (SPLIT) {
      // a part streams keys [ks, ke) of the item.  Everything below works in
      // key coordinates local to the part: K/V start at key ks, and Sk and
      // the causal offset shrink by ks (a whole number of tiles), so the
      // masks, the mask-free tile counts and the buffer bounds carry over.
      const int ks = t0 * BN, ke = min(t1 * BN, kv_end);
      kvbase += (long long)ks * KRS;
      Sk -= ks;
      kv_off -= ks;
      kv_end = max(ke - ks, 0);
      wave_end = min(max(wave_end - ks, 0), kv_end);
    }
    const int ntiles = (kv_end + BN - 1) / BN;
    // tiles [0, free_tiles) are admissible for every row of this wave, tiles
    // [0, main_tiles) for every row of the workgroup (the mask-free body)
    int free_tiles = Sk / BN, main_tiles = Sk / BN;
    if (CAUSAL) {
      free_tiles = min(free_tiles, max(rw0 + kv_off + 1, 0) / BN);
      main_tiles = min(main_tiles, max(q0 + kv_off + 1, 0) / BN);
    }
    main_tiles = min(main_tiles, ntiles);


    f32x16 oacc[DTILES];
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = f32x16{};
    float m_run = -__builtin_inff();  // exp2 reference max (log2 domain)
    float l_run = 0.f;                // this lane's half of the row sum

    // One group (4 waves) copies the K or the V half of each tile, straight
    // from global memory into LDS (16-byte buffer loads to LDS: lane j of a
    // load writes bytes [16 j, 16 j + 16) after the load's LDS base), so the
    // copy holds no registers and issues no LDS stores.  A tile's LDS image,
    // padding included, is cut into 1 KiB pieces, one per load; image chunk
    // c is row c / RC, column c % RC, and padding columns (>= CH) load from
    // an offset past the buffer, which reads zeros.  Buffer descriptors end
    // right after this (sequence, kv head)'s last key row, so rows >= Sk read
    // zeros too.
    const int kv_bytes = Sk > 0 ? ((Sk - 1) * KRS + D) * 2 : 0;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kg + kvbase), (short)0, kv_bytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(vg + kvbase), (short)0, kv_bytes, kBufferFlags);
    const int gw = wave % (kPrefillWaves / 2);  // wave index inside its group
    // lane's global byte offset for load u of this wave (loads gw, gw+4, ...)
    auto dma_offset = [&](int rc, int u) -> unsigned {
      const int cidx = 64 * (gw + 4 * u) + lane;
      const int rr = cidx / rc, cc = cidx - rr * rc;
      return cc < CH ? (unsigned)((rr * KRS + cc * 8) * 2) : kPastEnd;
    };
    auto dma_tile = [&](__amdgpu_buffer_rsrc_t rs, uint16_t* dst, int t, int ni,
                        const unsigned* offs) {
#pragma unroll
      for (int u = 0; u < kDmaSlots; ++u) {
        if (gw + 4 * u < ni)
          lds_dma16(rs, dst + (gw + 4 * u) * 512, offs[u], t * BN * KRS * 2);
      }
    };

    // ---- the stages of a tile ---------------------------------------------------
    // B1: row max of the tile (log2 domain; the tile is held as NST S
    // accumulators of 32 keys); move the reference max and rescale O and l
    // when some row of the wave jumped above it by > tau
    auto stage_maxn = [&](const f32x16 (&S)[NST]) {
      float mx = fmaxf(fmaxf(S[0][0], S[0][1]), S[1][0]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(fmaxf(mx, S[0][r]), S[1][r - 1]);
      mx = fmaxf(mx, S[1][15]);
#pragma unroll
      for (int st = 2; st < NST; ++st) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, S[st][r]), S[st][r + 1]);
      }
      mx = pair_max(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleTau)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - ((m_new == -__builtin_inff()) ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
    };
    // B2: p = exp2(s c - m), row-sum partial, pack to the P operand
    auto stage_exp = [&](f32x16& S, u32x4 (&P)[2]) {
      const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S[r] = fast_exp2(__builtin_fmaf(S[r], c, -m_use));
        psum += S[r];
      }
      l_run += psum;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int r0 = 8 * kk;
        P[kk] = u32x4{E::pack2(S[r0 + 0], S[r0 + 1]), E::pack2(S[r0 + 2], S[r0 + 3]),
                      E::pack2(S[r0 + 4], S[r0 + 5]), E::pack2(S[r0 + 6], S[r0 + 7])};
      }
    };
    // M step: NPV PV MFMAs then NQK QK MFMAs.
    //   PV (C): O^T += V^T P^T for tile Vb; MFMA j = (sub-tile st, k-step kk,
    //     column tile dt) reads its V^T operand with two transposing reads
    //     of the row-major V tile
    //   QK (A): S^T = K Q^T for tile Kb; MFMA j = (sub-tile st, k-step kk)
    //     reads one 16-byte K row chunk
    auto m_step = [&](auto npv_c, auto nqk_c, const uint16_t* Vb, const uint16_t* Kb,
                      const u32x4 (&P)[NST][2], f32x16 (&S)[NST]) {
      constexpr int NPV = decltype(npv_c)::value, NQK = decltype(nqk_c)::value;
      auto load = [&](auto jc) -> u32x4 {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < NPV) {
          constexpr int st = j / (2 * DTILES), kk = (j / DTILES) % 2, dt = j % DTILES;
          const uint16_t* vrow = Vb + v_lane + (32 * st + 16 * kk) * VST + 32 * dt;
          const u32x2 lo = lds_read_tr16(vrow);
          const u32x2 hi = lds_read_tr16(vrow + 8 * VST);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          constexpr int q = j - NPV, st = q / KSTEPS, kk = q % KSTEPS;
          return lds_read16(Kb + k_lane + 32 * st * KST + 16 * kk);
        }
      };
      auto mfma = [&](auto jc, u32x4 a) {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < NPV) {
          constexpr int st = j / (2 * DTILES), kk = (j / DTILES) % 2, dt = j % DTILES;
          oacc[dt] = E::mfma(a, P[st][kk], oacc[dt]);
        } else {
          constexpr int q = j - NPV, st = q / KSTEPS, kk = q % KSTEPS;
          S[st] = E::mfma(a, qr[kk], kk == 0 ? f32x16{} : S[st]);
        }
      };
      m_pipeline<NPV + NQK, kLookahead>(load, mfma);
    };
    // V step of the straight-line body in the queue-driven launches: p =
    // exp2(s c - m) against the current reference first.  Every p is >= 0,
    // so when no lane's partial row sum exceeds 2^tau no p does, the
    // reference stands, and the tile's row max is not needed at all.
    // Otherwise (rare) the max of p decides: a row whose p went above 2^tau
    // moves its reference up by the binary exponent e of that max and scales
    // its p, l and O by 2^-e (exact), which leaves every p <= 1; a row without
    // a reference yet adopts the one its exps used.  An exp that overflowed
    // leaves l infinite (or NaN): the last phase sees it and the item runs
    // again with the max-first step (the lost scores cannot be formed here
    // without registers the kernel does not have).
    auto stage_fast = [&](f32x16 (&S)[NST], u32x4 (&P)[NST][2]) {
      const bool fresh = m_run == -__builtin_inff();
      const float m_use = fresh ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          S[st][r] = fast_exp2(__builtin_fmaf(S[st][r], c, -m_use));
          psum += S[st][r];
        }
      if (__builtin_amdgcn_ballot_w64(!(psum <= kRescaleGate) || fresh)) {
        float pm = S[0][0];
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) pm = fmaxf(pm, S[st][r]);
        pm = pair_max(pm);
        const int e = pm > kRescaleGate ? __builtin_amdgcn_frexp_expf(pm) : 0;
        if (__builtin_amdgcn_ballot_w64(e != 0)) {
          const float a = __builtin_amdgcn_ldexpf(1.0f, -e);
#pragma unroll
          for (int st = 0; st < NST; ++st) S[st] *= a;
          psum *= a;
          l_run *= a;
#pragma unroll
          for (int dt = 0; dt < DTILES; ++dt) oacc[dt] *= a;
        }
        m_run = m_use + (float)e;
      }
      l_run += psum;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int r0 = 8 * kk;
          P[st][kk] = u32x4{E::pack2(S[st][r0 + 0], S[st][r0 + 1]), E::pack2(S[st][r0 + 2], S[st][r0 + 3]),
                            E::pack2(S[st][r0 + 4], S[st][r0 + 5]), E::pack2(S[st][r0 + 6], S[st][r0 + 7])};
        }
    };

    // ---- ping-pong schedule ----------------------------------------------------
    // Each wave runs the step sequence M(0) V(0) M(1) V(1) ... M(ntiles) over
    // its BN-key tiles:
    //   M(t): S_t = K_t Q^T, then O^T += V_{t-1}^T P_{t-1}^T
    //   V(t): mask (diagonal / tail only), online softmax of S_t -> P_t
    // The two waves that share a SIMD run the sequence one phase apart (waves
    // 0-3 lead, 4-7 follow): while one issues MFMAs the other runs its softmax
    // on the vector unit.  Every phase ends with a workgroup barrier.  LDS
    // holds rings of NBUF K and NBUF V tiles: K(t) is read in phases 2t,
    // 2t+1 and V(t) in 2t+2, 2t+3, so K(X) copied in phase 2X - 2 NBUF + 3
    // and V(X) in phase 2X - 2 NBUF + 4 land after the last read of the tile
    // that held their slot and before the barrier ahead of their first read.
    // ring slot of a tile; readfirstlane keeps it a per-phase scalar instead
    // of letting strength reduction turn every LDS address into a live
    // induction register
    auto slot = [&](int tile) { return uniform((tile + ring) % NBUF); };
    // tile t is needed by this wave iff t*BN < wave_end; sub-tile keys past
    // free_keys need the mask for some row of this wave
    int free_keys = Sk;
    if (CAUSAL) free_keys = min(free_keys, max(rw0 + kv_off + 1, 0));
    const int nphase = ntiles > 0 ? 2 * ntiles + 2 : 0;
    // phases [4, main_end) run straight-line steps: every tile they touch
    // (t-1, t with t <= main_tiles - 2 for the lagging group) is needed by
    // every wave and mask-free
    const int main_end = 2 * main_tiles - 2;

    constexpr int KRC = KST / 8, VRC = VST / 8;        // 16-byte chunks per LDS row
    constexpr int KNI = BN * KRC / 64, VNI = BN * VRC / 64;  // 1 KiB pieces per tile
    static_assert(BN * KRC % 64 == 0 && BN * VRC % 64 == 0, "tile images are whole KiB");
    static_assert(KNI <= 4 * kDmaSlots && VNI <= 4 * kDmaSlots, "copy slots per wave");
    const bool lead = wave < kPrefillWaves / 2;
    // this wave's per-lane source offsets: K pieces for the leading group,
    // V pieces for the following one
    unsigned dma_offs[kDmaSlots];
#pragma unroll
    for (int u = 0; u < kDmaSlots; ++u) dma_offs[u] = dma_offset(lead ? KRC : VRC, u);

    // prologue (unless the item before loaded it): Q, and the leading group
    // copies K of tiles 0 .. NBUF - 2, the following group V of the same tiles
    if (!have_pf) {
      load_q(L);
      if (lead) {
        dma_tile(krs, Ks + slot(0) * KTILE, 0, KNI, dma_offs);
        if (NBUF > 2 && ntiles > 1) dma_tile(krs, Ks + slot(1) * KTILE, 1, KNI, dma_offs);
      } else {
        dma_tile(vrs, Vs + slot(0) * VTILE, 0, VNI, dma_offs);
        if (NBUF > 2 && ntiles > 1) dma_tile(vrs, Vs + slot(1) * VTILE, 1, VNI, dma_offs);
      }
    }
    // the next item of this workgroup, prefetched in this item's last phases
    ItemLoc N;
    bool pf = false;
    __amdgpu_buffer_rsrc_t krs_n = krs, vrs_n = vrs;
    if constexpr (kPrefetch) {
      const int nr = qround;  // the next round that takes an item
      if (!safe && p.persistent && ntiles > 0 && (qmode || nr * NP < list_items)) {
        const int wn = qmode ? uniform((int)q_item[nr & 1]) : nr * NP + ((nr & 1) ? (NP - 1 - cta) : cta);
        if (wn < list_items && locate(wn, N)) {
          pf = true;
          const int nb = N.Sk > 0 ? ((N.Sk - 1) * N.KRS + D) * 2 : 0;
          krs_n = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg + N.kvbase), (short)0,
                                                    nb, kBufferFlags);
          vrs_n = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg + N.kvbase), (short)0,
                                                    nb, kBufferFlags);
        }
      }
    }
    if constexpr (SPLIT) {
      if (!safe && nparts > 1 && tid == 0) split_word[0] = add_flag(p.split_cnt + 2 * w, 1u);
    }
    wait_vmem();
    __syncthreads();
    fold_q();

    auto run = [&](auto lag_c) {
      constexpr int LAG = decltype(lag_c)::value;
      unsigned q_tk = 0;  // (thread 0) ticket in flight across the final two phases
      f32x16 S[NST];   // S of the tile between its M and V steps
      u32x4 P[NST][2];  // P of the tile between its V and next M steps
#pragma unroll
      for (int st = 0; st < NST; ++st) S[st] = f32x16{};
      auto needed = [&](int t) { return t >= 0 && t < ntiles && t * BN < wave_end; };
      // one phase of kind KIND (0: M step, 1: V step) for this wave; ALL: every
      // operation of the step is known to be needed and mask-free
      auto phase = [&](int g, auto kind_c, auto all_c, auto last_c) {
        constexpr int KIND = decltype(kind_c)::value;
        constexpr bool ALL = decltype(all_c)::value;
        // LAST: one of the final two phases (2 ntiles, 2 ntiles + 1), which
        // have no QK product (there is no tile ntiles), so Q is free: the
        // first of them loads the next item's Q, ahead of the next item's
        // K/V copies that the following group issues in the same phase
        constexpr bool LAST = decltype(last_c)::value;
        if constexpr (LAST && kPrefetch) {
          // the ticket for the item after the next one: taken at the start
          // of the first final phase (ahead of the Q loads, so that waiting
          // for it does not wait for them), written to LDS at the end of the
          // second, so the atomic's round trip overlaps both
          if (qmode && !safe && g == nphase - 2 && tid == 0) q_tk = add_flag(qctr(), 1u);
          if (pf && g == nphase - 2) load_q(N);
        }
        // the leading group copies K(X) in its V phase 2X - 2 NBUF + 3, the
        // following group V(X) in its V phase 2X - 2 NBUF + 4 (tiles below
        // NBUF - 1 come with the prologue): the slot it fills was last read
        // in the phase before, and the tile lands before the barrier that
        // precedes its first read
        const int Xld = LAG == 0 ? (g + 2 * NBUF - 3) >> 1 : (g + 2 * NBUF - 4) >> 1;
        // in the straight-line body every V phase copies (a copy of tile
        // ntiles reads zeros past Sk into a ring slot no one reads), so the
        // copy and its completion wait carry no branch: a branch there lets
        // the compiler sink the softmax below the wait and expose the load
        // latency
        const bool do_load = KIND == 1 && (ALL || (Xld >= NBUF - 1 && Xld < ntiles));
        if (do_load) {
          if (LAG == 0) dma_tile(krs, Ks + slot(Xld) * KTILE, Xld, KNI, dma_offs);
          else dma_tile(vrs, Vs + slot(Xld) * VTILE, Xld, VNI, dma_offs);
        }
        if constexpr (KIND == 1 && kPrefetch && !ALL) {
          // this group's last V phase: the slot of tile ntiles was last read
          // a phase ago.  Nothing waits for the copy until the next item
          // starts.
          if (pf && Xld == ntiles) {
            if (LAG == 0) dma_tile(krs_n, Ks + slot(Xld) * KTILE, 0, KNI, dma_offs);
            else dma_tile(vrs_n, Vs + slot(Xld) * VTILE, 0, VNI, dma_offs);
          }
        }
        const int sidx = g - LAG;
        const int t = sidx >> 1;
        if constexpr (KIND == 0 && kMfmaPrio > 0) __builtin_amdgcn_s_setprio(kMfmaPrio);
        if (KIND == 0 && ALL) {
          // M(t), steady state: 2*NST*DTILES PV MFMAs (P_{t-1} dies) then NST*KSTEPS
          // QK MFMAs (S_t is born), LDS reads kLookahead MFMAs ahead
          const uint16_t* Kb = Ks + slot(t) * KTILE;
          const uint16_t* Vb = Vs + slot(t - 1) * VTILE;
          m_step(std::integral_constant<int, NST * 2 * DTILES>{}, std::integral_constant<int, NST * KSTEPS>{},
                 Vb, Kb, P, S);
        } else if (KIND == 0) {
          // M(t): PV of tile t-1, QK of tile t, each when needed by this wave
          if (sidx >= 0 && needed(t - 1)) {
            const uint16_t* Vb = Vs + slot(t - 1) * VTILE;
            m_step(std::integral_constant<int, NST * 2 * DTILES>{}, std::integral_constant<int, 0>{},
                   Vb, Ks, P, S);
          }
          if constexpr (!LAST) {
            if (sidx >= 0 && needed(t)) {
              const uint16_t* Kb = Ks + slot(t) * KTILE;
              m_step(std::integral_constant<int, 0>{}, std::integral_constant<int, NST * KSTEPS>{},
                     Vs, Kb, P, S);
            }
          }
        } else if (ALL || (sidx >= 0 && needed(t))) {
          // V(t): mask and softmax of the BN keys of tile t
          if (!ALL && t * BN + BN > free_keys) {
            // register r of S[st] holds key t*BN + 32 st + 4*lh + off(r): keep
            // keys <= lim = min(row + Sk - Sq, Sk - 1) of this lane's row
            int lim = Sk - 1;
            if (CAUSAL) lim = min(lim, row + kv_off);
            lim -= t * BN + 4 * lh;
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int off = 32 * st + 8 * (r >> 2) + (r & 3);
                S[st][r] = off > lim ? -__builtin_inff() : S[st][r];
              }
          }
          if constexpr (ALL) {
            stage_fast(S, P);
          } else {
            stage_maxn(S);
#pragma unroll
            for (int st = 0; st < NST; ++st) stage_exp(S[st], P[st]);
          }
        }
        if constexpr (KIND == 0 && kMfmaPrio > 0) __builtin_amdgcn_s_setprio(0);
        if constexpr (LAST && kPrefetch) {
          if (qmode && !safe && g == nphase - 1 && tid == 0) q_tick = q_tk;
        }
        if constexpr (LAST) {
          // every softmax step of the item is done: an overflowed exp left l
          // non-finite (seen by all after this phase's barrier)
          if (!safe && g == nphase - 1 &&
              __builtin_amdgcn_ballot_w64(!__builtin_isfinite(l_run)))
            redo_item = round + 1;
        }
        // each phase is its own scheduling region: nothing drifts across the
        // barrier that separates the two waves' roles; the tile copied in
        // this phase has landed in LDS before the barrier
        __builtin_amdgcn_sched_barrier(0);
        if (do_load) wait_vmem();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      };
      // phase g runs step g - LAG: an M step when it is even, a V step when odd
      using K0 = std::integral_constant<int, LAG>;      // kind of even phases
      using K1 = std::integral_constant<int, 1 - LAG>;  // kind of odd phases
      using F = std::false_type;
      using T = std::true_type;
      int g = 0;
      for (; g + 1 < min(4, nphase - 2); g += 2) {
        phase(g, K0{}, F{}, F{});
        phase(g + 1, K1{}, F{}, F{});
      }
      for (; g + 1 < (safe ? 0 : main_end); g += 2) {
        phase(g, K0{}, T{}, F{});
        phase(g + 1, K1{}, T{}, F{});
      }
      for (; g + 1 < nphase - 2; g += 2) {
        phase(g, K0{}, F{}, F{});
        phase(g + 1, K1{}, F{}, F{});
      }
      if (nphase > 0) {
        phase(nphase - 2, K0{}, F{}, T{});
        phase(nphase - 1, K1{}, F{}, T{});
      }
    };
    if (wave < kPrefillWaves / 2) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
    (void)free_tiles;
    if constexpr (kPrefetch) {
      have_pf = pf;
      ring = uniform((ring + ntiles) % NBUF);
    }
    if (redo_item == round + 1) {
      // run the item again in the next round, from its own prologue (the
      // next item's Q and first tile, if prefetched here, are loaded again
      // after it)
      wait_vmem();
      __syncthreads();
      have_pf = false;
      again = true;
      w_again = w;
      continue;
    }

    // ---- epilogue: O = O^T / l, rows < Sq --------------------------------------
    float l_tot = pair_sum(l_run);
    if constexpr (SPLIT) {
      if (nparts > 1 &&
          !merge_parts(p, w, part, nparts, split_word[0], split_word, oacc, m_run, l_tot))
        continue;
    }
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    // With 128-key tiles at D = 128 the wave's O rows go through LDS, so that
    // each global store writes four whole rows instead of 8 bytes of each of
    // 32 rows.  The staging slot is the ring slot of tile ntiles + 1 (ring
    // already advanced past this item): the next item's first tile, when it
    // was prefetched, went to the slot of tile ntiles, a prologue copies into
    // the slot of tile 0 of the next item (that same slot), and every read of
    // this item's tiles ended before the last phase's barrier.  The leading
    // group stages in the K ring, the following group in the V ring, 32 rows
    // of D + 8 elements per wave (8-byte writes and 16-byte row reads
    // without bank conflicts).
    constexpr bool kStagedStore = D == 128 && NBUF == 2;
    if constexpr (kStagedStore) {
      constexpr int OST = D + 8;
      constexpr int LPR = D / 8;        // lanes per row of a store
      constexpr int RPI = 64 / LPR;     // rows per store
      static_assert((kPrefillWaves / 2) * 32 * OST <= KTILE && (kPrefillWaves / 2) * 32 * OST <= VTILE,
                    "four waves' O rows fit a ring slot");
      const int es = uniform((ring + 1) % NBUF);
      uint16_t* ob = (wave < kPrefillWaves / 2 ? Ks + es * KTILE : Vs + es * VTILE) +
                     (wave % (kPrefillWaves / 2)) * 32 * OST;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 pk = {E::pack2(oacc[dt][4 * a + 0] * inv, oacc[dt][4 * a + 1] * inv),
                            E::pack2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(ob + li * OST + 32 * dt + 8 * a + 4 * lh) = pk;
        }
      }
      const int rl = lane / LPR, cl = lane % LPR;
#pragma unroll
      for (int j = 0; j < 32 / RPI; ++j) {
        const int r = RPI * j + rl;
        const u32x4 v = lds_read16(ob + r * OST + 8 * cl);
        if (rw0 + r < Sq)
          *reinterpret_cast<u32x4*>(og + qbase + (long long)(rw0 + r) * QRS + 8 * cl) = v;
      }
    }
    if (row < Sq) {
      if constexpr (!kStagedStore) {
        uint16_t* orow = og + qbase + (long long)row * QRS + 4 * lh;
#pragma unroll
        for (int dt = 0; dt < DTILES; ++dt) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const u32x2 pk = {E::pack2(oacc[dt][4 * a + 0] * inv, oacc[dt][4 * a + 1] * inv),
                              E::pack2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv)};
            *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a) = pk;
          }
        }
      }
      if (LSE && lh == 0) {
        const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        if constexpr (VARLEN) p.lse[(long long)hq * p.total_q + q_lo + row] = lse;
        else p.lse[((long long)b * p.Hq + hq) * Sq + row] = lse;
      }
    }
  }
  if (qmode && tid == 0) {
    // every ticket of this workgroup has been taken and used; the last
    // workgroup to finish leaves the counters at zero for the next launch
    if (add_flag(p.queue + kXcds, 1u) == gridDim.x - 1) {
      for (int x = 0; x < kXcds; ++x) st_flag(p.queue + x, 0u);
      st_flag(p.queue + kXcds, 0u);
    }
  }
}

template <int D, int DT, bool CAUSAL, bool LSE, bool VARLEN, bool SPLIT, bool PF>
hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, DT, CAUSAL, LSE, VARLEN, SPLIT, PF>), dim3(grid),
                     dim3(kPrefillWaves * 64), 0, stream, p);
  return hipGetLastError();
}

// Instances: varlen; dense with the key split; dense persistent with the work
// queue and the cross-item prefetch (measured to pay only together, on long
// launches); and the plain dense kernel for everything else
template <int D, int DT, bool CAUSAL>
hipError_t launch_c(const PrefillParams& p, int grid, hipStream_t stream) {
  const bool lse = p.lse != nullptr;
  if (p.cu_q != nullptr)
    return lse ? launch_one<D, DT, CAUSAL, true, true, false, false>(p, grid, stream)
               : launch_one<D, DT, CAUSAL, false, true, false, false>(p, grid, stream);
  if (p.split_tiles > 0)
    return lse ? launch_one<D, DT, CAUSAL, true, false, true, false>(p, grid, stream)
               : launch_one<D, DT, CAUSAL, false, false, true, false>(p, grid, stream);
  if (p.queue != nullptr && p.persistent)
    return lse ? launch_one<D, DT, CAUSAL, true, false, false, true>(p, grid, stream)
               : launch_one<D, DT, CAUSAL, false, false, false, true>(p, grid, stream);
  return lse ? launch_one<D, DT, CAUSAL, true, false, false, false>(p, grid, stream)
             : launch_one<D, DT, CAUSAL, false, false, false, false>(p, grid, stream);
}

template <int D, int DT>
hipError_t launch_dt(const PrefillParams& p, bool causal, int grid, hipStream_t stream) {
  return causal ? launch_c<D, DT, true>(p, grid, stream) : launch_c<D, DT, false>(p, grid, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int D, int dtype, bool causal, int grid,
                          hipStream_t stream) {
  if (D == 128) {
    return dtype == kBF16 ? launch_dt<128, kBF16>(p, causal, grid, stream)
                          : launch_dt<128, kFP16>(p, causal, grid, stream);
  }
  return dtype == kBF16 ? launch_dt<64, kBF16>(p, causal, grid, stream)
                        : launch_dt<64, kFP16>(p, causal, grid, stream);
}

}  // namespace fa
