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
//  * KV tiles of 64 keys stream through double-buffered, row-padded LDS
//    ("Baked-in levers": K rows padded against bank conflicts, V pad);
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
//    p = exp2(s*c - m) whose argument is <= 0 ("native exp2_fast").
//  * O^T += V^T P^T: P is fed straight from the S accumulator registers as
//    the B operand.  The contraction over keys is permuted to the order in
//    which P already sits in registers, and V (A operand) is read from LDS
//    with the gfx950 transposing read in that same permuted order -- no
//    cross-lane relayout of P ("CK-1 transposed PV" describes the same
//    idea).  O^T keeps one query row per lane, so the rescale by
//    exp2(m_old - m_new) is lane-local and is skipped when no row of the
//    wave raised its max (x * 1.0 == x, so skipping changes no bit).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kKPad = 8;   // K LDS row = D + 8 elements (16-byte skew per row)
constexpr int kVPad = 32;  // V LDS row = D + 32 elements (64-byte skew per row)

// The exp2 reference max of a row moves only when the row's running max
// exceeds it by more than kRescaleTau (log2 units), so p = exp2(s*c - m_ref)
// stays <= 2^kRescaleTau and the O accumulator is rescaled only on the rare
// tiles where some row of the wave jumps that far.  The final O / l and the
// LSE are exact for any reference, so this changes rounding only.
#ifndef FA_RESCALE_TAU
#define FA_RESCALE_TAU 8.0f
#endif
constexpr float kRescaleTau = FA_RESCALE_TAU;
#ifndef FA_MFMA_SETPRIO
#define FA_MFMA_SETPRIO 0
#endif

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

template <int D, int DT, bool CAUSAL, bool LSE>
__global__ __launch_bounds__(kPrefillWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillParams p) {
  using E = Elt<DT>;
  constexpr int NT = kPrefillWaves * 64;
  constexpr int BM = kPrefillBM;
  constexpr int BN = kPrefillBN;
  constexpr int KST = D + kKPad;
  constexpr int VST = D + kVPad;
  constexpr int KSTEPS = D / 16;    // k-steps of the QK product
  constexpr int DTILES = D / 32;    // 32-wide column tiles of O
  constexpr int CH = D / 8;         // 16-byte chunks per K/V row
  constexpr int PER = BN * CH / NT; // chunks per thread per tile
  static_assert(BN * CH % NT == 0, "tile copy must divide evenly");
  static_assert(BN == 64, "the softmax below assumes two 32-key S tiles");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * BN * VST];

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

  const int NP = gridDim.x;
  for (int round = 0;; ++round) {
    int w;
    if (p.persistent) {
      if (round * NP >= p.work_items) break;
      // snake order: even rounds ascend, odd rounds descend, so every CTA
      // pairs a heavy item with a light one
      w = round * NP + ((round & 1) ? (NP - 1 - (int)blockIdx.x) : (int)blockIdx.x);
      if (w >= p.work_items) continue;
    } else {
      if (round > 0) break;
      w = blockIdx.x;
    }
    int b, hq, qb;
    decode_item(p, w, b, hq, qb);
    const int hk = hq / p.gqa;
    const int q0 = qb * BM;
    const int rw0 = q0 + wave * 32;  // first row of this wave
    const int row = rw0 + li;        // this lane's query row
    const long long qbase = (long long)b * p.q_bstride + (long long)hq * p.Sq * D;
    const long long kvbase = (long long)b * p.kv_bstride + (long long)hk * p.Sk * D;

    // keys [0, kv_end) are streamed for the item; this wave needs [0, wave_end)
    int kv_end = p.Sk, wave_end = p.Sk;
    if (CAUSAL) {
      kv_end = min(max(min(p.Sq, q0 + BM) + p.kv_off, 0), p.Sk);
      wave_end = min(max(min(p.Sq, rw0 + 32) + p.kv_off, 0), p.Sk);
    }
    if (rw0 >= p.Sq) wave_end = 0;
    const int ntiles = (kv_end + BN - 1) / BN;
    // tiles [0, free_tiles) are admissible for every row of this wave
    int free_tiles = p.Sk / BN;
    if (CAUSAL) free_tiles = min(free_tiles, max(rw0 + p.kv_off + 1, 0) / BN);

    // Q rows of this wave as the B operand: lane holds q[row][16kk + 8lh .. +7]
    u32x4 qr[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < p.Sq) x = gload16(qg + qbase + (long long)row * D + 16 * kk + 8 * lh);
      if (p.q_sign < 0) x ^= 0x80008000u;
      if (p.q_sign == 0) x = u32x4{0u, 0u, 0u, 0u};
      qr[kk] = x;
    }

    f32x16 oacc[DTILES];
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = f32x16{};
    float m_run = -__builtin_inff();
    float l_run = 0.f;

    // global -> registers -> LDS staging of one KV tile
    u32x4 kst[PER], vst[PER];
    auto gload_tile = [&](int t) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int cidx = tid + u * NT;
        const int rr = cidx / CH, cc = cidx % CH;
        const int key = t * BN + rr;
        u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
        if (key < p.Sk) {
          const long long off = kvbase + (long long)key * D + cc * 8;
          kx = gload16(kg + off);
          vx = gload16(vg + off);
        }
        kst[u] = kx;
        vst[u] = vx;
      }
    };
    auto lstore_tile = [&](int buf) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int cidx = tid + u * NT;
        const int rr = cidx / CH, cc = cidx % CH;
        lds_write16(Ks + buf * BN * KST + rr * KST + cc * 8, kst[u]);
        lds_write16(Vs + buf * BN * VST + rr * VST + cc * 8, vst[u]);
      }
    };

    if (ntiles > 0) {
      gload_tile(0);
      lstore_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) gload_tile(t + 1);

      if (t * BN < wave_end) {
        const uint16_t* Kb = Ks + buf * BN * KST;
        const uint16_t* Vb = Vs + buf * BN * VST;
        // ---- S^T = K Q^T for keys [t*BN, t*BN + 64) --------------------------
        f32x16 s0 = f32x16{}, s1 = f32x16{};
        if (FA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const u32x4 a0 = lds_read16(Kb + k_lane + 16 * kk);
          const u32x4 a1 = lds_read16(Kb + k_lane + 32 * KST + 16 * kk);
          s0 = E::mfma(a0, qr[kk], s0);
          s1 = E::mfma(a1, qr[kk], s1);
        }
        if (FA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(0);
        // ---- mask (diagonal / tail tiles only) -----------------------------
        if (t >= free_tiles) {
          const int kb = t * BN + 4 * lh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j0 = kb + 8 * (r >> 2) + (r & 3);
            const int j1 = j0 + 32;
            bool bad0 = j0 >= p.Sk, bad1 = j1 >= p.Sk;
            if (CAUSAL) {
              bad0 = bad0 || (j0 > row + p.kv_off);
              bad1 = bad1 || (j1 > row + p.kv_off);
            }
            if (bad0) s0[r] = -__builtin_inff();
            if (bad1) s1[r] = -__builtin_inff();
          }
        }
        // ---- online softmax -------------------------------------------------
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
        mx = pair_max(mx) * c;  // this tile's row max, log2 domain
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleTau)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = fast_exp2(m_run - ((m_new == -__builtin_inff()) ? 0.f : m_new));
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < DTILES; ++dt) oacc[dt] *= alpha;
          m_run = m_new;
        }
        const float m_use = (m_run == -__builtin_inff()) ? 0.f : m_run;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = fast_exp2(__builtin_fmaf(s0[r], c, -m_use));
          s1[r] = fast_exp2(__builtin_fmaf(s1[r], c, -m_use));
          psum += s0[r] + s1[r];
        }
        l_run += psum;
        // ---- O^T += V^T P^T ---------------------------------------------------
        if (FA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const f32x16& sp = st ? s1 : s0;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int r0 = 8 * kk;
            const u32x4 pb = {E::pack2(sp[r0 + 0], sp[r0 + 1]), E::pack2(sp[r0 + 2], sp[r0 + 3]),
                              E::pack2(sp[r0 + 4], sp[r0 + 5]), E::pack2(sp[r0 + 6], sp[r0 + 7])};
            const uint16_t* vrow = Vb + v_lane + (32 * st + 16 * kk) * VST;
#pragma unroll
            for (int dt = 0; dt < DTILES; ++dt) {
              const u32x2 lo = lds_read_tr16(vrow + 32 * dt);
              const u32x2 hi = lds_read_tr16(vrow + 8 * VST + 32 * dt);
              const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
              oacc[dt] = E::mfma(a, pb, oacc[dt]);
            }
          }
        }
        if (FA_MFMA_SETPRIO) __builtin_amdgcn_s_setprio(0);
      }

      if (t + 1 < ntiles) lstore_tile(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: O = O^T / l, rows < Sq --------------------------------------
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    if (row < p.Sq) {
      uint16_t* orow = og + qbase + (long long)row * D + 4 * lh;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const u32x2 pk = {E::pack2(oacc[dt][4 * a + 0] * inv, oacc[dt][4 * a + 1] * inv),
                            E::pack2(oacc[dt][4 * a + 2] * inv, oacc[dt][4 * a + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a) = pk;
        }
      }
      if (LSE && lh == 0) {
        const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
        p.lse[((long long)b * p.Hq + hq) * p.Sq + row] = lse;
      }
    }
  }
}

template <int D, int DT, bool CAUSAL, bool LSE>
hipError_t launch_one(const PrefillParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<D, DT, CAUSAL, LSE>), dim3(grid), dim3(kPrefillWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_dt(const PrefillParams& p, bool causal, int grid, hipStream_t stream) {
  const bool lse = p.lse != nullptr;
  if (causal) return lse ? launch_one<D, DT, true, true>(p, grid, stream)
                         : launch_one<D, DT, true, false>(p, grid, stream);
  return lse ? launch_one<D, DT, false, true>(p, grid, stream)
             : launch_one<D, DT, false, false>(p, grid, stream);
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
