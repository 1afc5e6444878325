// Attention backward pass for gfx950: dQ, dK, dV of O = softmax(scale Q K^T +
// mask) V given dO and the forward's row log-sum-exp, as three kernels in the
// textbook FA-2 split (tessera PR page, flash_attn backward commit: a pre-pass
// for D = rowsum(O * dO), dK/dV per key tile, dQ per query tile; P and dS are
// recomputed tile by tile, no score matrix is stored):
//
//   pre   D_i = sum_d dO[i,d] O[i,d]                                 (fp32)
//   dq    per 256 query rows (8 waves, Q and dO in registers), 32-key K/V
//         tiles: S^T = K Q^T, dP^T = V dO^T, P = exp2(S c - LSE_i log2 e),
//         dS = P (dP - D_i), dQ^T += K^T dS^T
//   dkdv  per 128 keys (8 waves, K and V in LDS), 32-row Q/dO tiles:
//         S = Q K^T, dP = dO V^T, P and dS as above, dV^T += dO^T P,
//         dK^T += Q^T dS; the query heads of a GQA group add into their kv
//         head inside the loop, so no atomics are needed anywhere
//
// Both main kernels follow the forward: two groups of 4 waves, one wave of
// each per SIMD, run one phase apart (MFMA phase against vector phase), with
// a workgroup barrier per phase; tiles are copied by buffer loads straight to
// LDS in the vector phases; every product runs on the 32x32x16 matrix core
// with the forward's operand layouts (transposed operands from the gfx950
// transposing LDS read, P and dS fed from the accumulator registers in their
// register order).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// LDS rows of every tile are padded to D + 8 elements.  A 16-byte row read
// serves 16 lanes of consecutive rows per pass; at this stride their rows
// start on distinct 4-bank groups of the 128 banks, so row reads never
// conflict.  Tiles that are also read by the transposing read (8 consecutive
// rows of 64 bytes per instruction, which need 8 disjoint 16-bank groups)
// keep row r of each 32-row block at position tr_pos(r) = 4 (r % 8) + r / 8:
// the 8 rows of a transposing read then sit 4 positions apart, 16 banks
// apart, and any 16 consecutive rows still fall on 16 distinct positions
// mod 32, so neither read conflicts.  Offsets of both reads stay
// compile-time constants on top of a per-lane base (row r of a transposing
// read is 16 kk + 8 h + e with e = 0..7 the lane's: position 4 e + 2 kk + h).
constexpr int kRowPad = 8;
__device__ __forceinline__ int tr_pos(int r) { return 32 * (r >> 5) + 4 * (r & 7) + ((r >> 3) & 3); }
__device__ __forceinline__ int tr_row(int pos) {
  return 32 * (pos >> 5) + 8 * (pos & 3) + ((pos >> 2) & 7);
}
// MFMAs an LDS operand read runs ahead of its use
#ifndef FA_BWD_PIPE
#define FA_BWD_PIPE 4
#endif
constexpr int kPipe = FA_BWD_PIPE;
// dQ kernel: keys per K/V tile (32; 64 needs more registers than two waves
// per SIMD allow at D = 128), waves per workgroup (two groups)
#ifndef FA_BWD_DQ_KEYS
#define FA_BWD_DQ_KEYS 32
#endif
constexpr int kDqKeys = FA_BWD_DQ_KEYS;
constexpr int kDqWaves = 8;
// dK/dV kernel: waves per workgroup (two groups of 4 sharing the block's keys)
// and keys per workgroup
constexpr int kDkdvWaves = 8;
constexpr int kDkdvKeys = 128;
// dK/dV: operand pairs (both MFMA operands from LDS) read this many MFMAs ahead
#ifndef FA_BWD_PAIR_PIPE
#define FA_BWD_PAIR_PIPE 3
#endif
constexpr int kPairPipe = FA_BWD_PAIR_PIPE;

// ---- pre: D_i = rowsum(dO * O), 8 threads per row ------------------------------
template <int D, int DT>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  using E = Elt<DT>;
  constexpr int PER = D / 8;  // elements per thread
  const long long rows = (long long)p.B * p.Hq * p.Sq;
  const long long row = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const uint16_t* o = static_cast<const uint16_t*>(p.o) + row * D + part * PER;
    const uint16_t* g = static_cast<const uint16_t*>(p.dout) + row * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      const u32x4 a = gload16(o + c), b = gload16(g + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += E::widen((unsigned short)(a[i] & 0xFFFFu)) * E::widen((unsigned short)(b[i] & 0xFFFFu));
        acc += E::widen((unsigned short)(a[i] >> 16)) * E::widen((unsigned short)(b[i] >> 16));
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  if (row < rows && part == 0) p.dsum[row] = acc;
}

// ---- dq: one workgroup of 8 waves per (batch, query head, 256 query rows) ---------
// The forward's structure: each wave owns 32 rows (Q and dO resident in
// registers as B operands), the two wave groups walk the same 32-key K/V
// tiles one phase apart:
//   M(t): dQ^T += K^T dS^T of tile t - 1 (K^T by transposing reads), then
//         S^T = K Q^T and dP^T = V dO^T of tile t: 24 MFMAs a wave, one
//         software pipeline of LDS reads ahead of the MFMAs
//   V(t): P = exp2(S c - LSE log2 e) masked, dS = P (dP - D), packed, and
//         the copies of the ring below
// K(t) is read as rows in phases 2t, 2t + 1 and transposed in 2t + 2, 2t + 3;
// V(t) as rows in 2t, 2t + 1.  So K has a ring of three slots and V of two:
// the leading group copies K(X) in phase 2X - 1 into the slot of K(X - 3),
// last read in 2X - 3; the following group copies V(X) in phase 2X - 2 into
// the slot of V(X - 2), last read in 2X - 3; each copy lands before the
// barrier ahead of its first read.
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kDqWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  using E = Elt<DT>;
  constexpr int BM = 32 * kDqWaves;      // query rows per workgroup
  constexpr int BN = kDqKeys;            // keys per K/V tile (32-key sub-tiles)
  constexpr int NST = BN / 32;
  constexpr int KSTEPS = D / 16, DTILES = D / 32;
  constexpr int KST = D + kRowPad;       // K: row reads (S) and transposed reads (dQ), tr_pos order
  constexpr int VST = D + kRowPad;       // V: row reads (dP)
  constexpr int KRC = KST / 8, VRC = VST / 8;
  static_assert(KRC == VRC, "K and V images share their copy offsets");
  // 1 KiB pieces per tile image, rounded up: the chunks past the tile's BN
  // rows land in the slot's tail and are never read
  constexpr int KNI = (BN * KRC + 63) / 64, VNI = (BN * VRC + 63) / 64;
  constexpr int KT = KNI * 512, VT = VNI * 512;             // slot sizes in elements
  constexpr int KPW = (KNI + 3) / 4, VPW = (VNI + 3) / 4;   // pieces per wave of a group
  __shared__ __attribute__((aligned(16))) uint16_t Ks[3 * KT];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * VT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5, ti = lane & 15;
  const int grp = wave >> 2, gw = wave & 3;
  // items heaviest first: query block level descending, then batch and head.
  // Workgroup i runs on XCD i % kXcds; each XCD gets a contiguous run of the
  // level's (batch, head) items, so the query heads of a kv head run on one
  // XCD and stream its K/V through one L2
  const int nqb = (p.Sq + BM - 1) / BM;
  const int per_lvl = p.B * p.Hq;
  const int lvl = (int)blockIdx.x / per_lvl, pos = (int)blockIdx.x - lvl * per_lvl;
  const int rr0 = per_lvl % kXcds == 0 ? (pos % kXcds) * (per_lvl / kXcds) + pos / kXcds : pos;
  const int qb = nqb - 1 - lvl, b = rr0 / p.Hq, hq = rr0 - b * p.Hq;
  const int hk = hq / p.gqa;
  const int q0 = qb * BM, rw0 = q0 + wave * 32, row = rw0 + li;
  const int Sq = p.Sq, Sk = p.Sk, kv_off = Sk - Sq;
  const long long qbase = ((long long)b * p.Hq + hq) * Sq * D;   // q, dO, dQ
  const long long kvbase = ((long long)b * p.Hkv + hk) * Sk * D;

  // Q (sign-folded) and dO rows as B operands: lane row li, d = 16 kk + 8 lh + e
  u32x4 qr[KSTEPS], gr[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (row < Sq) {
      x = gload16(static_cast<const uint16_t*>(p.q) + qbase + (long long)row * D + 16 * kk + 8 * lh);
      y = gload16(static_cast<const uint16_t*>(p.dout) + qbase + (long long)row * D + 16 * kk +
                  8 * lh);
    }
    if (p.q_sign < 0) x ^= 0x80008000u;
    if (p.q_sign == 0) x = u32x4{0u, 0u, 0u, 0u};
    qr[kk] = x;
    gr[kk] = y;
  }
  const long long srow = ((long long)b * p.Hq + hq) * Sq + row;
  const float lse2 = row < Sq ? p.lse[srow] * kLog2e : 0.f;
  const float dr = row < Sq ? p.dsum[srow] : 0.f;
  const float c = p.c_log2;

  // keys [0, kv_end) are streamed for the workgroup; this wave needs [0, wave_end)
  int kv_end = Sk, wave_end = Sk;
  if (CAUSAL) {
    kv_end = min(max(min(Sq, q0 + BM) + kv_off, 0), Sk);
    wave_end = min(max(min(Sq, rw0 + 32) + kv_off, 0), Sk);
  }
  if (rw0 >= Sq) wave_end = 0;
  const int ntiles = (kv_end + BN - 1) / BN;
  // the transposing read's lane base: row e = 4 lh + ti / 4 of 8 at position 4 e
  const int v_lane = 4 * (4 * lh + (ti >> 2)) * KST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);
  const int k_row = tr_pos(li) * KST + 8 * lh;  // row li of a 32-key sub-tile

  // tile copies: the leading group copies K images, the following group V
  const int kv_bytes = Sk > 0 ? Sk * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.k) + kvbase)),
      (short)0, kv_bytes, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.v) + kvbase)),
      (short)0, kv_bytes, kBufferFlags);
  const bool lead = grp == 0;
  constexpr int NPW = KPW > VPW ? KPW : VPW;
  // image chunk c: LDS row c / KRC (K: the position of key tr_row of it),
  // column c % KRC; the slot's tail past BN rows reads zeros
  unsigned offs[NPW];
#pragma unroll
  for (int u = 0; u < NPW; ++u) {
    const int cidx = 64 * (gw + 4 * u) + lane;
    const int pos = cidx / KRC, cc = cidx - pos * KRC;
    const int rr = lead ? tr_row(pos) : pos;
    offs[u] = (pos < BN && cc < D / 8) ? (unsigned)((rr * D + cc * 8) * 2) : kPastEnd;
  }
  auto copy = [&](int X) {
    if (lead) {
      uint16_t* dst = Ks + (X % 3) * KT;
#pragma unroll
      for (int u = 0; u < KPW; ++u)
        if (gw + 4 * u < KNI) lds_dma16(krs, dst + (gw + 4 * u) * 512, offs[u], X * BN * D * 2);
    } else {
      uint16_t* dst = Vs + (X % 2) * VT;
#pragma unroll
      for (int u = 0; u < VPW; ++u)
        if (gw + 4 * u < VNI) lds_dma16(vrs, dst + (gw + 4 * u) * 512, offs[u], X * BN * D * 2);
    }
  };
  if (ntiles > 0) copy(0);
  // the third K slot is first filled in phase 3: zeros until then, so the
  // dQ half of M(0) multiplies finite values (by a zero dS)
  for (int i = tid; i < KT / 8; i += kDqWaves * 64)
    lds_write16(Ks + 2 * KT + 8 * i, u32x4{0u, 0u, 0u, 0u});
  wait_vmem();
  __syncthreads();

  f32x16 dq[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) dq[dt] = f32x16{};

  auto run = [&](auto lag_c) {
    constexpr int LAG = decltype(lag_c)::value;
    f32x16 S[NST], dP[NST];  // the tile between its M and V steps
    u32x4 db[NST][2];        // dS of the tile between its V and next M steps
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      S[st] = f32x16{};
      dP[st] = f32x16{};
      db[st][0] = db[st][1] = u32x4{0u, 0u, 0u, 0u};
    }
    auto needed = [&](int t) { return t >= 0 && t < ntiles && t * BN < wave_end; };
    const int nphase = ntiles > 0 ? 2 * ntiles + 2 : 0;
    auto phase = [&](int g, auto kind_c) {
      constexpr int KIND = decltype(kind_c)::value;
      const int step = g - LAG;
      const int t = step >> 1;
      // copies: K(X) by the leading group in phase 2X - 1, V(X) by the
      // following group in phase 2X - 2 (both V phases of their group)
      const int Xk = (g + 1) >> 1, Xv = (g >> 1) + 1;
      bool do_load = false;
      if constexpr (KIND == 1) {
        if (LAG == 0 && (g & 1) && Xk < ntiles) {
          copy(Xk);
          do_load = true;
        }
        if (LAG == 1 && !(g & 1) && Xv < ntiles) {
          copy(Xv);
          do_load = true;
        }
      }
      if (KIND == 0 && step >= 0) {
        // ---- M(t): dQ of tile t - 1, then S and dP of tile t, as one
        // pipeline (the first S/dP operands are read during the last dQ
        // MFMAs instead of after them)
        const uint16_t* Kp = Ks + ((t + 2) % 3) * KT;  // K(t - 1)
        auto load_q = [&](auto jc) -> u32x4 {
          constexpr int j = decltype(jc)::value, dt = j % DTILES, kk = (j / DTILES) % 2;
          constexpr int st = j / (2 * DTILES);
          const uint16_t* kr = Kp + v_lane + (32 * st + 2 * kk) * KST + 32 * dt;
          const u32x2 lo = lds_read_tr16(kr), hi = lds_read_tr16(kr + KST);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto mfma_q = [&](auto jc, u32x4 a) {
          constexpr int j = decltype(jc)::value, dt = j % DTILES, kk = (j / DTILES) % 2;
          constexpr int st = j / (2 * DTILES);
          dq[dt] = E::mfma(a, db[st][kk], dq[dt]);
        };
        const uint16_t* Kb = Ks + (t % 3) * KT;
        const uint16_t* Vb = Vs + (t % 2) * VT;
        // S^T = K Q^T and dP^T = V dO^T, alternating
        auto load_s = [&](auto jc) -> u32x4 {
          constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
          if constexpr (j % 2) return lds_read16(Vb + (32 * st + li) * VST + 16 * kk + 8 * lh);
          else return lds_read16(Kb + k_row + 32 * st * KST + 16 * kk);
        };
        auto mfma_s = [&](auto jc, u32x4 a) {
          constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
          if constexpr (j % 2) dP[st] = E::mfma(a, gr[kk], kk == 0 ? f32x16{} : dP[st]);
          else S[st] = E::mfma(a, qr[kk], kk == 0 ? f32x16{} : S[st]);
        };
        // Both halves run in every M step (one code path keeps the
        // register allocation at two waves per SIMD without spills).  A dQ
        // half without a tile t - 1 adds exact zeros: dS is zero until the
        // first V step and is zeroed by every V step whose tile this wave
        // skips, and the K slot it reads holds finite data (K tiles, or the
        // zeros the third slot starts with).  S and dP of a tile the wave
        // does not need are never read.
        constexpr int NQ = 2 * NST * DTILES, NS = 2 * NST * KSTEPS;
        auto load = [&](auto jc) -> u32x4 {
          constexpr int j = decltype(jc)::value;
          if constexpr (j < NQ) return load_q(jc);
          else return load_s(std::integral_constant<int, j - NQ>{});
        };
        auto mfma = [&](auto jc, u32x4 a) {
          constexpr int j = decltype(jc)::value;
          if constexpr (j < NQ) mfma_q(jc, a);
          else mfma_s(std::integral_constant<int, j - NQ>{}, a);
        };
        m_pipeline<NQ + NS, kPipe>(load, mfma);
      } else if (KIND == 1 && step >= 0 && needed(t)) {
        // ---- V(t): lane = query row; register r of sub-tile st is key
        // t*BN + 32 st + 8 (r/4) + 4 lh + r%4.  Every exp2 is evaluated and
        // masked pairs are selected to 0 (no branch).
        const bool full = rw0 + 32 <= Sq && (t + 1) * BN <= Sk &&
                          (!CAUSAL || t * BN + BN - 1 <= rw0 + kv_off);
        auto grad = [&](auto mask_c) {
          constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
          for (int st = 0; st < NST; ++st) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = t * BN + 32 * st + 8 * (r >> 2) + 4 * lh + (r & 3);
              const bool ok = !MASK || (row < Sq && key < Sk && (!CAUSAL || key <= row + kv_off));
              const float e = fast_exp2(__builtin_fmaf(S[st][r], c, -lse2));
              const float pr = ok ? e : 0.f;
              S[st][r] = pr * (dP[st][r] - dr);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              const int r0 = 8 * kk;
              db[st][kk] = u32x4{E::pack2(S[st][r0 + 0], S[st][r0 + 1]),
                                 E::pack2(S[st][r0 + 2], S[st][r0 + 3]),
                                 E::pack2(S[st][r0 + 4], S[st][r0 + 5]),
                                 E::pack2(S[st][r0 + 6], S[st][r0 + 7])};
            }
          }
        };
        if (full) grad(std::false_type{});
        else grad(std::true_type{});
      } else if (KIND == 1 && step >= 0) {
        // a tile this wave skips: the next M step's dQ half adds zeros
#pragma unroll
        for (int st = 0; st < NST; ++st) db[st][0] = db[st][1] = u32x4{0u, 0u, 0u, 0u};
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_load) wait_vmem();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    using K0 = std::integral_constant<int, LAG>;
    using K1 = std::integral_constant<int, 1 - LAG>;
    for (int g = 0; g < nphase; g += 2) {
      phase(g, K0{});
      phase(g + 1, K1{});
    }
  };
  if (lead) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  // dQ = scale * (dS K): lane row li, d = 32 dt + 8 (r/4) + 4 lh + r%4
  if (row < Sq) {
    uint16_t* orow = static_cast<uint16_t*>(p.dq) + qbase + (long long)row * D + 4 * lh;
    const float sc = p.scale;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const u32x2 pk = {E::pack2(dq[dt][4 * a + 0] * sc, dq[dt][4 * a + 1] * sc),
                          E::pack2(dq[dt][4 * a + 2] * sc, dq[dt][4 * a + 3] * sc)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * a) = pk;
      }
  }
}

// the two operands of one MFMA, both read from LDS
struct OpPair {
  u32x4 a, b;
};

// ---- dkdv: one workgroup of 8 waves per (batch, kv head, 128 keys) ---------------
// Waves w and w + 4 own the same 32 keys (K and V rows of the block stay in
// LDS, read as B operands) and take alternate 32-row query tiles of the
// (row tile, query head of the group) list, row tiles from the last down and
// heads innermost: the leading group (waves 0-3) the
// even tiles, the following group the odd ones.  The two groups run the
// forward's ping-pong one phase apart, so the wave pair of a SIMD alternates
// MFMA and vector work:
//   M(t): dV^T += dO^T P and dK^T += Q^T dS of the group's tile t - 1 (dO^T, Q^T
//         by transposing reads, P and dS from registers in their register
//         order), then S = Q K^T and dP = dO V^T of its tile t: 32 MFMAs a wave
//   V(t): P = exp2(S c - LSE log2 e) masked, dS = P (dP - D), packed to the
//         input type; and the copy of the group's tile t + 1 into its LDS ring
//         slot (buffer loads straight to LDS: no registers, no LDS stores)
// Tile t is read as rows in M(t) and transposed in M(t + 1), so two ring slots
// per group suffice: tile t + 1 lands in the slot of tile t - 1, whose last
// read was in the M(t) just before.  At the end the following group's fp32
// partial sums go through LDS and the leading group adds them (in that fixed
// order, so results are deterministic) and writes dK = scale dK^T^T, dV.
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kDkdvWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p) {
  using E = Elt<DT>;
  constexpr int BM = 32;                 // query rows per tile
  constexpr int KSTEPS = D / 16, DTILES = D / 32;
  constexpr int KST = D + kRowPad;       // K, V rows: 16-byte row reads only
  constexpr int QST = D + kRowPad;       // Q, dO rows: row and transposed reads, tr_pos order
  constexpr int KV = kDkdvKeys * KST;    // elements of the block's K (or V)
  constexpr int KRC = KST / 8, QRC = QST / 8;       // 16-byte chunks per LDS row
  constexpr int KNI = kDkdvKeys * KRC / 64;         // 1 KiB pieces of a K (or V) image
  constexpr int QNI = (BM * QRC + 63) / 64;         // 1 KiB pieces of a Q (or dO) tile, rounded up
  constexpr int TILE = QNI * 512;                   // elements of one Q (or dO) slot
  static_assert(kDkdvKeys * KRC % 64 == 0, "K and V images are whole KiB");
  constexpr int NPW = (2 * QNI + 3) / 4;            // tile pieces per wave of a group
  // LDS: K, V | Q tiles [group][slot] | dO tiles [group][slot] | LSE, D [group][slot][64]
  constexpr int Q_OFF = 2 * KV, G_OFF = Q_OFF + 4 * TILE, LD_OFF = G_OFF + 4 * TILE;
  constexpr int LDS_ELEMS = LD_OFF + 2 * 4 * 64 * 2;   // floats as pairs of elements
  // the final reduction: 4 waves x 64 lanes x (dK and dV: D floats per lane)
  static_assert(LDS_ELEMS * 2 >= (kDkdvWaves / 2) * 64 * D * 4, "the final reduction fits");
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS_ELEMS];
  uint16_t* const Ks = lds;
  uint16_t* const Vs = lds + KV;
  float* const LD = reinterpret_cast<float*>(lds + LD_OFF);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int li = lane & 31, lh = lane >> 5, ti = lane & 15;
  // blocks key-block-major: the heaviest causal key blocks of every head first
  const int nkb = (p.Sk + kDkdvKeys - 1) / kDkdvKeys;
  const int units = p.B * p.Hkv;
  const int kb = (int)blockIdx.x / units, unit = (int)blockIdx.x - kb * units;
  const int hk = unit % p.Hkv, b = unit / p.Hkv;
  const int k0 = kb * kDkdvKeys, kw0 = k0 + 32 * gw, key = kw0 + li;
  const int Sq = p.Sq, Sk = p.Sk, kv_off = Sk - Sq;
  const long long kvbase = ((long long)b * p.Hkv + hk) * Sk * D;
  const float c = p.c_log2;
  (void)nkb;

  // row tiles that see a key of this block: row + kv_off >= k0 when causal;
  // the (row tile, query head g of the group) list runs the row tiles from
  // the last one down with g innermost.  Every key block of a kv head then
  // starts on the same last row tile and walks the rows in step with the
  // others, so the workgroups of that kv head read each Q/dO tile at about
  // the same time and share it in L2 instead of streaming it separately.
  const int r_first = CAUSAL ? (max(0, k0 - kv_off) / BM) * BM : 0;
  const int nrt = r_first < Sq ? (Sq - r_first + BM - 1) / BM : 0;
  const int total = p.gqa * nrt;
  const int n_lead = (total + 1) / 2, n_mine = grp == 0 ? n_lead : total / 2;
  auto tile_row0 = [&](int t) {  // first row of this group's tile t
    const int it = 2 * t + grp;
    return r_first + (nrt - 1 - it / p.gqa) * BM;
  };
  auto tile_head = [&](int t) { return hk * p.gqa + (2 * t + grp) % p.gqa; };

  // ---- copies (buffer loads to LDS, 1 KiB pieces; lane j of a load writes
  // bytes [16 j, 16 j + 16) of its piece).  Image chunk c is row c / RC,
  // column c % RC; padding columns and rows past the range read zeros.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.k) + kvbase)),
      (short)0, Sk * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.v) + kvbase)),
      (short)0, Sk * D * 2, kBufferFlags);
  {
    // the block's K and V images, all 8 waves
    for (int u = wave; u < 2 * KNI; u += kDkdvWaves) {
      const int pc = u < KNI ? u : u - KNI;
      const int cidx = 64 * pc + lane;
      const int rr = cidx / KRC, cc = cidx - rr * KRC;
      const unsigned off = cc < D / 8 ? (unsigned)(((k0 + rr) * D + cc * 8) * 2) : kPastEnd;
      lds_dma16(u < KNI ? krs : vrs, (u < KNI ? Ks : Vs) + pc * 512, off, 0);
    }
  }
  // this wave's per-lane source offsets inside a tile: pieces gw, gw + 4, ...
  // of the Q image (pieces < QNI) then the dO image
  unsigned toff[NPW];
#pragma unroll
  for (int i = 0; i < NPW; ++i) {
    const int pc = gw + 4 * i;
    const int pp = pc < QNI ? pc : pc - QNI;
    const int cidx = 64 * pp + lane;
    const int pos = cidx / QRC, cc = cidx - pos * QRC;
    toff[i] = (pos < BM && cc < D / 8) ? (unsigned)((tr_row(pos) * D + cc * 8) * 2) : kPastEnd;
  }
  // copy this group's tile t into ring slot t % 2 (the group's 4 waves), with
  // the rows' LSE and D (wave gw == 0, 64 rows from r0, those past Sq zero)
  auto copy_tile = [&](int t) {
    const int r0 = tile_row0(t), hq = tile_head(t), slot = t & 1;
    const int valid = min(BM, Sq - r0);
    const long long qoff = (((long long)b * p.Hq + hq) * Sq + r0) * D;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.q) + qoff)),
        (short)0, valid * D * 2, kBufferFlags);
    const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(static_cast<const void*>(static_cast<const uint16_t*>(p.dout) + qoff)),
        (short)0, valid * D * 2, kBufferFlags);
    uint16_t* qd = lds + Q_OFF + (grp * 2 + slot) * TILE;
    uint16_t* gd = lds + G_OFF + (grp * 2 + slot) * TILE;
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      const int pc = gw + 4 * i;
      if (pc < QNI) lds_dma16(qrs, qd + pc * 512, toff[i], 0);
      else if (pc < 2 * QNI) lds_dma16(grs, gd + (pc - QNI) * 512, toff[i], 0);
    }
    if (gw == 0) {
      const long long srow = ((long long)b * p.Hq + hq) * Sq + r0;
      const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p.lse + srow), (short)0, valid * 4, kBufferFlags);
      const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc(
          p.dsum + srow, (short)0, valid * 4, kBufferFlags);
      float* l = LD + ((grp * 2 + slot) * 2) * 64;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (__attribute__((address_space(3))) void*)l, 4,
                                               lane * 4, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(l + 64),
                                               4, lane * 4, 0, 0, 0);
    }
  };
  if (n_mine > 0) copy_tile(0);
  wait_vmem();
  __syncthreads();

  f32x16 dk[DTILES], dv[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  // the transposing read's lane base: row e = 4 lh + ti / 4 of 8 at position 4 e
  const int v_lane = 4 * (4 * lh + (ti >> 2)) * QST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);
  const int q_row = tr_pos(li) * QST + 8 * lh;  // row li of a tile
  // the wave's keys as B operands: key kw0 + li, d = 16 kk + 8 lh + e
  const uint16_t* const kb_row = Ks + (32 * gw + li) * KST + 8 * lh;
  const uint16_t* const vb_row = Vs + (32 * gw + li) * KST + 8 * lh;
  // K is the B operand of S = q_sign * Q K^T: the sign of the scale goes on
  // the scores (exact), Q and K stay as stored
  const float cs = p.q_sign == 0 ? 0.f : (p.q_sign < 0 ? -c : c);

  // tile t of this group is needed by this wave when the wave has keys and
  // (causal) some pair of the tile is admissible
  auto needed = [&](int t) {
    if (t < 0 || t >= n_mine || kw0 >= Sk) return false;
    return !CAUSAL || kw0 <= tile_row0(t) + BM - 1 + kv_off;
  };

  f32x16 S, dP;         // the tile between its M and V steps
  u32x4 pb[2], db[2];   // P and dS of the tile between its V and next M steps
  // the LSE and D of the rows of registers 0-7 of the tile between its M and
  // V steps: read from LDS at the start of the M step, whose MFMAs hide the
  // read's latency (the LDS queue is long while the other group's M step
  // streams its operands)
  f32x4 lse_a[2] = {}, d_a[2] = {};
  S = f32x16{};
  dP = f32x16{};
  auto run = [&](auto lag_c) {
    constexpr int LAG = decltype(lag_c)::value;
    const int nphase = n_lead > 0 ? 2 * n_lead + 2 : 0;
    // one phase of kind KIND (0: M step, 1: V step) of this group
    auto phase = [&](int g, auto kind_c) {
      constexpr int KIND = decltype(kind_c)::value;
      const int step = g - LAG;
      const int t = step >> 1;
      bool do_load = false;
      if (KIND == 0 && step >= 0) {
        // ---- M(t)
        const bool pv = needed(t - 1), qk = needed(t);
        if (qk) {
          const float* l = LD + ((grp * 2 + (t & 1)) * 2) * 64;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            lse_a[q] = *reinterpret_cast<const f32x4*>(l + 8 * q + 4 * lh);
            d_a[q] = *reinterpret_cast<const f32x4*>(l + 64 + 8 * q + 4 * lh);
          }
        }
        if (pv) {
          const int sl = (t - 1) & 1;
          const uint16_t* Gb = lds + G_OFF + (grp * 2 + sl) * TILE;
          const uint16_t* Qb = lds + Q_OFF + (grp * 2 + sl) * TILE;
          // MFMA j: (k-step kk, column tile dt), dV (j even) or dK
          auto load = [&](auto jc) -> u32x4 {
            constexpr int j = decltype(jc)::value, dt = (j / 2) % DTILES, kk = j / (2 * DTILES);
            const uint16_t* src = ((j % 2) ? Qb : Gb) + v_lane + 2 * kk * QST + 32 * dt;
            const u32x2 lo = lds_read_tr16(src), hi = lds_read_tr16(src + QST);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
          };
          auto mfma = [&](auto jc, u32x4 a) {
            constexpr int j = decltype(jc)::value, dt = (j / 2) % DTILES, kk = j / (2 * DTILES);
            if constexpr (j % 2) dk[dt] = E::mfma(a, db[kk], dk[dt]);
            else dv[dt] = E::mfma(a, pb[kk], dv[dt]);
          };
          m_pipeline<4 * DTILES, kPipe>(load, mfma);
        }
        if (qk) {
          const int sl = t & 1;
          const uint16_t* Qb = lds + Q_OFF + (grp * 2 + sl) * TILE + q_row;
          const uint16_t* Gb = lds + G_OFF + (grp * 2 + sl) * TILE + q_row;
          // S = Q K^T and dP = dO V^T, alternating; both operands from LDS,
          // read together kPipe MFMAs ahead
          auto load = [&](auto jc) -> OpPair {
            constexpr int j = decltype(jc)::value, kk = j / 2;
            return OpPair{lds_read16(((j % 2) ? Gb : Qb) + 16 * kk),
                          lds_read16(((j % 2) ? vb_row : kb_row) + 16 * kk)};
          };
          auto mfma = [&](auto jc, const OpPair& o) {
            constexpr int j = decltype(jc)::value, kk = j / 2;
            if constexpr (j % 2) dP = E::mfma(o.a, o.b, kk == 0 ? f32x16{} : dP);
            else S = E::mfma(o.a, o.b, kk == 0 ? f32x16{} : S);
          };
          m_pipeline<2 * KSTEPS, kPairPipe>(load, mfma);
        }
      } else if (KIND == 1 && step >= 0) {
        // ---- V(t): the LSE and D of the rows of registers 8-15 (LDS reads
        // before this phase's copy is issued; those of registers 0-7 came
        // with the M step), then the copy of tile t + 1, then the gradient math
        const bool use = needed(t);
        const int r0 = tile_row0(t), sl = t & 1;
        const float* l = LD + ((grp * 2 + sl) * 2) * 64;
        f32x4 lse_b[2], d_b[2];
        if (use) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            lse_b[q] = *reinterpret_cast<const f32x4*>(l + 16 + 8 * q + 4 * lh);
            d_b[q] = *reinterpret_cast<const f32x4*>(l + 64 + 16 + 8 * q + 4 * lh);
          }
        }
        if (t + 1 < n_mine) {
          copy_tile(t + 1);
          do_load = true;
        }
        if (use) {
          // lane = key; register r is query row r0 + 8 (r/4) + 4 lh + r%4.  Every
          // exp2 is evaluated and masked pairs are selected to 0 (no branch).
          const bool full = r0 + BM <= Sq && kw0 + 32 <= Sk && (!CAUSAL || kw0 + 31 <= r0 + kv_off);
          auto grad = [&](auto mask_c, auto half_c, const f32x4 (&lse4)[2], const f32x4 (&d4)[2]) {
            constexpr bool MASK = decltype(mask_c)::value;
            constexpr int H = decltype(half_c)::value;
#pragma unroll
            for (int r = 8 * H; r < 8 * H + 8; ++r) {
              const int rowi = r0 + 8 * (r >> 2) + 4 * lh + (r & 3);
              const bool ok = !MASK || (rowi < Sq && key < Sk && (!CAUSAL || key <= rowi + kv_off));
              const float e =
                  fast_exp2(__builtin_fmaf(S[r], cs, -lse4[(r >> 2) & 1][r & 3] * kLog2e));
              const float pr = ok ? e : 0.f;
              S[r] = pr;
              dP[r] = pr * (dP[r] - d4[(r >> 2) & 1][r & 3]);
            }
            const int q = 8 * H;
            pb[H] = u32x4{E::pack2(S[q + 0], S[q + 1]), E::pack2(S[q + 2], S[q + 3]),
                          E::pack2(S[q + 4], S[q + 5]), E::pack2(S[q + 6], S[q + 7])};
            db[H] = u32x4{E::pack2(dP[q + 0], dP[q + 1]), E::pack2(dP[q + 2], dP[q + 3]),
                          E::pack2(dP[q + 4], dP[q + 5]), E::pack2(dP[q + 6], dP[q + 7])};
          };
          using H0 = std::integral_constant<int, 0>;
          using H1 = std::integral_constant<int, 1>;
          if (full) grad(std::false_type{}, H0{}, lse_a, d_a);
          else grad(std::true_type{}, H0{}, lse_a, d_a);
          if (full) grad(std::false_type{}, H1{}, lse_b, d_b);
          else grad(std::true_type{}, H1{}, lse_b, d_b);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (do_load) wait_vmem();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    // phase g runs step g - LAG: an M step when it is even, a V step when odd
    using K0 = std::integral_constant<int, LAG>;
    using K1 = std::integral_constant<int, 1 - LAG>;
    for (int g = 0; g < nphase; g += 2) {
      phase(g, K0{});
      phase(g + 1, K1{});
    }
  };
  if (grp == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

  // ---- the two groups' partial sums: the following group's through LDS
  // (the ring is no longer read), added by the leading group in that order
  float* red = reinterpret_cast<float*>(lds);
  if (grp == 1) {
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[((gw * 2 * DTILES + dt) * 16 + r) * 64 + lane] = dk[dt][r];
        red[((gw * 2 * DTILES + DTILES + dt) * 16 + r) * 64 + lane] = dv[dt][r];
      }
  }
  __syncthreads();
  if (grp == 0 && key < Sk) {
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[dt][r] += red[((gw * 2 * DTILES + dt) * 16 + r) * 64 + lane];
        dv[dt][r] += red[((gw * 2 * DTILES + DTILES + dt) * 16 + r) * 64 + lane];
      }
    // dK = scale * (dS^T Q) with the signed scale, dV = P^T dO: lane key li,
    // d = 32 dt + 8 (r/4) + 4 lh + r%4
    uint16_t* krow = static_cast<uint16_t*>(p.dk) + kvbase + (long long)key * D + 4 * lh;
    uint16_t* vrow = static_cast<uint16_t*>(p.dv) + kvbase + (long long)key * D + 4 * lh;
    const float sc = p.scale;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const u32x2 pk = {E::pack2(dk[dt][4 * a + 0] * sc, dk[dt][4 * a + 1] * sc),
                          E::pack2(dk[dt][4 * a + 2] * sc, dk[dt][4 * a + 3] * sc)};
        *reinterpret_cast<u32x2*>(krow + 32 * dt + 8 * a) = pk;
        const u32x2 pv = {E::pack2(dv[dt][4 * a + 0], dv[dt][4 * a + 1]),
                          E::pack2(dv[dt][4 * a + 2], dv[dt][4 * a + 3])};
        *reinterpret_cast<u32x2*>(vrow + 32 * dt + 8 * a) = pv;
      }
  }
}

template <int D, int DT, bool CAUSAL>
hipError_t launch_bwd_c(const BwdParams& p, hipStream_t stream) {
  // Sq = 0 still writes dK = dV = 0, Sk = 0 still writes dQ = 0
  const long long rows = (long long)p.B * p.Hq * p.Sq;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_pre_kernel<D, DT>), dim3((unsigned)((rows + 31) / 32)), dim3(256), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (p.Sq + 32 * kDqWaves - 1) / (32 * kDqWaves);
    hipLaunchKernelGGL((bwd_dq_kernel<D, DT, CAUSAL>), dim3(p.B * p.Hq * nqb),
                       dim3(kDqWaves * 64), 0, stream, p);
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
  }
  const int nkb = (p.Sk + kDkdvKeys - 1) / kDkdvKeys;
  if (nkb > 0 && p.B * p.Hkv > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, CAUSAL>), dim3(p.B * p.Hkv * nkb),
                       dim3(kDkdvWaves * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_bwd_d(const BwdParams& p, bool causal, hipStream_t stream) {
  return causal ? launch_bwd_c<D, DT, true>(p, stream) : launch_bwd_c<D, DT, false>(p, stream);
}

}  // namespace

hipError_t launch_backward(const BwdParams& p, int D, int dtype, bool causal,
                           hipStream_t stream) {
  if (D == 128) {
    return dtype == kBF16 ? launch_bwd_d<128, kBF16>(p, causal, stream)
                          : launch_bwd_d<128, kFP16>(p, causal, stream);
  }
  return dtype == kBF16 ? launch_bwd_d<64, kBF16>(p, causal, stream)
                        : launch_bwd_d<64, kFP16>(p, causal, stream);
}

}  // namespace fa
