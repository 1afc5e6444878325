// Attention backward pass for gfx950: dQ, dK, dV of O = softmax(scale Q K^T +
// mask) V given dO and the forward's row log-sum-exp, as three kernels in the
// textbook FA-2 split (tessera PR page, flash_attn backward commit: a pre-pass
// for D = rowsum(O * dO), dK/dV per key tile, dQ per query tile; P and dS are
// recomputed tile by tile, no score matrix is stored):
//
//   pre   D_i = sum_d dO[i,d] O[i,d]                                 (fp32)
//   dq    per 128 query rows, 32 keys a step (few enough registers for two
//         waves per SIMD): S^T = K Q^T, dP^T = V dO^T,
//         P = exp2(S c - LSE_i log2 e), dS = P (dP - D_i),
//         dQ^T += K^T dS^T                       (Q and dO stay in registers)
//   dkdv  per 128 keys, 64 query rows a step: S = Q K^T, dP = dO V^T, P and dS as above,
//         dV^T += dO^T P, dK^T += Q^T dS   (K and V stay in registers; the
//         query heads of a GQA group add into their kv head in the loop, so
//         no atomics are needed anywhere)
//
// Every product runs on the 32x32x16 matrix core with the operand layouts of
// the forward kernel: a wave owns 32 rows (dq) or 32 keys (dkdv), the operand
// that varies along the loop is read from LDS, transposed operands come from
// the gfx950 transposing LDS read, and P / dS feed the next product straight
// from the accumulator registers in their register order.  Tiles are staged
// global -> registers -> LDS with one barrier on each side; this version
// favours simplicity over overlap.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdWaves = 4;        // waves per workgroup, 32 rows or keys each
constexpr int kRowPad = 8;          // pad of tiles read by 16-byte row reads only
constexpr int kTrPad = 32;          // pad of tiles that are also read transposed
// MFMAs an LDS operand read runs ahead of its use
#ifndef FA_BWD_PIPE
#define FA_BWD_PIPE 4
#endif
constexpr int kPipe = FA_BWD_PIPE;
// dQ kernel: keys per K/V tile, and the waves per SIMD its registers must allow
#ifndef FA_BWD_DQ_KEYS
#define FA_BWD_DQ_KEYS 32
#endif
constexpr int kDqKeys = FA_BWD_DQ_KEYS;
constexpr int kDqWaves = kDqKeys == 32 ? 2 : 1;
// dK/dV kernel: query rows per step
#ifndef FA_BWD_DKDV_ROWS
#define FA_BWD_DKDV_ROWS 64
#endif
constexpr int kDkdvRows = FA_BWD_DKDV_ROWS;

// A ROWS x D tile in flight between global memory and LDS: each of the
// workgroup's threads holds N of its 16-byte chunks in registers, so the next
// tile's loads can be issued before the current tile is used.
template <int D, int ROWS>
struct TileRegs {
  static constexpr int CH = D / 8;                          // chunks per row
  static constexpr int N = ROWS * CH / (kBwdWaves * 64);    // chunks per thread
  static_assert(ROWS * CH % (kBwdWaves * 64) == 0, "whole chunks per thread");
  u32x4 x[N];
};

// Load `valid` rows (row stride D elements in global memory) of a tile; rows
// past `valid` are zero.  The tile is a buffer range that ends after its last
// valid row, so those rows read zeros without a branch per load.  `src` and
// `valid` are the same for every lane.
template <int D, int ROWS>
__device__ __forceinline__ void fetch_tile(TileRegs<D, ROWS>& t, const uint16_t* src, int valid) {
  using T = TileRegs<D, ROWS>;
  // read from the first lane so that the range is built in scalar registers
  const uintptr_t a = reinterpret_cast<uintptr_t>(src);
  const uintptr_t lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)a);
  const uintptr_t hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32));
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<uint16_t*>((hi << 32) | lo), (short)0, max(uniform(valid), 0) * D * 2,
      kBufferFlags);
#pragma unroll
  for (int i = 0; i < T::N; ++i) {
    const int c = (int)threadIdx.x + i * kBwdWaves * 64;
    const int r = c / T::CH, cc = c - r * T::CH;
    t.x[i] = __builtin_bit_cast(u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, (r * D + cc * 8) * 2, 0, 0));
  }
}

// Write a fetched tile to LDS rows of LST elements.
template <int D, int ROWS, int LST>
__device__ __forceinline__ void store_tile(uint16_t* lds, const TileRegs<D, ROWS>& t) {
  using T = TileRegs<D, ROWS>;
#pragma unroll
  for (int i = 0; i < T::N; ++i) {
    const int c = (int)threadIdx.x + i * kBwdWaves * 64;
    const int r = c / T::CH, cc = c - r * T::CH;
    lds_write16(lds + r * LST + cc * 8, t.x[i]);
  }
}


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

// ---- dq: one workgroup per (batch, query head, 128 query rows) ------------------
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(kDqWaves, 2)))
void bwd_dq_kernel(BwdParams p) {
  using E = Elt<DT>;
  constexpr int BN = kDqKeys;            // keys per tile (32-key sub-tiles)
  constexpr int NST = BN / 32;
  constexpr int KSTEPS = D / 16, DTILES = D / 32;
  constexpr int KST = D + kTrPad;        // K: row reads (S) and transposed reads (dQ)
  constexpr int VST = D + kRowPad;       // V: row reads (dP)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KST];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[BN * VST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5, ti = lane & 15;
  const int nqb = (p.Sq + 127) / 128;
  int blk = blockIdx.x;
  const int qb = blk % nqb;
  blk /= nqb;
  const int hq = blk % p.Hq;
  const int b = blk / p.Hq;
  const int hk = hq / p.gqa;
  const int q0 = qb * 128, rw0 = q0 + wave * 32, row = rw0 + li;
  const int Sq = p.Sq, Sk = p.Sk, kv_off = Sk - Sq;
  const long long qbase = ((long long)b * p.Hq + hq) * Sq * D;   // q, dO, dQ
  const long long kvbase = ((long long)b * p.Hkv + hk) * Sk * D;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + kvbase;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + kvbase;

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

  int kv_end = Sk, wave_end = Sk;
  if (CAUSAL) {
    kv_end = min(max(min(Sq, q0 + 128) + kv_off, 0), Sk);
    wave_end = min(max(min(Sq, rw0 + 32) + kv_off, 0), Sk);
  }
  if (rw0 >= Sq) wave_end = 0;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int v_lane = (4 * lh + (ti >> 2)) * KST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);

  f32x16 dq[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) dq[dt] = f32x16{};

  // tile t + 1 is loaded into registers while tile t is used
  TileRegs<D, BN> kt, vt;
  if (ntiles > 0) {
    fetch_tile(kt, kg, min(BN, Sk));
    fetch_tile(vt, vg, min(BN, Sk));
  }
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // the previous tile is no longer read
    store_tile<D, BN, KST>(Ks, kt);
    store_tile<D, BN, VST>(Vs, vt);
    __syncthreads();
    if (t + 1 < ntiles) {
      const int valid = min(BN, Sk - (t + 1) * BN);
      fetch_tile(kt, kg + (long long)(t + 1) * BN * D, valid);
      fetch_tile(vt, vg + (long long)(t + 1) * BN * D, valid);
    }
    if (t * BN >= wave_end) continue;
    // S^T = K Q^T and dP^T = V dO^T, the two products' MFMAs alternating,
    // each LDS operand read kPipe MFMAs ahead
    f32x16 S[NST], dP[NST];
    {
      auto load = [&](auto jc) -> u32x4 {
        constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
        if constexpr (j % 2) return lds_read16(Vs + (32 * st + li) * VST + 16 * kk + 8 * lh);
        else return lds_read16(Ks + (32 * st + li) * KST + 16 * kk + 8 * lh);
      };
      auto mfma = [&](auto jc, u32x4 a) {
        constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
        if constexpr (j % 2) dP[st] = E::mfma(a, gr[kk], kk == 0 ? f32x16{} : dP[st]);
        else S[st] = E::mfma(a, qr[kk], kk == 0 ? f32x16{} : S[st]);
      };
      m_pipeline<2 * NST * KSTEPS, kPipe>(load, mfma);
    }
    // lane = query row; register r of sub-tile st is key t*BN + 32 st + 8 (r/4) + 4 lh + r%4
    u32x4 db[NST][2];
    // every pair of the tile is admissible for this wave when all its rows
    // and keys exist and (causal) the tile's last key is at or below the
    // wave's first row's diagonal: the mask is then left out.  Every exp2 is
    // evaluated and masked pairs are selected to 0, so the loop has no branch.
    const bool full = rw0 + 32 <= Sq && (t + 1) * BN <= Sk && (!CAUSAL || t * BN + BN - 1 <= rw0 + kv_off);
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
          db[st][kk] = u32x4{E::pack2(S[st][r0 + 0], S[st][r0 + 1]), E::pack2(S[st][r0 + 2], S[st][r0 + 3]),
                             E::pack2(S[st][r0 + 4], S[st][r0 + 5]), E::pack2(S[st][r0 + 6], S[st][r0 + 7])};
        }
      }
    };
    if (full) grad(std::false_type{});
    else grad(std::true_type{});
    // dQ^T += K^T dS^T: K^T by transposing reads, keys in dS's register
    // order; MFMA j = (sub-tile st, k-step kk, column tile dt)
    {
      auto load = [&](auto jc) -> u32x4 {
        constexpr int j = decltype(jc)::value, dt = j % DTILES, kk = (j / DTILES) % 2;
        constexpr int st = j / (2 * DTILES);
        const uint16_t* kr = Ks + v_lane + (32 * st + 16 * kk) * KST + 32 * dt;
        const u32x2 lo = lds_read_tr16(kr), hi = lds_read_tr16(kr + 8 * KST);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      auto mfma = [&](auto jc, u32x4 a) {
        constexpr int j = decltype(jc)::value, dt = j % DTILES, kk = (j / DTILES) % 2;
        constexpr int st = j / (2 * DTILES);
        dq[dt] = E::mfma(a, db[st][kk], dq[dt]);
      };
      m_pipeline<2 * NST * DTILES, kPipe>(load, mfma);
    }
  }

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

// ---- dkdv: one workgroup per (batch, kv head, 128 keys) -------------------------
template <int D, int DT, bool CAUSAL>
__global__ __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p) {
  using E = Elt<DT>;
  constexpr int BM = kDkdvRows;          // query rows per step (32-row sub-tiles)
  constexpr int NST = BM / 32;
  constexpr int KSTEPS = D / 16, DTILES = D / 32;
  constexpr int QST = D + kTrPad;        // Q and dO: row reads and transposed reads
  __shared__ __attribute__((aligned(16))) uint16_t Qs[BM * QST];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[BM * QST];
  __shared__ __attribute__((aligned(16))) float Ls[BM];
  __shared__ __attribute__((aligned(16))) float Ds[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5, ti = lane & 15;
  const int nkb = (p.Sk + 127) / 128;
  int blk = blockIdx.x;
  const int kb = blk % nkb;
  blk /= nkb;
  const int hk = blk % p.Hkv;
  const int b = blk / p.Hkv;
  const int k0 = kb * 128, kw0 = k0 + wave * 32, key = kw0 + li;
  const int Sq = p.Sq, Sk = p.Sk, kv_off = Sk - Sq;
  const long long kvbase = ((long long)b * p.Hkv + hk) * Sk * D;

  // K (sign-folded: the scores come out as q_sign * S, the sign of the scale
  // applied once here instead of to every Q tile) and V rows as B operands:
  // lane key li, d = 16 kk + 8 lh + e
  u32x4 kr[KSTEPS], vr[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < Sk) {
      x = gload16(static_cast<const uint16_t*>(p.k) + kvbase + (long long)key * D + 16 * kk + 8 * lh);
      y = gload16(static_cast<const uint16_t*>(p.v) + kvbase + (long long)key * D + 16 * kk + 8 * lh);
    }
    if (p.q_sign < 0) x ^= 0x80008000u;
    if (p.q_sign == 0) x = u32x4{0u, 0u, 0u, 0u};
    kr[kk] = x;
    vr[kk] = y;
  }
  const float c = p.c_log2;
  const int v_lane = (4 * lh + (ti >> 2)) * QST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);

  f32x16 dk[DTILES], dv[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // rows that see a key of this block: row + kv_off >= k0 when causal.  The
  // steps run over (query head g of the group, 32-row tile) pairs; step it + 1
  // is loaded into registers while step it is used.
  const int r_first = CAUSAL ? (max(0, k0 - kv_off) / BM) * BM : 0;
  const int nrt = r_first < Sq ? (Sq - r_first + BM - 1) / BM : 0;
  const int total = p.gqa * nrt;
  TileRegs<D, BM> qt, gt;
  float lnext = 0.f, dnext = 0.f;
  auto fetch = [&](int it) {
    const int g = it / nrt;
    const int r0 = r_first + (it - g * nrt) * BM;
    const int hq = hk * p.gqa + g;
    const long long qbase = ((long long)b * p.Hq + hq) * Sq * D + (long long)r0 * D;
    const long long sbase = ((long long)b * p.Hq + hq) * Sq;
    const int valid = min(BM, Sq - r0);
    fetch_tile(qt, static_cast<const uint16_t*>(p.q) + qbase, valid);
    fetch_tile(gt, static_cast<const uint16_t*>(p.dout) + qbase, valid);
    if (tid < BM) {
      const int r = r0 + tid;
      lnext = r < Sq ? p.lse[sbase + r] * kLog2e : 0.f;
      dnext = r < Sq ? p.dsum[sbase + r] : 0.f;
    }
  };
  if (total > 0) fetch(0);
  for (int it = 0; it < total; ++it) {
    {
      const int r0 = r_first + (it % nrt) * BM;
      __syncthreads();  // the previous tile is no longer read
      store_tile<D, BM, QST>(Qs, qt);
      store_tile<D, BM, QST>(Gs, gt);
      if (tid < BM) {
        Ls[tid] = lnext;
        Ds[tid] = dnext;
      }
      __syncthreads();
      if (it + 1 < total) fetch(it + 1);
      if (kw0 >= Sk) continue;                            // no keys in this wave
      if (CAUSAL && kw0 > r0 + BM - 1 + kv_off) continue;  // every pair masked
      // S = Q K^T and dP = dO V^T, the two products' MFMAs alternating, each
      // LDS operand read kPipe MFMAs ahead (one wave per SIMD: nothing else
      // hides the LDS latency)
      f32x16 S[NST], dP[NST];
      {
        auto load = [&](auto jc) -> u32x4 {
          constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
          const uint16_t* src = (j % 2) ? Gs : Qs;
          return lds_read16(src + (32 * st + li) * QST + 16 * kk + 8 * lh);
        };
        auto mfma = [&](auto jc, u32x4 a) {
          constexpr int j = decltype(jc)::value, st = j / (2 * KSTEPS), kk = (j / 2) % KSTEPS;
          if constexpr (j % 2) dP[st] = E::mfma(a, vr[kk], kk == 0 ? f32x16{} : dP[st]);
          else S[st] = E::mfma(a, kr[kk], kk == 0 ? f32x16{} : S[st]);
        };
        m_pipeline<2 * NST * KSTEPS, kPipe>(load, mfma);
      }
      // lane = key; register r of sub-tile st is query row r0 + 32 st + 8 (r/4) + 4 lh + r%4
      u32x4 pb[NST][2], db[NST][2];
      // every pair of this step is admissible for this wave when all its
      // rows and keys exist and (causal) its last key is at or below its
      // first row's diagonal: the mask is then left out
      const bool full = r0 + BM <= Sq && kw0 + 32 <= Sk && (!CAUSAL || kw0 + 31 <= r0 + kv_off);
      auto grad = [&](auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          // the rows' LSE and D, four consecutive rows per 16-byte read, read
          // before any is used; every exp2 is evaluated and masked pairs are
          // then selected to 0, so the loop has no branch
          f32x4 lse4[4], d4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lse4[q] = *reinterpret_cast<const f32x4*>(Ls + 32 * st + 8 * q + 4 * lh);
            d4[q] = *reinterpret_cast<const f32x4*>(Ds + 32 * st + 8 * q + 4 * lh);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = 32 * st + 8 * (r >> 2) + 4 * lh + (r & 3);
            const int rowi = r0 + rr;
            const bool ok = !MASK || (rowi < Sq && key < Sk && (!CAUSAL || key <= rowi + kv_off));
            const float e = fast_exp2(__builtin_fmaf(S[st][r], c, -lse4[r >> 2][r & 3]));
            const float pr = ok ? e : 0.f;
            S[st][r] = pr;
            dP[st][r] = pr * (dP[st][r] - d4[r >> 2][r & 3]);
          }
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const int q = 8 * kk;
            pb[st][kk] = u32x4{E::pack2(S[st][q + 0], S[st][q + 1]), E::pack2(S[st][q + 2], S[st][q + 3]),
                               E::pack2(S[st][q + 4], S[st][q + 5]), E::pack2(S[st][q + 6], S[st][q + 7])};
            db[st][kk] = u32x4{E::pack2(dP[st][q + 0], dP[st][q + 1]), E::pack2(dP[st][q + 2], dP[st][q + 3]),
                               E::pack2(dP[st][q + 4], dP[st][q + 5]), E::pack2(dP[st][q + 6], dP[st][q + 7])};
          }
        }
      };
      if (full) grad(std::false_type{});
      else grad(std::true_type{});
      // dV^T += dO^T P and dK^T += Q^T dS: dO^T, Q^T by transposing reads,
      // rows in the register order of P and dS
      {
        // MFMA j: (sub-tile st, k-step kk, column tile dt), dV (j even) or dK
        auto load = [&](auto jc) -> u32x4 {
          constexpr int j = decltype(jc)::value, dt = (j / 2) % DTILES;
          constexpr int kk = (j / (2 * DTILES)) % 2, st = j / (4 * DTILES);
          const uint16_t* src = ((j % 2) ? Qs : Gs) + v_lane + (32 * st + 16 * kk) * QST + 32 * dt;
          const u32x2 lo = lds_read_tr16(src), hi = lds_read_tr16(src + 8 * QST);
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        auto mfma = [&](auto jc, u32x4 a) {
          constexpr int j = decltype(jc)::value, dt = (j / 2) % DTILES;
          constexpr int kk = (j / (2 * DTILES)) % 2, st = j / (4 * DTILES);
          if constexpr (j % 2) dk[dt] = E::mfma(a, db[st][kk], dk[dt]);
          else dv[dt] = E::mfma(a, pb[st][kk], dv[dt]);
        };
        m_pipeline<4 * NST * DTILES, kPipe>(load, mfma);
      }
    }
  }

  // dK = scale * (dS^T Q), dV = P^T dO: lane key li, d = 32 dt + 8 (r/4) + 4 lh + r%4
  if (key < Sk) {
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
  const int nqb = (p.Sq + 127) / 128, nkb = (p.Sk + 127) / 128;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_pre_kernel<D, DT>), dim3((unsigned)((rows + 31) / 32)), dim3(256), 0,
                       stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, DT, CAUSAL>), dim3(p.B * p.Hq * nqb),
                       dim3(kBwdWaves * 64), 0, stream, p);
    const hipError_t e2 = hipGetLastError();
    if (e2 != hipSuccess) return e2;
  }
  if (nkb > 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, DT, CAUSAL>), dim3(p.B * p.Hkv * nkb),
                       dim3(kBwdWaves * 64), 0, stream, p);
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
