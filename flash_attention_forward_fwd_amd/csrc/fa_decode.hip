// Single-token (Sq = 1) attention over a contiguous token-major KV cache, gfx950.
//
// The cache is [B, capacity, Hkv, D]; batch b attends to its first
// L = clamp(valid_len[b], 0, capacity) tokens, where valid_len lives on the
// device (decode PR page, PR description: "device INT32 valid-length scalar",
// "contiguous token-major KV").  Tokens at or past L are never loaded: their
// K and V operands are zero in registers / LDS and their scores are -inf, so
// NaN or garbage in the unused tail cannot reach O (decode PR page, review:
// masking scores alone leaves 0 * NaN in the P*V product; the invalid V
// operands must be made safe before it).
//
// Split-KV (named as follow-up work on the decode PR page): the L tokens of
// each (batch, kv head) are cut into `nsplit` equal runs of 32-token chunks,
// one workgroup per run.  Each workgroup produces an unnormalised partial
// (m, l, acc) per query head -- m the running max in the log2 domain, l the
// sum of exp2(s - m), acc the exp2-weighted sum of V rows -- and the partials
// are merged by
//     M = max_s m_s,  O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// in a second kernel launched right after on the same stream (one workgroup
// per (unit, head group, 32 columns of O)).  With kMergeKernel off the merge
// runs inside the decode launch instead, in two levels: the last workgroup to
// finish in each group of kMergeGroup splits merges that group, and the last
// group merger merges the groups and writes O.  "Last" is decided by a ticket
// counter per group that the merger resets to zero, so the workspace is ready
// for the next call.  A single split skips the merge and writes O directly.
//
// Per wave and 32-token chunk, on the 32x32x16 matrix core (the query heads
// that share a kv head form the MFMA N dimension, up to 32):
//   S^T = K Q^T   K rows straight from global memory as the A operand;
//   O^T += V^T P^T  V staged through wave-private LDS and read back with the
//   transposing LDS read, in the key order in which P sits in its registers.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kMergeGroup = 16;  // partials merged by one workgroup
// Merge the split records in a second, stream-ordered kernel (1) instead of
// by the last workgroups of the decode kernel through tickets (0).
#ifndef FA_DECODE_MERGE_KERNEL
#define FA_DECODE_MERGE_KERNEL 1
#endif
constexpr bool kMergeKernel = FA_DECODE_MERGE_KERNEL != 0;
constexpr int kDVPad = 32;       // V staging row pad (elements)
// 32-token chunks per split at full capacity
#ifndef FA_DECODE_CHUNKS_PER_SPLIT
#define FA_DECODE_CHUNKS_PER_SPLIT 8
#endif
constexpr int kChunksPerSplit = FA_DECODE_CHUNKS_PER_SPLIT;

// Query heads of head group hg (groups of hpg heads of one kv head's gqa).
__device__ __forceinline__ int heads_in_group(int hpg, int gqa, int hg) {
  return min(hpg, gqa - hpg * hg);
}

// Partials cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other) through loads and stores with the sc1 cache policy (what an
// agent-scope relaxed atomic access compiles to): they are written through to
// the device-coherent level and read from it, so no whole-cache writeback or
// invalidate (what a device-scope fence costs on gfx950) is needed.  Ordering
// comes from waiting for the stores to complete (vmcnt(0)) before the ticket
// is taken.
// A transposing 64-bit LDS read (see the lane mapping in the common header)
// as inline asm, opaque to the compiler's memory-dependency tracking; the
// caller waits for it (lgkmcnt) and then passes the value through
// after_wait(), which orders its uses after that wait.
// (The host pass of the compiler sees no body: the asm names GPU registers.)
__device__ __forceinline__ u32x2 lds_read_tr16_opaque(const uint16_t* lds) {
  u32x2 r = {0u, 0u};
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)lds;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
#else
  (void)lds;
#endif
  return r;
}
__device__ __forceinline__ void after_wait(u32x2& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#else
  (void)x;
#endif
}

// Coherent 16- and 8-byte accesses to one unit's partial records.
constexpr int kCoherent = 16;  // cache-policy bits: sc1
__device__ __forceinline__ f32x4 ld4_coherent(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent));
}
__device__ __forceinline__ void st4_coherent(__amdgpu_buffer_rsrc_t rs, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCoherent);
}
__device__ __forceinline__ f32x2 ld2_coherent(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kCoherent));
}
__device__ __forceinline__ void st2_coherent(__amdgpu_buffer_rsrc_t rs, int off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, kCoherent);
}

// Merge records [first, first + n) (n <= kMergeGroup) of one unit's partials
// in global memory -- o records of gg x D floats at byte 0 of `ro`, (m, l)
// pairs at byte 0 of `rml` -- into record `dst` of the same unit, or, when
// `out` is not null, normalise and write O.  Column g of a record is query
// token g / gh, head g % gh of the group; its O row starts at
// out + out_base + (g / gh) * ostride + (g % gh) * D.  Every thread issues all of its
// record loads before using any, so a merge costs about one memory round trip.
template <int D, int DT, bool MULTI>
__device__ void merge_global(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml, int first,
                             int n, int gg, int cs, int dst, uint16_t* out, long long out_base,
                             int gh, long long ostride, float* lds_scratch) {
  using E = Elt<DT>;
  constexpr int Q = D / 4;              // 16-byte pieces per head row
  float* w = lds_scratch;               // [gg][kMergeGroup] weights 2^(m_s - M)
  float* den = w + gg * kMergeGroup;    // [gg]
  float* Mh = den + gg;                 // [gg]
  for (int g = threadIdx.x; g < gg; g += blockDim.x) {
    f32x2 ml[kMergeGroup];
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s)
      if (s < n) ml[s] = ld2_coherent(rml, ((first + s) * cs + g) * 8);
    float M = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s)
      if (s < n) M = fmaxf(M, ml[s][0]);
    const float Mu = (M == -__builtin_inff()) ? 0.f : M;
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s) {
      if (s < n) {
        const float f = fast_exp2(ml[s][0] - Mu);  // m = -inf -> 0
        w[g * kMergeGroup + s] = f;
        dsum += f * ml[s][1];
      }
    }
    den[g] = dsum;
    Mh[g] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < gg * Q; idx += blockDim.x) {
    const int g = idx / Q, q = idx - g * Q;
    f32x4 x[kMergeGroup];
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s)
      if (s < n) x[s] = ld4_coherent(ro, (((first + s) * cs + g) * D + 4 * q) * 4);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s) {
      if (s < n) {
        const float f = w[g * kMergeGroup + s];
        if (f != 0.f) acc += f * x[s];
      }
    }
    if (out) {
      const float dd = den[g];
      const float inv = dd > 0.f ? 1.0f / dd : 0.f;
      const u32x2 pk = {E::pack2(acc[0] * inv, acc[1] * inv), E::pack2(acc[2] * inv, acc[3] * inv)};
      const long long orow =
          MULTI ? (long long)(g / gh) * ostride + (long long)(g % gh) * D : (long long)g * D;
      *reinterpret_cast<u32x2*>(out + out_base + orow + 4 * q) = pk;
    } else {
      st4_coherent(ro, ((dst * cs + g) * D + 4 * q) * 4, acc);
    }
  }
  if (!out) {
    for (int g = threadIdx.x; g < gg; g += blockDim.x)
      st2_coherent(rml, (dst * cs + g) * 8, f32x2{Mh[g], den[g]});
  }
  __syncthreads();
}

// Merge the workgroup's `n` wave records (o: [n][cs][D], ml: [n][cs][2], in
// LDS; columns g < gg in use) into record `dst` of the unit's partials in
// global memory (records of cs columns, written coherently, 16 bytes at a
// time), or, when `out` is not null, normalise and write O as merge_global
// does.
template <int D, int DT, bool MULTI>
__device__ void merge_waves(const float* src_o, const float* src_ml, int n, int gg, int cs,
                            __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml, int dst,
                            uint16_t* out, long long out_base, int gh, long long ostride,
                            float* lds_scratch) {
  using E = Elt<DT>;
  constexpr int Q = D / 4;
  float* w = lds_scratch;              // [gg][n] weights 2^(m_s - M)
  float* den = lds_scratch + gg * n;   // [gg]
  float* Mh = den + gg;                // [gg]
  for (int g = threadIdx.x; g < gg; g += blockDim.x) {
    float M = -__builtin_inff();
    for (int s = 0; s < n; ++s) M = fmaxf(M, src_ml[(s * cs + g) * 2]);
    const float Mu = (M == -__builtin_inff()) ? 0.f : M;
    float dsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float f = fast_exp2(src_ml[(s * cs + g) * 2] - Mu);  // m = -inf -> 0
      w[g * n + s] = f;
      dsum += f * src_ml[(s * cs + g) * 2 + 1];
    }
    den[g] = dsum;
    Mh[g] = M;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < gg * Q; idx += blockDim.x) {
    const int g = idx / Q, q = idx - g * Q;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n; ++s) {
      const float f = w[g * n + s];
      const f32x4 x = *reinterpret_cast<const f32x4*>(src_o + (s * cs + g) * D + 4 * q);
      if (f != 0.f) acc += f * x;
    }
    if (out) {
      const float dd = den[g];
      const float inv = dd > 0.f ? 1.0f / dd : 0.f;
      const u32x2 pk = {E::pack2(acc[0] * inv, acc[1] * inv), E::pack2(acc[2] * inv, acc[3] * inv)};
      const long long orow =
          MULTI ? (long long)(g / gh) * ostride + (long long)(g % gh) * D : (long long)g * D;
      *reinterpret_cast<u32x2*>(out + out_base + orow + 4 * q) = pk;
    } else {
      st4_coherent(ro, ((dst * cs + g) * D + 4 * q) * 4, acc);
    }
  }
  if (!out) {
    for (int g = threadIdx.x; g < gg; g += blockDim.x)
      st2_coherent(rml, (dst * cs + g) * 8, f32x2{Mh[g], den[g]});
  }
  __syncthreads();
}

// Workgroup-wide ticket after this workgroup's record is stored: true in every
// thread of the workgroup that arrives last (count reaches `total`); that
// workgroup also resets the counter for the next call.
__device__ __forceinline__ bool take_ticket(unsigned* counter, unsigned total, int* lds_flag) {
  wait_vmem();  // this workgroup's record stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned t =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = (t == total - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last ? 1 : 0;
  }
  __syncthreads();
  return *lds_flag != 0;
}

template <int D, int DT, bool PAGED, bool MULTI>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_kernel(DecodeParams p) {
  using E = Elt<DT>;
  constexpr int NW = kDecodeWaves;
  constexpr int KSTEPS = D / 16;
  constexpr int DTILES = D / 32;
  constexpr int VST = D + kDVPad;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const int ti = lane & 15;

  // grid: x = split, y = unit (b, kv head, head group)
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  // a unit's MFMA columns are (query token t, head g of the group): column
  // t * gh + g for t < sq, g < gh, at most 32 of them
  // (one query token: MULTI off, sq = 1 and 32 heads per group at compile time)
  const int sq = MULTI ? p.sq : 1;
  const int hpg = MULTI ? p.hpg : 32;
  const int HG = (p.gqa + hpg - 1) / hpg;
  const int hg = unit % HG;
  const int bk = unit / HG;
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const int gh = heads_in_group(hpg, p.gqa, hg);
  const int gg = gh * sq;                        // columns in use
  const int cstride = min(hpg, p.gqa) * sq;     // columns per record
  const int hq0 = hk * p.gqa + hpg * hg;  // first query head of this group

  // Q of the group's heads (lane: column li, d = 16kk + 8lh + e) does not
  // depend on the valid length: its loads are issued first, without
  // branches (columns past gg read column 0 and are zeroed below), so their
  // round trip overlaps the valid-length read and the compiler can count
  // them exactly when it later waits for them
  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  u32x4 qr[KSTEPS];
  {
    const int col = li < gg ? li : 0;
    const int t = MULTI ? col / gh : 0;
    const uint16_t* qrow = qg + (((long long)b * sq + t) * p.Hq + hq0 + col - t * gh) * D + 8 * lh;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qr[kk] = gload16(qrow + 16 * kk);
  }
  __builtin_amdgcn_sched_barrier(0);

  int L = p.valid_len[b];
  L = min(max(L, 0), p.capacity);

  // Q as the B operand: columns past the group's gg are zero, and the sign
  // of the scale is applied to Q (q_sign -1: negated, 0: zero), so the
  // scores' scale factor c is never negative.  The empty asm pins the
  // result here, ahead of every K/V load: computed later (where the
  // compiler would sink it), its wait for Q would also wait for the first
  // chunk's loads.
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = qr[kk];
    x = p.q_sign < 0 ? (x ^ 0x80008000u) : x;
    qr[kk] = (li < gg && p.q_sign != 0) ? x : u32x4{0u, 0u, 0u, 0u};
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(qr[kk]));
#endif
  }
  const int nchunks = (L + 31) / 32;
  const int cps = (nchunks + p.nsplit - 1) / p.nsplit;  // chunks per split
  const int c0 = min(split * cps, nchunks);
  const int c1 = min(c0 + cps, nchunks);

  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);
  const float c = p.c_log2;
  const long long tok_stride = (long long)p.Hkv * D;  // elements between tokens
  const long long cache_base =
      PAGED ? (long long)hk * D : (long long)b * p.capacity * tok_stride + (long long)hk * D;

  // Paged cache: logical page lp of batch b is physical page
  // page_table[b][lp] of a pool [num_pages, page_size, Hkv, D]; page_size is
  // a multiple of 32, so a 32-token chunk never straddles two pages.  Lane j
  // of a wave holds the physical page of the wave's j-th chunk (a wave has at
  // most 64 chunks; the host bounds the capacity for that).  Entries are
  // clamped to the pool, so no table value leads outside it.
  int my_page = 0;
  if constexpr (PAGED) {
    const int chj = c0 + wave + NW * lane;
    if (chj < c1) {
      const int e = p.page_table[(long long)b * p.pages_per_seq + (chj * 32) / p.page_size];
      my_page = min(max(e, 0), p.num_pages - 1);
    }
  }


  // K and V of this (batch, kv head) as buffer ranges that end at token L:
  // token j's row sits at byte j * tok_stride * 2, and rows at or past L read
  // zeros, so the invalid tail is never fetched
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kg + cache_base), (short)0, (int)(L * tok_stride * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vg + cache_base), (short)0, (int)(L * tok_stride * 2), kBufferFlags);

  // V of a chunk goes straight into wave-private LDS (two buffers, so the next
  // chunk lands while this one is used) with 16-byte buffer loads to LDS: the
  // padded 32-row image is cut into 1 KiB pieces, chunk c of the image being
  // row c / RC, column c % RC; padding columns read from past the buffer.
  constexpr int RC = VST / 8;                 // 16-byte chunks per staged row
  constexpr int NPC = 32 * RC / 64;           // 1 KiB pieces per chunk
  static_assert(32 * RC % 64 == 0, "staged V chunk is whole KiB");
  uint16_t* vst0 = reinterpret_cast<uint16_t*>(dyn_lds) + wave * 2 * 32 * VST;
  unsigned voffs[NPC];
#pragma unroll
  for (int i = 0; i < NPC; ++i) {
    const int cidx = 64 * i + lane;
    const int rr = cidx / RC, cc = cidx - rr * RC;
    voffs[i] = cc < D / 8 ? (unsigned)((rr * tok_stride + cc * 8) * 2) : kPastEnd;
  }
  const int v_lane = (4 * lh + (ti >> 2)) * VST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);
  // K rows (A operand): lane row li, d = 16kk + 8lh
  const unsigned k_off = (unsigned)((li * tok_stride + 8 * lh) * 2);

  // Query token t of the sq sits at position L - sq + t: with the causal
  // mask (bottom-right) it sees keys j <= L - sq + t, else every j < L.
  // key_lim is the last key this lane's column sees, mask_from the first key
  // that some column does not see.
  const int key_lim = MULTI && p.causal ? L - sq + (li < gg ? li / gh : 0) : L - 1;
  const int mask_from = MULTI && p.causal ? L - sq + 1 : L;

  f32x16 oacc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  auto load_chunk = [&](int ch, u32x4 (&kr)[KSTEPS], uint16_t* vbuf) {
    int soff;
    __amdgpu_buffer_rsrc_t kc = krs, vc = vrs;
    if constexpr (!PAGED) {
      soff = ch * 32 * (int)tok_stride * 2;
    } else {
      // this chunk's page as a buffer range ending at token L
      const int lp = (ch * 32) / p.page_size;
      const int phys = __builtin_amdgcn_readlane(my_page, (ch - c0 - wave) / NW);
      const int in_page = min(p.page_size, L - lp * p.page_size);
      const long long base = (long long)phys * p.page_size * tok_stride + cache_base;
      kc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg + base), (short)0,
                                             (int)(in_page * tok_stride * 2), kBufferFlags);
      vc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg + base), (short)0,
                                             (int)(in_page * tok_stride * 2), kBufferFlags);
      soff = (ch * 32 - lp * p.page_size) * (int)tok_stride * 2;
    }
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      kr[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kc, k_off + 32 * kk, soff, 0));
#pragma unroll
    for (int i = 0; i < NPC; ++i)
      lds_dma16(vc, vbuf + i * 512, voffs[i], soff);
  };
  auto compute_chunk = [&](int ch, const u32x4 (&kr)[KSTEPS], const uint16_t* vbuf) {
    const int tok0 = ch * 32;
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) s = E::mfma(kr[kk], qr[kk], s);
    // scores of keys a column does not see are excluded (keys >= L had zero
    // K rows, not -inf)
    if (tok0 + 32 > mask_from) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = tok0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (j > key_lim) s[r] = -__builtin_inff();
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = fast_exp2(__builtin_fmaf(s[r], c, -m_use));
      psum += s[r];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt) oacc[dt] *= alpha;
    // V^T operands by transposing LDS reads, all issued before any is used.
    // They are written as inline asm: the compiler cannot tell which LDS
    // bytes a buffer load to LDS fills, and for its own reads it would wait
    // for every such load in flight -- including the next chunk's, which is
    // what must stay in flight here.  This chunk's pieces landed at the
    // vmcnt wait before the call, and the lgkmcnt wait below is the reads' own.
    u32x2 tr[2][DTILES][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          tr[kk][dt][h] = lds_read_tr16_opaque(vbuf + v_lane + 16 * kk * VST + 8 * h * VST + 32 * dt);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) after_wait(tr[kk][dt][h]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r0 = 8 * kk;
      const u32x4 pb = {E::pack2(s[r0 + 0], s[r0 + 1]), E::pack2(s[r0 + 2], s[r0 + 3]),
                        E::pack2(s[r0 + 4], s[r0 + 5]), E::pack2(s[r0 + 6], s[r0 + 7])};
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const u32x4 a = {tr[kk][dt][0][0], tr[kk][dt][0][1], tr[kk][dt][1][0], tr[kk][dt][1][1]};
        oacc[dt] = E::mfma(a, pb, oacc[dt]);
      }
    }
  };

  // chunks c0 + wave, + NW, ...: the next chunk's K and V loads are issued
  // before the current one is computed, so two chunks are in flight per wave
  {
    u32x4 kA[KSTEPS], kB[KSTEPS];
    uint16_t* vA = vst0;
    uint16_t* vB = vst0 + 32 * VST;
    int ch = c0 + wave;
    if (ch < c1) load_chunk(ch, kA, vA);
    while (ch < c1) {
      const int nx = ch + NW;
      if (nx < c1) {
        load_chunk(nx, kB, vB);
        wait_vmem_le<KSTEPS + NPC>();  // chunk ch is in (registers and LDS)
      } else {
        wait_vmem();
      }
      compute_chunk(ch, kA, vA);
      if (nx >= c1) break;
      const int nx2 = nx + NW;
      if (nx2 < c1) {
        load_chunk(nx2, kA, vA);
        wait_vmem_le<KSTEPS + NPC>();
      } else {
        wait_vmem();
      }
      compute_chunk(nx, kB, vB);
      ch = nx2;
    }
  }

  // ---- merge the waves of this workgroup (through LDS) -> split partial ----
  __syncthreads();  // V staging no longer needed; reuse dyn_lds
  // wave records in LDS and global records alike hold cstride columns, of
  // which the first gg are in use: [NW][cstride][D] and [NW][cstride][2]
  float* wo = reinterpret_cast<float*>(dyn_lds);
  float* wml = wo + NW * cstride * D;
  const float l_tot = pair_sum(l_run);
  if (li < gg) {
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * lh + (r & 3);
        wo[(wave * cstride + li) * D + d] = oacc[dt][r];
      }
    if (lh == 0) {
      wml[(wave * cstride + li) * 2 + 0] = m_run;
      wml[(wave * cstride + li) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  float* scratch = wml + NW * cstride * 2;  // merge weights and per-column sums
  const int ngroups = (p.nsplit + kMergeGroup - 1) / kMergeGroup;
  const int nrec = p.nsplit + ngroups;  // level-0 records, then level-1 records
  const long long unit_parts = (long long)unit * nrec;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      p.part_o + unit_parts * cstride * D, (short)0, nrec * cstride * D * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + unit_parts * cstride * 2, (short)0, nrec * cstride * 2 * 4, kBufferFlags);
  uint16_t* og = static_cast<uint16_t*>(p.o);
  // O is [B, sq, Hq, D]: column (t, g) -> row (b, t, hq0 + g)
  const long long out_base = ((long long)b * sq * p.Hq + hq0) * D;
  const long long ostride = (long long)p.Hq * D;

  if (p.nsplit == 1) {
    merge_waves<D, DT, MULTI>(wo, wml, NW, gg, cstride, ro, rml, 0, og, out_base, gh, ostride,
                              scratch);
    return;
  }
  merge_waves<D, DT, MULTI>(wo, wml, NW, gg, cstride, ro, rml, split, nullptr, 0, gh, ostride,
                            scratch);
  if (kMergeKernel) return;  // the split records are merged by decode_merge_kernel

  // ---- level 1: last workgroup of the group merges the group -------------------
  const int grp = split / kMergeGroup;
  const int gfirst = grp * kMergeGroup;
  const int gsize = min(kMergeGroup, p.nsplit - gfirst);
  unsigned* cnt0 = p.tickets + (long long)unit * (ngroups + 1);
  // the ticket flag sits in the last word of the dynamic LDS, past the merge
  // scratch (two workgroups of 80 KiB fill the 160 KiB of a CU exactly, so
  // the kernel has no static LDS)
  int* ticket_flag = reinterpret_cast<int*>(dyn_lds + p.lds_bytes) - 1;
  if (!take_ticket(cnt0 + grp, (unsigned)gsize, ticket_flag)) return;
  if (ngroups == 1) {
    merge_global<D, DT, MULTI>(ro, rml, gfirst, gsize, gg, cstride, 0, og, out_base, gh, ostride,
                               scratch);
    return;
  }
  merge_global<D, DT, MULTI>(ro, rml, gfirst, gsize, gg, cstride, p.nsplit + grp, nullptr, 0, gh,
                             ostride, scratch);
  // ---- level 2: last group merger merges the groups and writes O -----------
  if (!take_ticket(cnt0 + ngroups, (unsigned)ngroups, ticket_flag)) return;
  merge_global<D, DT, MULTI>(ro, rml, p.nsplit, ngroups, gg, cstride, 0, og, out_base, gh, ostride,
                             scratch);
}

// Reduction over the lanes of a wave that differ in lane bits 3..5 (lane % 8
// fixed), every lane receiving the result, on the vector unit: a DPP rotate
// of the 16-lane row by 8 (lane ^ 8), then the gfx950 swaps of 16-lane rows
// (lane ^ 16) and 32-lane halves (lane ^ 32).  Each step combines a lane with
// its partner symmetrically, so all lanes of a group hold the same bits.
template <class Op>
__device__ __forceinline__ float reduce_lane_bits345(float x, Op op) {
  x = op(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128 /* row_ror:8 */,
                                                       0xF, 0xF, false)));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return op(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

// Second kernel: merges the nsplit (<= 256, see decode_num_splits) split
// records of (unit, column g = (query token, head) of the group) for 32
// columns of O.  Thread t takes columns 4 (t % 8) .. + 3 of records
// s = t / 8 + 32 k, k < 8, together with those records' (m, l).  The kernel
// boundary makes the records visible, so plain loads suffice, and all of
// them are issued before any is used: the merge costs one memory round trip,
// two lane reductions and two barriers (the maximum M over the records, then
// the weighted sums).
constexpr int kMergeThreads = 256;
template <int D, int DT>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeParams p) {
  using E = Elt<DT>;
  constexpr int NW = kMergeThreads / 64;
  __shared__ float red_m[NW];
  __shared__ f32x4 part[NW][8];
  __shared__ float part_l[NW][8];
  const int unit = blockIdx.x, g = blockIdx.y, col0 = 32 * blockIdx.z;  // g: record column
  const int HG = (p.gqa + p.hpg - 1) / p.hpg;
  const int hg = unit % HG;
  const int bk = unit / HG;
  const int b = bk / p.Hkv, hk = bk - b * p.Hkv;
  const int gh = heads_in_group(p.hpg, p.gqa, hg);
  const int cs = min(p.hpg, p.gqa) * p.sq;  // columns per record
  if (g >= gh * p.sq) return;
  const int ns = p.nsplit;
  const int ngroups = (ns + kMergeGroup - 1) / kMergeGroup;
  const long long rec0 = (long long)unit * (ns + ngroups);  // this unit's first record
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int cg = t & 7, rl = t >> 3;
  const float* po = p.part_o + (rec0 * cs + g) * D + col0 + 4 * cg;
  const float* pml = p.part_ml + (rec0 * cs + g) * 2;
  f32x4 x[8];
  f32x2 ml[8];
  // loads without branches: records past ns read record 0 (always written)
  // and are then replaced by an empty record (m = -inf, l = 0, acc = 0)
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int s = rl + 32 * k;
    const int sc = s < ns ? s : 0;
    x[k] = *reinterpret_cast<const f32x4*>(po + (long long)sc * cs * D);
    ml[k] = *reinterpret_cast<const f32x2*>(pml + (long long)sc * cs * 2);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before any is used
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool in = rl + 32 * k < ns;
    ml[k][0] = in ? ml[k][0] : -__builtin_inff();
  }
  // M = max_s m_s over all records
  float M = ml[0][0];
#pragma unroll
  for (int k = 1; k < 8; ++k) M = fmaxf(M, ml[k][0]);
  M = reduce_lane_bits345(M, [](float a, float c) { return fmaxf(a, c); });
  if (lane == 0) red_m[wv] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red_m[i]);
  // weights w_s = 2^(m_s - M); sum_s w_s acc_s and sum_s w_s l_s
  const float Mu = (M == -__builtin_inff()) ? 0.f : M;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // a record of weight 0 (an empty split, or past ns) adds nothing, its
    // contents unread
    const float w = fast_exp2(ml[k][0] - Mu);  // m = -inf -> 0
    const bool use = w != 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(w, use ? x[k][i] : 0.f, acc[i]);
    den = __builtin_fmaf(w, use ? ml[k][1] : 0.f, den);
  }
  auto add = [](float a, float c) { return a + c; };
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = reduce_lane_bits345(acc[i], add);
  den = reduce_lane_bits345(den, add);
  if (lane < 8) {
    part[wv][lane] = acc;
    part_l[wv][lane] = den;
  }
  __syncthreads();
  if (t < 8) {
    f32x4 sum = part[0][t];
    float dsum = part_l[0][t];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      sum += part[i][t];
      dsum += part_l[i][t];
    }
    const float inv = dsum > 0.f ? 1.0f / dsum : 0.f;
    const u32x2 pk = {E::pack2(sum[0] * inv, sum[1] * inv), E::pack2(sum[2] * inv, sum[3] * inv)};
    uint16_t* og = static_cast<uint16_t*>(p.o);
    const int qt = g / gh;                              // query token of the column
    const int hq = hk * p.gqa + p.hpg * hg + g - qt * gh;
    *reinterpret_cast<u32x2*>(og + (((long long)b * p.sq + qt) * p.Hq + hq) * D + col0 + 4 * t) = pk;
  }
}

template <int D, int DT, bool PAGED, bool MULTI>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const int HG = (p.gqa + p.hpg - 1) / p.hpg;
  const int gg = min(p.hpg, p.gqa) * p.sq;  // columns per record
  const int ngroups = (p.nsplit + kMergeGroup - 1) / kMergeGroup;
  const size_t stage = (size_t)kDecodeWaves * 2 * 32 * (D + kDVPad) * 2;
  int nmax = kDecodeWaves;  // most records any merge step reads
  if (kMergeGroup > nmax) nmax = kMergeGroup;
  if (ngroups > nmax) nmax = ngroups;
  const size_t merge = ((size_t)kDecodeWaves * gg * (D + 2) + (size_t)gg * (nmax + 2)) * 4 + 16;
  const size_t lds = stage > merge ? stage : merge;
  DecodeParams q = p;
  q.lds_bytes = (int)lds;
  dim3 grid(p.nsplit, p.B * p.Hkv * HG);
  hipLaunchKernelGGL((decode_kernel<D, DT, PAGED, MULTI>), grid, dim3(kDecodeWaves * 64), lds,
                     stream, q);
  if (kMergeKernel && p.nsplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D, DT>), dim3(p.B * p.Hkv * HG, gg, D / 32),
                       dim3(kMergeThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_p(const DecodeParams& p, hipStream_t stream) {
  if (p.sq > 1)
    return p.page_table ? launch_d<D, DT, true, true>(p, stream)
                        : launch_d<D, DT, false, true>(p, stream);
  return p.page_table ? launch_d<D, DT, true, false>(p, stream)
                      : launch_d<D, DT, false, false>(p, stream);
}

}  // namespace

int decode_num_splits(int B, int Hkv, int capacity) {
  // about kChunksPerSplit (8: 256 tokens) chunks per split at full capacity, and at
  // most 256 splits per (batch, kv head): 64 MiB of K+V over 512 workgroups
  // at the largest cache of the decode workload
  const int chunks = (capacity + 31) / 32;
  int ns = (chunks + kChunksPerSplit - 1) / kChunksPerSplit;
  if (ns > 256) ns = 256;
  if (ns < 1) ns = 1;
  (void)B;
  (void)Hkv;
  return ns;
}

int decode_heads_per_group(int gqa, int sq) {
  const int h = 32 / sq;
  return gqa < h ? gqa : h;
}

size_t decode_workspace_layout(int B, int Sq, int Hq, int Hkv, int D, int capacity,
                               size_t* off_ml, size_t* off_tickets) {
  const int gqa = Hq / Hkv;
  const int hpg = decode_heads_per_group(gqa, Sq);
  const int HG = (gqa + hpg - 1) / hpg;
  const int gg = hpg * Sq;  // columns per record
  const int ns = decode_num_splits(B, Hkv, capacity);
  const int ngroups = (ns + kMergeGroup - 1) / kMergeGroup;
  const size_t units = (size_t)B * Hkv * HG;
  const size_t recs = units * (size_t)(ns + ngroups) * gg;
  size_t bytes = recs * (size_t)D * 4;          // part_o
  bytes = (bytes + 255) & ~(size_t)255;
  if (off_ml) *off_ml = bytes;
  bytes += recs * 2 * 4;                        // part_ml
  bytes = (bytes + 255) & ~(size_t)255;
  if (off_tickets) *off_tickets = bytes;
  bytes += units * (size_t)(ngroups + 1) * 4;   // tickets
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t stream) {
  if (D == 128) {
    return dtype == kBF16 ? launch_p<128, kBF16>(p, stream) : launch_p<128, kFP16>(p, stream);
  }
  return dtype == kBF16 ? launch_p<64, kBF16>(p, stream) : launch_p<64, kFP16>(p, stream);
}

}  // namespace fa
