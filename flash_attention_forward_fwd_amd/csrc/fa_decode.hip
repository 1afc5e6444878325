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
// are merged in the same launch:
//     M = max_s m_s,  O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// in two levels: the last workgroup to finish in each group of kMergeGroup
// splits merges that group, and the last group merger merges the groups and
// writes O.  "Last" is decided by a ticket counter per group that the merger
// resets to zero, so the workspace is ready for the next call.
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
constexpr int kDVPad = 32;       // V staging row pad (elements)

__device__ __forceinline__ int heads_in_group(int gqa, int hg) { return min(32, gqa - 32 * hg); }

// Partials cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other) through loads and stores with the sc1 cache policy (what an
// agent-scope relaxed atomic access compiles to): they are written through to
// the device-coherent level and read from it, so no whole-cache writeback or
// invalidate (what a device-scope fence costs on gfx950) is needed.  Ordering
// comes from waiting for the stores to complete (vmcnt(0)) before the ticket
// is taken.
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
// `out` is not null, normalise and write O.  Every thread issues all of its
// record loads before using any, so a merge costs about one memory round trip.
template <int D, int DT>
__device__ void merge_global(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml, int first,
                             int n, int gg, int dst, uint16_t* out, long long out_base,
                             float* lds_scratch) {
  using E = Elt<DT>;
  constexpr int Q = D / 4;              // 16-byte pieces per head row
  float* w = lds_scratch;               // [gg][kMergeGroup] weights 2^(m_s - M)
  float* den = w + gg * kMergeGroup;    // [gg]
  float* Mh = den + gg;                 // [gg]
  for (int g = threadIdx.x; g < gg; g += blockDim.x) {
    f32x2 ml[kMergeGroup];
#pragma unroll
    for (int s = 0; s < kMergeGroup; ++s)
      if (s < n) ml[s] = ld2_coherent(rml, ((first + s) * gg + g) * 8);
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
      if (s < n) x[s] = ld4_coherent(ro, (((first + s) * gg + g) * D + 4 * q) * 4);
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
      *reinterpret_cast<u32x2*>(out + out_base + (long long)g * D + 4 * q) = pk;
    } else {
      st4_coherent(ro, ((dst * gg + g) * D + 4 * q) * 4, acc);
    }
  }
  if (!out) {
    for (int g = threadIdx.x; g < gg; g += blockDim.x)
      st2_coherent(rml, (dst * gg + g) * 8, f32x2{Mh[g], den[g]});
  }
  __syncthreads();
}

// Merge the workgroup's `n` wave records (o: [n][gg][D], ml: [n][gg][2], in
// LDS) into record `dst` of the unit's partials in global memory (written
// coherently, 16 bytes at a time), or, when `out` is not null, normalise and
// write O.
template <int D, int DT>
__device__ void merge_waves(const float* src_o, const float* src_ml, int n, int gg,
                            __amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml, int dst,
                            uint16_t* out, long long out_base, float* lds_scratch) {
  using E = Elt<DT>;
  constexpr int Q = D / 4;
  float* w = lds_scratch;              // [gg][n] weights 2^(m_s - M)
  float* den = lds_scratch + gg * n;   // [gg]
  float* Mh = den + gg;                // [gg]
  for (int g = threadIdx.x; g < gg; g += blockDim.x) {
    float M = -__builtin_inff();
    for (int s = 0; s < n; ++s) M = fmaxf(M, src_ml[(s * gg + g) * 2]);
    const float Mu = (M == -__builtin_inff()) ? 0.f : M;
    float dsum = 0.f;
    for (int s = 0; s < n; ++s) {
      const float f = fast_exp2(src_ml[(s * gg + g) * 2] - Mu);  // m = -inf -> 0
      w[g * n + s] = f;
      dsum += f * src_ml[(s * gg + g) * 2 + 1];
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
      const f32x4 x = *reinterpret_cast<const f32x4*>(src_o + (s * gg + g) * D + 4 * q);
      if (f != 0.f) acc += f * x;
    }
    if (out) {
      const float dd = den[g];
      const float inv = dd > 0.f ? 1.0f / dd : 0.f;
      const u32x2 pk = {E::pack2(acc[0] * inv, acc[1] * inv), E::pack2(acc[2] * inv, acc[3] * inv)};
      *reinterpret_cast<u32x2*>(out + out_base + (long long)g * D + 4 * q) = pk;
    } else {
      st4_coherent(ro, ((dst * gg + g) * D + 4 * q) * 4, acc);
    }
  }
  if (!out) {
    for (int g = threadIdx.x; g < gg; g += blockDim.x)
      st2_coherent(rml, (dst * gg + g) * 8, f32x2{Mh[g], den[g]});
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

template <int D, int DT>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 8))) void decode_kernel(DecodeParams p) {
  using E = Elt<DT>;
  constexpr int NW = kDecodeWaves;
  constexpr int KSTEPS = D / 16;
  constexpr int DTILES = D / 32;
  constexpr int VST = D + kDVPad;
  constexpr int VPER = 32 * (D / 8) / 64;  // 16-byte V pieces per lane per chunk
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];
  __shared__ int ticket_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const int ti = lane & 15;

  // grid: x = split, y = unit (b, kv head, head group)
  const int split = blockIdx.x;
  const int unit = blockIdx.y;
  const int HG = (p.gqa + 31) / 32;
  const int hg = unit % HG;
  const int bk = unit / HG;
  const int b = bk / p.Hkv;
  const int hk = bk - b * p.Hkv;
  const int gg = heads_in_group(p.gqa, hg);
  const int hq0 = hk * p.gqa + 32 * hg;  // first query head of this group

  int L = p.valid_len[b];
  L = min(max(L, 0), p.capacity);
  const int nchunks = (L + 31) / 32;
  const int cps = (nchunks + p.nsplit - 1) / p.nsplit;  // chunks per split
  const int c0 = min(split * cps, nchunks);
  const int c1 = min(c0 + cps, nchunks);

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);
  const float c = p.c_log2;
  const long long tok_stride = (long long)p.Hkv * D;  // elements between tokens
  const long long cache_base = (long long)b * p.capacity * tok_stride + (long long)hk * D;

  // Q of the group's heads as the B operand (lane: head li, d = 16kk + 8lh + e)
  u32x4 qr[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (li < gg) x = gload16(qg + ((long long)b * p.Hq + hq0 + li) * D + 16 * kk + 8 * lh);
    if (p.q_sign < 0) x ^= 0x80008000u;
    if (p.q_sign == 0) x = u32x4{0u, 0u, 0u, 0u};
    qr[kk] = x;
  }

  uint16_t* vst = reinterpret_cast<uint16_t*>(dyn_lds) + wave * 32 * VST;
  const int v_lane = (4 * lh + (ti >> 2)) * VST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3);

  f32x16 oacc[DTILES];
#pragma unroll
  for (int dt = 0; dt < DTILES; ++dt) oacc[dt] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.f;

  for (int ch = c0 + wave; ch < c1; ch += NW) {
    const int tok0 = ch * 32;
    // K rows (A operand): lane row li, d = 16kk + 8lh
    u32x4 kr[KSTEPS];
    const int ktok = tok0 + li;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ktok < L) x = gload16(kg + cache_base + (long long)ktok * tok_stride + 16 * kk + 8 * lh);
      kr[kk] = x;
    }
    // V rows -> wave-private LDS, invalid rows as zeros
    u32x4 vr[VPER];
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int piece = lane + 64 * u;
      const int rr = piece / (D / 8), cc = piece % (D / 8);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (tok0 + rr < L) x = gload16(vg + cache_base + (long long)(tok0 + rr) * tok_stride + cc * 8);
      vr[u] = x;
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) s = E::mfma(kr[kk], qr[kk], s);
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int piece = lane + 64 * u;
      const int rr = piece / (D / 8), cc = piece % (D / 8);
      lds_write16(vst + rr * VST + cc * 8, vr[u]);
    }
    // scores of tokens >= L are excluded (their K rows were zero, not -inf)
    if (tok0 + 32 > L) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = tok0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (j >= L) s[r] = -__builtin_inff();
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
    // LDS writes above must land before the transposing reads: one wave,
    // in-order LDS queue, but make the dependency explicit
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r0 = 8 * kk;
      const u32x4 pb = {E::pack2(s[r0 + 0], s[r0 + 1]), E::pack2(s[r0 + 2], s[r0 + 3]),
                        E::pack2(s[r0 + 4], s[r0 + 5]), E::pack2(s[r0 + 6], s[r0 + 7])};
      const uint16_t* vrow = vst + v_lane + 16 * kk * VST;
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const u32x2 lo = lds_read_tr16(vrow + 32 * dt);
        const u32x2 hi = lds_read_tr16(vrow + 8 * VST + 32 * dt);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
        oacc[dt] = E::mfma(a, pb, oacc[dt]);
      }
    }
    // the next chunk overwrites this wave's V staging: reads must be done
    __builtin_amdgcn_s_waitcnt(0xc07f);
  }

  // ---- merge the waves of this workgroup (through LDS) -> split partial ----
  __syncthreads();  // V staging no longer needed; reuse dyn_lds
  float* wo = reinterpret_cast<float*>(dyn_lds);      // [NW][gg][D]
  float* wml = wo + NW * gg * D;                       // [NW][gg][2]
  const float l_tot = pair_sum(l_run);
  if (li < gg) {
#pragma unroll
    for (int dt = 0; dt < DTILES; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * dt + 8 * (r >> 2) + 4 * lh + (r & 3);
        wo[(wave * gg + li) * D + d] = oacc[dt][r];
      }
    if (lh == 0) {
      wml[(wave * gg + li) * 2 + 0] = m_run;
      wml[(wave * gg + li) * 2 + 1] = l_tot;
    }
  }
  __syncthreads();
  float* scratch = wml + NW * gg * 2;  // merge weights and per-head sums
  const int ngroups = (p.nsplit + kMergeGroup - 1) / kMergeGroup;
  const int nrec = p.nsplit + ngroups;  // level-0 records, then level-1 records
  const long long unit_parts = (long long)unit * nrec;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      p.part_o + unit_parts * gg * D, (short)0, nrec * gg * D * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + unit_parts * gg * 2, (short)0, nrec * gg * 2 * 4, kBufferFlags);
  uint16_t* og = static_cast<uint16_t*>(p.o);
  const long long out_base = ((long long)b * p.Hq + hq0) * D;

  if (p.nsplit == 1) {
    merge_waves<D, DT>(wo, wml, NW, gg, ro, rml, 0, og, out_base, scratch);
    return;
  }
  merge_waves<D, DT>(wo, wml, NW, gg, ro, rml, split, nullptr, 0, scratch);

  // ---- level 1: last workgroup of the group merges the group -------------------
  const int grp = split / kMergeGroup;
  const int gfirst = grp * kMergeGroup;
  const int gsize = min(kMergeGroup, p.nsplit - gfirst);
  unsigned* cnt0 = p.tickets + (long long)unit * (ngroups + 1);
  if (!take_ticket(cnt0 + grp, (unsigned)gsize, &ticket_flag)) return;
  if (ngroups == 1) {
    merge_global<D, DT>(ro, rml, gfirst, gsize, gg, 0, og, out_base, scratch);
    return;
  }
  merge_global<D, DT>(ro, rml, gfirst, gsize, gg, p.nsplit + grp, nullptr, 0, scratch);
  // ---- level 2: last group merger merges the groups and writes O -----------
  if (!take_ticket(cnt0 + ngroups, (unsigned)ngroups, &ticket_flag)) return;
  merge_global<D, DT>(ro, rml, p.nsplit, ngroups, gg, 0, og, out_base, scratch);
}

template <int D, int DT>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const int HG = (p.gqa + 31) / 32;
  const int gg = min(32, p.gqa);
  const int ngroups = (p.nsplit + kMergeGroup - 1) / kMergeGroup;
  const size_t stage = (size_t)kDecodeWaves * 32 * (D + kDVPad) * 2;
  int nmax = kDecodeWaves;  // most records any merge step reads
  if (kMergeGroup > nmax) nmax = kMergeGroup;
  if (ngroups > nmax) nmax = ngroups;
  const size_t merge = ((size_t)kDecodeWaves * gg * (D + 2) + (size_t)gg * (nmax + 2)) * 4;
  const size_t lds = stage > merge ? stage : merge;
  dim3 grid(p.nsplit, p.B * p.Hkv * HG);
  hipLaunchKernelGGL((decode_kernel<D, DT>), grid, dim3(kDecodeWaves * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

int decode_num_splits(int B, int Hkv, int capacity) {
  // about 256 tokens (8 chunks of 32) per split at full capacity, and at
  // most 256 splits per (batch, kv head): 64 MiB of K+V over 512 workgroups
  // at the largest cache of the decode workload
  const int chunks = (capacity + 31) / 32;
  int ns = (chunks + 7) / 8;
  if (ns > 256) ns = 256;
  if (ns < 1) ns = 1;
  (void)B;
  (void)Hkv;
  return ns;
}

size_t decode_workspace_layout(int B, int Hq, int Hkv, int D, int capacity, size_t* off_ml,
                               size_t* off_tickets) {
  const int gqa = Hq / Hkv;
  const int HG = (gqa + 31) / 32;
  const int gg = gqa < 32 ? gqa : 32;
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
    return dtype == kBF16 ? launch_d<128, kBF16>(p, stream) : launch_d<128, kFP16>(p, stream);
  }
  return dtype == kBF16 ? launch_d<64, kBF16>(p, stream) : launch_d<64, kFP16>(p, stream);
}

}  // namespace fa
