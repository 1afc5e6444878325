// Single-token (Sq = 1) attention over a contiguous token-major KV cache, gfx950.
//
// The cache is [B, capacity, Hkv, D]; batch b attends to its first
// L = clamp(valid_len[b], 0, capacity) tokens, where valid_len lives on the
// device (decode PR page, PR description: device int32 valid length,
// contiguous token-major KV).  Tokens at or past L are never loaded: the K
// and V bytes of those rows come from past the end of a buffer range that
// ends at token L, which reads zeros, and their scores are selected to -inf,
// so NaN or garbage in the unused tail cannot reach O (decode PR page,
// review: masking the scores alone leaves 0 * NaN in the P*V product; the
// invalid V operands must be made safe before it).
//
// Split-KV (named as follow-up work on the decode PR page).  One launch holds
// two kinds of workgroups:
//  * split workgroups: the L tokens of each unit (batch, kv head, head group)
//    are cut into at most `nsplit` runs of whole 32-token chunks; one
//    workgroup per run produces an unnormalised partial per query column --
//    m (running max, log2 domain), l (sum of exp2(s - m)) and acc (the
//    exp2-weighted sum of V rows) -- stores it as a record, waits until the
//    stores are complete, and then raises one flag per merger of its unit;
//  * merger workgroups (the last blocks of the grid): each owns 4 query
//    columns x 32 dims of one unit's output, polls its flags until every
//    non-empty run has raised its flag, reads the records' slices in one
//    round of loads, forms
//        M = max_s m_s,  O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
//    in a fixed order (so repeated calls give the same bits), writes O and
//    lowers its flags again, leaving the workspace ready for the next call.
// The split plan is made on the device from L: runs have at least
// kMinSplitChunks chunks, so a short L uses few workgroups, and when one run
// covers all of L its workgroup writes O itself and the mergers return at once.
// Records and flags cross workgroups (and XCDs, whose L2 caches are not
// coherent with each other) through loads and stores with the sc1 cache
// policy -- what an agent-scope relaxed atomic access compiles to -- so no
// L2 writeback or invalidate is needed; ordering comes from waiting for the
// record stores to complete before a flag is raised, and from issuing the
// record loads only after every flag was seen.  Mergers never wait on each
// other, are at most kMaxMergers per launch (far fewer than the CUs, so the
// split workgroups always find room to run), and give up after a bounded
// number of polls, so every workgroup of the launch finishes.
//
// Per wave and 32-token chunk, on the 32x32x16 matrix core (the query columns
// that share a kv head form the MFMA N dimension, up to 32):
//   S^T = K Q^T     K rows from LDS as the A operand, Q resident in VGPRs;
//   O^T += V^T P^T  V read from LDS with the transposing read, in the key
//                   order in which P sits in its registers.
// K and V of a chunk are copied global -> LDS by 16-byte buffer loads that
// write LDS directly and bypass the caches' retention (nontemporal: each byte
// is read once); a wave's next chunk is in flight while it computes one.
#include <mutex>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

// Workspace of the decode entry point that allocates nothing: one array per
// GPU, held until the process ends.  Zero at load (no initializer); every
// completed call leaves its flags at zero again.  In host code its name is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress (decode_scratch below).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];
// every single-token plan fits: split runs x record columns x (D + 2) floats,
// plus the flags and the layout's alignment
static_assert(kDecodeFlagBytes + (size_t)kDecodeTargetWGs * kDecodeMaxGqa * (128 + 2) * 4 + 512 <=
                  kDecodeScratchBytes,
              "the largest single-token decode workspace fits the built-in array");

namespace {

constexpr int kSlots = 1;        // chunks in flight per wave
constexpr int kKPadD = 8;        // K LDS row = D + 8 elements
constexpr int kDVPad = 32;       // V LDS row = D + 32 elements
constexpr int kMergeDims = 32;   // output dims per merger
constexpr int kMergeBatch = 16;  // records per thread per round of loads
constexpr int kThreads = kDecodeWaves * 64;
constexpr int kSpinLimit = 1 << 20;
constexpr int kNtPolicy = 2;     // buffer-load cache policy: nontemporal
constexpr float kRescaleTau = 8.0f;  // lazy rescale threshold (log2 units)


// LDS image sizes of one chunk (bytes): K rows padded by 16 bytes against bank
// conflicts of the 16-byte operand reads, rounded up to whole KiB (one buffer
// load to LDS fills 1 KiB); V rows padded by 64 bytes for the transposing read
template <int D>
struct Stage {
  static constexpr int KST = D + kKPadD;
  static constexpr int VST = D + kDVPad;
  static constexpr int KNI = (32 * KST * 2 + 1023) / 1024;  // K loads per chunk
  static constexpr int VNI = 32 * VST * 2 / 1024;           // V loads per chunk
  static_assert(32 * VST * 2 % 1024 == 0, "V image is whole KiB");
  static constexpr int KBYTES = KNI * 1024;
  static constexpr int VBYTES = VNI * 1024;
  static constexpr int SLOT = KBYTES + VBYTES;
  static constexpr int NPC = KNI + VNI;  // loads per chunk
  static constexpr int WG_BYTES = kDecodeWaves * kSlots * SLOT;
};
static_assert(Stage<128>::WG_BYTES <= 160 * 1024, "one workgroup per CU");

__device__ __forceinline__ int heads_in_group(int hpg, int gqa, int hg) {
  return min(hpg, gqa - hpg * hg);
}

// 16-byte buffer load straight to LDS with the nontemporal policy
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rs, void* dst, unsigned voff,
                                             int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, kNtPolicy);
}

// The operands of one chunk, read from LDS in one inline-asm block that also
// waits for them (lgkmcnt(0)): the compiler cannot tell which LDS bytes a
// buffer load to LDS fills, and for its own LDS reads it would wait for every
// such load in flight -- including the next chunk's, which must stay in
// flight here.  The chunk's own loads have landed at the vmcnt wait before
// the call.  K: KSTEPS 16-byte reads (k-step kk at +32 kk bytes); V: the
// transposing 8-byte reads (k-step kk of 16 keys, half h of 8, column tile dt).
#define FA_DS_K(o, off) "ds_read_b128 %" #o ", %[ka] offset:" #off "\n"
#define FA_DS_V(o, off) "ds_read_b64_tr_b16 %" #o ", %[va] offset:" #off "\n"

template <int D>
struct ChunkOperands;

template <>
struct ChunkOperands<128> {
  u32x4 k[8];
  u32x2 v[2][4][2];  // [kk][dt][h]
  __device__ __forceinline__ void read(unsigned ka, unsigned va) {
#if defined(__HIP_DEVICE_COMPILE__)
    // V offsets: ((16 kk + 8 h) * VST + 32 dt) * 2 bytes, VST = 160
    asm volatile(
        FA_DS_K(0, 0) FA_DS_K(1, 32) FA_DS_K(2, 64) FA_DS_K(3, 96)
        FA_DS_K(4, 128) FA_DS_K(5, 160) FA_DS_K(6, 192) FA_DS_K(7, 224)
        FA_DS_V(8, 0) FA_DS_V(9, 2560) FA_DS_V(10, 64) FA_DS_V(11, 2624)
        FA_DS_V(12, 128) FA_DS_V(13, 2688) FA_DS_V(14, 192) FA_DS_V(15, 2752)
        FA_DS_V(16, 5120) FA_DS_V(17, 7680) FA_DS_V(18, 5184) FA_DS_V(19, 7744)
        FA_DS_V(20, 5248) FA_DS_V(21, 7808) FA_DS_V(22, 5312) FA_DS_V(23, 7872)
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]),
          "=&v"(k[6]), "=&v"(k[7]), "=&v"(v[0][0][0]), "=&v"(v[0][0][1]), "=&v"(v[0][1][0]),
          "=&v"(v[0][1][1]), "=&v"(v[0][2][0]), "=&v"(v[0][2][1]), "=&v"(v[0][3][0]),
          "=&v"(v[0][3][1]), "=&v"(v[1][0][0]), "=&v"(v[1][0][1]), "=&v"(v[1][1][0]),
          "=&v"(v[1][1][1]), "=&v"(v[1][2][0]), "=&v"(v[1][2][1]), "=&v"(v[1][3][0]),
          "=&v"(v[1][3][1])
        : [ka] "v"(ka), [va] "v"(va)
        : "memory");
#else
    (void)ka;
    (void)va;
#endif
  }
};

template <>
struct ChunkOperands<64> {
  u32x4 k[4];
  u32x2 v[2][2][2];
  __device__ __forceinline__ void read(unsigned ka, unsigned va) {
#if defined(__HIP_DEVICE_COMPILE__)
    // VST = 96: ((16 kk + 8 h) * 96 + 32 dt) * 2 bytes
    asm volatile(
        FA_DS_K(0, 0) FA_DS_K(1, 32) FA_DS_K(2, 64) FA_DS_K(3, 96)
        FA_DS_V(4, 0) FA_DS_V(5, 1536) FA_DS_V(6, 64) FA_DS_V(7, 1600)
        FA_DS_V(8, 3072) FA_DS_V(9, 4608) FA_DS_V(10, 3136) FA_DS_V(11, 4672)
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(v[0][0][0]),
          "=&v"(v[0][0][1]), "=&v"(v[0][1][0]), "=&v"(v[0][1][1]), "=&v"(v[1][0][0]),
          "=&v"(v[1][0][1]), "=&v"(v[1][1][0]), "=&v"(v[1][1][1])
        : [ka] "v"(ka), [va] "v"(va)
        : "memory");
#else
    (void)ka;
    (void)va;
#endif
  }
};
#undef FA_DS_K
#undef FA_DS_V

// Merge the workgroup's `n` wave partials (o: [n][cs][D], ml: [n][cs][2] in
// LDS; columns g < gg in use) into split record `dst` of the unit (records of
// cs columns at `ro` / `rml`, stored with the coherent policy), or, when `out`
// is not null, normalise and write O.  Column g is query token g / gh, head
// g % gh of the group; its O row starts at out + out_base + (g / gh) * ostride
// + (g % gh) * D.
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

// The split plan of one unit for L valid tokens: chunks per run and the
// number of non-empty runs (at least 1, so that an empty unit still writes
// its zero output).  Split and merger workgroups evaluate it alike.
__device__ __forceinline__ void split_plan(int L, int nsplit, int& cps, int& nruns) {
  const int nchunks = (L + 31) / 32;
  cps = max((nchunks + nsplit - 1) / nsplit, kMinSplitChunks);
  nruns = max((nchunks + cps - 1) / cps, 1);
}

struct UnitView {
  int b, hk, hg, gh, gg, cstride, hq0;
};

template <bool MULTI>
__device__ __forceinline__ UnitView unit_view(const DecodeParams& p, int unit) {
  UnitView u;
  const int sq = MULTI ? p.sq : 1;
  const int hpg = MULTI ? p.hpg : 32;
  const int HG = (p.gqa + hpg - 1) / hpg;
  u.hg = unit % HG;
  const int bk = unit / HG;
  u.b = bk / p.Hkv;
  u.hk = bk - u.b * p.Hkv;
  u.gh = heads_in_group(hpg, p.gqa, u.hg);
  u.gg = u.gh * sq;                       // columns in use
  u.cstride = min(hpg, p.gqa) * sq;      // columns per record
  u.hq0 = u.hk * p.gqa + hpg * u.hg;     // first query head of the group
  return u;
}

__device__ __forceinline__ int clamped_len(const DecodeParams& p, int b) {
  const int L = p.valid_len[b];
  return min(max(L, 0), p.capacity);
}

// ---------------------------------------------------------------------------
// merger workgroup: columns [col0, col0 + 4) x dims [32 db, 32 db + 32) of
// one unit's output
// ---------------------------------------------------------------------------
template <int D, int DT, bool MULTI>
__device__ void merger(const DecodeParams& p, int midx, unsigned char* lds) {
  using E = Elt<DT>;
  constexpr int DB = D / kMergeDims;
  const int M = p.nmerge, mc = p.merge_cols;
  const int unit = midx / M, m = midx - unit * M;
  const UnitView u = unit_view<MULTI>(p, unit);
  const int cb = m / DB, db = m - cb * DB;
  const int col0 = mc * cb;
  if (col0 >= u.gg) return;  // no columns here; the split workgroups raise no flag for it
  const int L = clamped_len(p, u.b);
  int cps, nruns;
  split_plan(L, p.nsplit, cps, nruns);
  if (nruns <= 1) return;  // the single run wrote O

  const int t = threadIdx.x, lane = t & 63;
  unsigned* fl = p.flags + ((long long)unit * M + m) * p.nsplit;
  int* ok = reinterpret_cast<int*>(lds);
  // wave 0 polls the flags of the nruns non-empty runs until all are raised
  if (t < 64) {
    int seen = 0;
    static_assert(kMaxSplits <= 4 * 64, "a poll reads at most 4 flags per lane");
    for (int it = 0; it < kSpinLimit && !seen; ++it) {
      unsigned f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // all loads of a poll in flight together
        const int s = 64 * i + lane;
        f[i] = s < nruns ? ld_flag(fl + s) : 1u;
      }
      const bool mine = f[0] != 0u && f[1] != 0u && f[2] != 0u && f[3] != 0u;
      seen = __builtin_amdgcn_ballot_w64(!mine) == 0;
    }
    if (t == 0) *ok = seen;
  }
  __syncthreads();
  const bool ready = *ok != 0;

  // threads form G groups of 8 mc: thread t takes runs s = tg + G j, column
  // col0 + cl, dims 32 db + 4 d4 .. + 3
  const int per = 8 * mc, G = kThreads / per;
  const int tg = t / per, w = t - tg * per, cl = w >> 3, d4 = w & 7;
  const int g = col0 + cl;
  const int gc = g < u.gg ? g : col0;  // columns past gg read column col0 and are dropped
  const long long rec0 = (long long)unit * p.nsplit;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      p.part_o + rec0 * u.cstride * D, (short)0, p.nsplit * u.cstride * D * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + rec0 * u.cstride * 2, (short)0, p.nsplit * u.cstride * 2 * 4, kBufferFlags);
  const int o_off = (gc * D + kMergeDims * db + 4 * d4) * 4;  // bytes inside a record
  float Mt = -__builtin_inff(), den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (ready) {
    for (int base = 0; base < nruns; base += G * kMergeBatch) {
      f32x4 x[kMergeBatch];
      f32x2 ml[kMergeBatch];
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const int s = base + tg + G * j;
        const int sc = s < nruns ? s : 0;  // run 0 is always written
        x[j] = ld4_coherent(ro, sc * u.cstride * D * 4 + o_off);
        ml[j] = ld2_coherent(rml, (sc * u.cstride + gc) * 8);
      }
      // running merge over this thread's runs, in run order
      float Mn = Mt;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j)
        if (base + tg + G * j < nruns) Mn = fmaxf(Mn, ml[j][0]);
      const float Mu = (Mn == -__builtin_inff()) ? 0.f : Mn;
      const float a = fast_exp2(Mt - Mu);  // Mt = -inf -> 0
      acc *= a;
      den *= a;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j) {
        const bool in = base + tg + G * j < nruns;
        const float wj = in ? fast_exp2(ml[j][0] - Mu) : 0.f;  // m = -inf -> 0
        const bool use = wj != 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(wj, use ? x[j][i] : 0.f, acc[i]);
        den = __builtin_fmaf(wj, use ? ml[j][1] : 0.f, den);
      }
      Mt = Mn;
    }
  }
  // combine the G run groups pairwise in a fixed tree (G is a power of two)
  float* red_m = reinterpret_cast<float*>(lds) + 4;             // [kThreads]
  float* red_d = red_m + kThreads;                              // [kThreads]
  f32x4* red_a = reinterpret_cast<f32x4*>(red_d + kThreads);    // [kThreads]
  red_m[t] = Mt;
  red_d[t] = den;
  red_a[t] = acc;
  __syncthreads();
  for (int half = G >> 1; half >= 1; half >>= 1) {
    if (tg < half) {
      const int o = t + half * per;
      const float Ma = red_m[t], Mb = red_m[o];
      const float Mn = fmaxf(Ma, Mb);
      const float Mu = (Mn == -__builtin_inff()) ? 0.f : Mn;
      const float wa = fast_exp2(Ma - Mu), wb = fast_exp2(Mb - Mu);  // -inf -> 0
      const bool ua = wa != 0.f, ub = wb != 0.f;
      const f32x4 aa = red_a[t], ab = red_a[o];
      f32x4 r;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        r[c] = __builtin_fmaf(wa, ua ? aa[c] : 0.f, wb * (ub ? ab[c] : 0.f));
      red_d[t] = __builtin_fmaf(wa, ua ? red_d[t] : 0.f, wb * (ub ? red_d[o] : 0.f));
      red_a[t] = r;
      red_m[t] = Mn;
    }
    __syncthreads();
  }
  if (tg == 0) {
    const f32x4 sum = red_a[t];
    const float dsum = red_d[t];
    const float inv = dsum > 0.f ? 1.0f / dsum : 0.f;
    u32x2 pk = {E::pack2(sum[0] * inv, sum[1] * inv), E::pack2(sum[2] * inv, sum[3] * inv)};
    if (!ready) pk = u32x2{0x7FC07FC0u, 0x7FC07FC0u};  // a merge that never saw its runs
    if (g < u.gg) {
      const int sq = MULTI ? p.sq : 1;
      const int qt = MULTI ? g / u.gh : 0;
      const int hq = u.hq0 + g - qt * u.gh;
      uint16_t* og = static_cast<uint16_t*>(p.o);
      *reinterpret_cast<u32x2*>(og + (((long long)u.b * sq + qt) * p.Hq + hq) * D +
                                kMergeDims * db + 4 * d4) = pk;
    }
  }
  // lower the flags for the next call (only this merger reads them)
  if (ready && t < 64) {
    for (int s = lane; s < nruns; s += 64) st_flag(fl + s, 0u);
  }
}

template <int D, int DT, bool PAGED, bool MULTI>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeParams p) {
  using E = Elt<DT>;
  using ST = Stage<D>;
  constexpr int NW = kDecodeWaves;
  constexpr int KSTEPS = D / 16;
  constexpr int DTILES = D / 32;
  constexpr int KST = ST::KST, VST = ST::VST;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];

  const int sq = MULTI ? p.sq : 1;
  const int hpg = MULTI ? p.hpg : 32;
  const int nunits = p.B * p.Hkv * ((p.gqa + hpg - 1) / hpg);
  const int nstream = nunits * p.nsplit;
  if ((int)blockIdx.x >= nstream) {
    merger<D, DT, MULTI>(p, (int)blockIdx.x - nstream, dyn_lds);
    return;
  }
  const int unit = (int)blockIdx.x / p.nsplit;
  const int split = (int)blockIdx.x - unit * p.nsplit;
  const UnitView u = unit_view<MULTI>(p, unit);
  const int b = u.b, hk = u.hk, gh = u.gh, gg = u.gg, cstride = u.cstride, hq0 = u.hq0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int li = lane & 31, lh = lane >> 5;
  const int ti = lane & 15;

  // Q of the group's columns (lane: column li, d = 16kk + 8lh + e) does not
  // depend on the valid length: its loads are issued first, without
  // branches (columns past gg read column 0 and are zeroed below), so their
  // round trip overlaps the valid-length read
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

  const int L = clamped_len(p, b);
  int cps, nruns;
  split_plan(L, p.nsplit, cps, nruns);
  if (split >= nruns) return;  // an empty run: no record, no flag
  const int nchunks = (L + 31) / 32;
  const int c0 = min(split * cps, nchunks);
  const int c1 = min(c0 + cps, nchunks);

  // Q as the B operand: columns past gg are zero, and the sign of the scale
  // is applied to Q (q_sign -1: negated, 0: zero), so the scores' scale
  // factor c is never negative.  The empty asm pins the result here, ahead
  // of every K/V load: computed later, its wait for Q would also wait for
  // the first chunk's loads.
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = qr[kk];
    x = p.q_sign < 0 ? (x ^ 0x80008000u) : x;
    qr[kk] = (li < gg && p.q_sign != 0) ? x : u32x4{0u, 0u, 0u, 0u};
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(qr[kk]));
#endif
  }

  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);
  const float c = p.c_log2;
  const long long tok_stride = (long long)p.Hkv * D;  // elements between tokens
  const long long cache_base =
      PAGED ? (long long)hk * D : (long long)b * p.capacity * tok_stride + (long long)hk * D;

  // Paged cache: logical page lp of batch b is physical page
  // page_table[b][lp] of a pool [num_pages, page_size, Hkv, D]; page_size is
  // a multiple of 32, so a 32-token chunk never straddles two pages.  Lane j
  // of a wave holds the physical page of the wave's j-th chunk.  Entries are
  // clamped to the pool, so no table value leads outside it.
  // (a wave with more than 64 chunks reloads the list for its next 64 every
  // 64 chunks)
  auto page_list = [&](int j0) {
    int pg = 0;
    const int chj = c0 + wave + NW * (j0 + lane);
    if (chj < c1) {
      const int e = p.page_table[(long long)b * p.pages_per_seq + (chj * 32) / p.page_size];
      pg = min(max(e, 0), p.num_pages - 1);
    }
    return pg;
  };
  int my_page = 0;
  if constexpr (PAGED) my_page = page_list(0);

  // K and V of this (batch, kv head) as buffer ranges that end at token L:
  // token j's row sits at byte j * tok_stride * 2, and rows at or past L read
  // zeros, so the invalid tail is never fetched
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kg + cache_base), (short)0, (int)(L * tok_stride * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vg + cache_base), (short)0, (int)(L * tok_stride * 2), kBufferFlags);

  // A chunk's padded LDS images are cut into 1 KiB pieces, one per buffer
  // load: image unit x (16 bytes) of K is row x / (KST/8), column x % (KST/8);
  // of V row x / (VST/8), column x % (VST/8).  Padding columns and rows past
  // the 32 of a chunk read from past the buffer's end (zeros).
  constexpr int KRC = KST / 8, VRC = VST / 8;
  unsigned koffs[ST::KNI], voffs[ST::VNI];
#pragma unroll
  for (int i = 0; i < ST::KNI; ++i) {
    const int x = 64 * i + lane;
    const int rr = x / KRC, cc = x - rr * KRC;
    koffs[i] = (rr < 32 && cc < D / 8) ? (unsigned)((rr * tok_stride + cc * 8) * 2) : kPastEnd;
  }
#pragma unroll
  for (int i = 0; i < ST::VNI; ++i) {
    const int x = 64 * i + lane;
    const int rr = x / VRC, cc = x - rr * VRC;
    voffs[i] = cc < D / 8 ? (unsigned)((rr * tok_stride + cc * 8) * 2) : kPastEnd;
  }
  unsigned char* wave_lds = dyn_lds + wave * kSlots * ST::SLOT;
  // per-lane LDS byte addresses of the operand reads inside a slot:
  // K row li, column 8 lh; V in the transposing read's lane pattern
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)wave_lds;
  const unsigned k_lane = (unsigned)((li * KST + 8 * lh) * 2);
  const unsigned v_lane =
      (unsigned)(ST::KBYTES + ((4 * lh + (ti >> 2)) * VST + 16 * ((lane >> 4) & 1) + 4 * (ti & 3)) * 2);

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

  auto load_chunk = [&](int ch, int slot) {
    int soff;
    __amdgpu_buffer_rsrc_t kc = krs, vc = vrs;
    if constexpr (!PAGED) {
      soff = ch * 32 * (int)tok_stride * 2;
    } else {
      // this chunk's page as a buffer range ending at token L
      const int lp = (ch * 32) / p.page_size;
      const int j = (ch - c0 - wave) / NW;  // the wave's j-th chunk
      if (j > 0 && (j & 63) == 0) my_page = page_list(j);
      const int phys = __builtin_amdgcn_readlane(my_page, j & 63);
      const int in_page = min(p.page_size, L - lp * p.page_size);
      const long long base = (long long)phys * p.page_size * tok_stride + cache_base;
      kc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kg + base), (short)0,
                                             (int)(in_page * tok_stride * 2), kBufferFlags);
      vc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vg + base), (short)0,
                                             (int)(in_page * tok_stride * 2), kBufferFlags);
      soff = (ch * 32 - lp * p.page_size) * (int)tok_stride * 2;
    }
    unsigned char* kdst = wave_lds + slot * ST::SLOT;
    unsigned char* vdst = kdst + ST::KBYTES;
#pragma unroll
    for (int i = 0; i < ST::KNI; ++i) lds_dma16_nt(kc, kdst + i * 1024, koffs[i], soff);
#pragma unroll
    for (int i = 0; i < ST::VNI; ++i) lds_dma16_nt(vc, vdst + i * 1024, voffs[i], soff);
  };

  auto compute_chunk = [&](int ch, const ChunkOperands<D>& op) {
    const int tok0 = ch * 32;
    // two independent accumulation chains (even / odd k-steps), added at the end
    f32x16 s = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; kk += 2) {
      s = E::mfma(op.k[kk], qr[kk], s);
      s1 = E::mfma(op.k[kk + 1], qr[kk + 1], s1);
    }
    s += s1;
    // scores of keys a column does not see are excluded (keys >= L had zero
    // K rows, not -inf)
    if (tok0 + 32 > mask_from) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = tok0 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (j > key_lim) s[r] = -__builtin_inff();
      }
    }
    // the exp2 reference m_run trails the running max by at most kRescaleTau:
    // it moves (and O and l are rescaled) only when some column of the wave
    // jumps above it by more than that, so p = exp2(s c - m_run) <= 2^tau and
    // the usual chunk touches none of the O accumulators.  O / l and the
    // merge are exact for any reference, so this changes rounding only.
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = pair_max(mx) * c;
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
      s[r] = fast_exp2(__builtin_fmaf(s[r], c, -m_use));
      psum += s[r];
    }
    l_run += psum;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r0 = 8 * kk;
      const u32x4 pb = {E::pack2(s[r0 + 0], s[r0 + 1]), E::pack2(s[r0 + 2], s[r0 + 3]),
                        E::pack2(s[r0 + 4], s[r0 + 5]), E::pack2(s[r0 + 6], s[r0 + 7])};
#pragma unroll
      for (int dt = 0; dt < DTILES; ++dt) {
        const u32x4 a = {op.v[kk][dt][0][0], op.v[kk][dt][0][1], op.v[kk][dt][1][0],
                         op.v[kk][dt][1][1]};
        oacc[dt] = E::mfma(a, pb, oacc[dt]);
      }
    }
  };

  // chunks c0 + wave, + NW, ...: the wave's slot is refilled with its next
  // chunk as soon as the current chunk's operands are in registers, before
  // the chunk's arithmetic; the other wave of the SIMD computes meanwhile
  {
    int ch = c0 + wave;
    if (ch < c1) load_chunk(ch, 0);
    while (ch < c1) {
      wait_vmem();  // chunk ch is in LDS
      ChunkOperands<D> op;
      op.read(lds_base + k_lane, lds_base + v_lane);
      const int nx = ch + NW;
      if (nx < c1) load_chunk(nx, 0);
      compute_chunk(ch, op);
      ch = nx;
    }
  }

  // ---- merge the waves of this workgroup (through LDS) -> run record ----
  __syncthreads();  // staging no longer needed; reuse dyn_lds
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
  float* merge_lds = wml + NW * cstride * 2;  // merge weights and per-column sums
  const long long recs = (long long)unit * p.nsplit;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      p.part_o + recs * cstride * D, (short)0, p.nsplit * cstride * D * 4, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + recs * cstride * 2, (short)0, p.nsplit * cstride * 2 * 4, kBufferFlags);
  uint16_t* og = static_cast<uint16_t*>(p.o);
  // O is [B, sq, Hq, D]: column (t, g) -> row (b, t, hq0 + g)
  const long long out_base = ((long long)b * sq * p.Hq + hq0) * D;
  const long long ostride = (long long)p.Hq * D;

  if (nruns == 1) {
    merge_waves<D, DT, MULTI>(wo, wml, NW, gg, cstride, ro, rml, 0, og, out_base, gh, ostride,
                              merge_lds);
    return;
  }
  merge_waves<D, DT, MULTI>(wo, wml, NW, gg, cstride, ro, rml, split, nullptr, 0, gh, ostride,
                            merge_lds);
  // the record is complete in memory before any flag goes up
  wait_vmem();
  __syncthreads();
  constexpr int DB = D / kMergeDims;
  if (tid < p.nmerge && p.merge_cols * (tid / DB) < gg)
    st_flag(p.flags + ((long long)unit * p.nmerge + tid) * p.nsplit + split, 1u);
}

template <int D, int DT, bool PAGED, bool MULTI>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  using ST = Stage<D>;
  const int HG = (p.gqa + p.hpg - 1) / p.hpg;
  const int cs = min(p.hpg, p.gqa) * p.sq;  // columns per record
  const int units = p.B * p.Hkv * HG;
  const size_t merge = ((size_t)kDecodeWaves * cs * (D + 2) + (size_t)cs * (kDecodeWaves + 2)) * 4;
  const size_t merger = 16 + (size_t)kThreads * (4 + 4 + 16);
  size_t lds = (size_t)ST::WG_BYTES;
  if (merge > lds) lds = merge;
  if (merger > lds) lds = merger;
  DecodeParams q = p;
  q.lds_bytes = (int)lds;
  const long long grid = (long long)units * p.nsplit + (p.nsplit > 1 ? (long long)units * p.nmerge : 0);
  hipLaunchKernelGGL((decode_kernel<D, DT, PAGED, MULTI>), dim3((unsigned)grid),
                     dim3(kDecodeWaves * 64), lds, stream, q);
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

int decode_heads_per_group(int gqa, int sq) {
  const int h = 32 / sq;
  return gqa < h ? gqa : h;
}

DecodePlan decode_plan(int B, int Sq, int Hq, int Hkv, int D, int capacity) {
  DecodePlan pl;
  const int gqa = Hq / Hkv;
  pl.hpg = decode_heads_per_group(gqa, Sq);
  const int HG = (gqa + pl.hpg - 1) / pl.hpg;
  pl.cstride = pl.hpg * Sq;
  const long long units = (long long)B * Hkv * HG;
  pl.units = units;
  // mergers per unit: merge_cols columns x 32 dims each, the fewest columns
  // (most parallel merge) that keep the mergers of the launch within
  // kMaxMergers; they wait on the split workgroups, so they must stay few
  pl.merge_cols = 0;
  pl.nmerge = 0;
  for (int mc = 1; mc <= 4; mc *= 2) {
    const int nm = ((pl.cstride + mc - 1) / mc) * (D / kMergeDims);
    if (units * nm <= kMaxMergers) {
      pl.merge_cols = mc;
      pl.nmerge = nm;
      break;
    }
  }
  // splits per unit: kDecodeTargetWGs split workgroups over all units, each
  // run at least kMinSplitChunks chunks long at full capacity, at most
  // kMaxSplits
  const long long chunks = ((long long)capacity + 31) / 32;
  long long ns = units > 0 ? kDecodeTargetWGs / units : 1;
  const long long by_len = (chunks + kMinSplitChunks - 1) / kMinSplitChunks;
  if (ns > by_len) ns = by_len;
  if (ns > kMaxSplits) ns = kMaxSplits;
  if (ns < 2 || pl.nmerge == 0) ns = 1;
  pl.nsplit = (int)ns;
  if (pl.nsplit == 1) {
    pl.nmerge = 0;
    pl.merge_cols = 0;
  }
  return pl;
}

size_t decode_workspace_layout(int B, int Sq, int Hq, int Hkv, int D, int capacity,
                               size_t* off_o, size_t* off_ml) {
  // The flags come first, in a region of fixed size (the most any split
  // launch raises: units x mergers <= kMaxMergers, runs <= kMaxSplits), so
  // that whatever shapes share a workspace, the flags of every call sit
  // where no call writes anything but flags -- and every completed call
  // leaves them at zero.  Records follow.
  const DecodePlan pl = decode_plan(B, Sq, Hq, Hkv, D, capacity);
  if (pl.nsplit <= 1) {
    if (off_o) *off_o = 0;
    if (off_ml) *off_ml = 0;
    return 256;
  }
  const size_t recs = (size_t)pl.units * pl.nsplit * (size_t)pl.cstride;
  size_t bytes = kDecodeFlagBytes;
  if (off_o) *off_o = bytes;
  bytes += recs * (size_t)D * 4;                // part_o
  bytes = (bytes + 255) & ~(size_t)255;
  if (off_ml) *off_ml = bytes;
  bytes += recs * 2 * 4;                        // part_ml
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t stream) {
  if (D == 128) {
    return dtype == kBF16 ? launch_p<128, kBF16>(p, stream) : launch_p<128, kFP16>(p, stream);
  }
  return dtype == kBF16 ? launch_p<64, kBF16>(p, stream) : launch_p<64, kFP16>(p, stream);
}

hipError_t decode_scratch(void** ptr) {
  // the address of `scratch` on the current device, looked up once per device
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa
