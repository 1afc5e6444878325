// C-ABI front end: argument checks (all before any HIP call), the prefill
// launch plan, and dispatch to the gfx950 kernels.
#include "../../include/fa.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "fa_internal.h"

namespace {

constexpr double kLog2e = 1.442695040888963407359924681001892137;
// persistent launches use the work queue from this many items per workgroup
constexpr int kQueueMinItemsPerCTA = 12;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// n = a*b*c*d elements with overflow detection (all factors >= 0)
bool mul_ok(long long a, long long b, long long* out) {
  if (a == 0 || b == 0) {
    *out = 0;
    return true;
  }
  if (a > LLONG_MAX / b) return false;
  *out = a * b;
  return true;
}
bool count4(long long a, long long b, long long c, long long d, long long* n) {
  long long t;
  return mul_ok(a, b, &t) && mul_ok(t, c, &t) && mul_ok(t, d, n);
}

bool overlaps(const void* a, long long abytes, const void* b, long long bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// scale -> (|scale| * log2 e, sign applied to q in registers).  A zero scale
// makes every admissible score 0: q is zeroed and c = 1.
void fold_scale(float scale, float* c, int* q_sign) {
  if (scale == 0.f) {
    *c = 1.f;
    *q_sign = 0;
  } else {
    *c = (float)(std::fabs((double)scale) * kLog2e);
    *q_sign = scale < 0.f ? -1 : 1;
  }
}

// KV tiles of query block qb of a dense work item (all tiles when not causal)
long long block_tiles(long long qb, int Sq, int Sk, int causal) {
  const int BM = fa::kPrefillBM, BN = fa::kPrefillBN;
  long long kv_end = Sk;
  if (causal) {
    const long long qlast = qb * BM + BM < Sq ? qb * BM + BM : Sq;  // one past the last row
    kv_end = qlast + (long long)Sk - Sq;
    if (kv_end < 0) kv_end = 0;
    if (kv_end > Sk) kv_end = Sk;
  }
  return (kv_end + BN - 1) / BN;
}

// workgroups of a key-split launch with at most T tiles per part: an item of
// nt tiles has ceil(nt / T) parts, at least one
long long split_parts(int B, int Hq, int Sq, int Sk, int causal, long long T) {
  const long long nqb = ((long long)Sq + fa::kPrefillBM - 1) / fa::kPrefillBM;
  long long n = 0;
  for (long long qb = 0; qb < nqb; ++qb) {
    const long long nt = block_tiles(qb, Sq, Sk, causal);
    n += nt > T ? (nt + T - 1) / T : 1;
  }
  return n * Hq * B;
}

// `dense`: a dense batch (the key split applies); varlen plans pass false
fa_status_t plan_prefill(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                         fa_fwd_plan_t* plan, bool dense = true) {
  if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const int BM = fa::kPrefillBM, BN = fa::kPrefillBN;
  const long long nqb = ((long long)Sq + BM - 1) / BM;
  long long items;
  if (!count4(nqb, Hq, B, 1, &items) || items > INT_MAX) return FA_ERR_SHAPE;
  std::memset(plan, 0, sizeof(*plan));
  plan->block_m = BM;
  plan->block_n = BN;
  plan->work_items = (int)items;
  const int NP = fa::kPersistentCTAs;
  // persistent grid-stride once there are at least as many items as CTAs
  // (page "Dense flash-attention prefill": dense_persistent="auto")
  const int persistent = items >= NP ? 1 : 0;
  plan->persistent = persistent;
  plan->grid = persistent ? (int)(items < NP ? items : NP) : (int)items;
  // kv-head-major order when GQA and gqa*NQB*B >= 2*NP, else query-block-major
  const long long gqa = Hq / Hkv;
  const int hkv = (persistent && gqa > 1 && gqa * nqb * B >= 2LL * NP) ? 1 : 0;
  // XCD-aware dealing of the (batch, kv head) units, possible when the
  // persistent grid and the unit count both split evenly over the XCDs (every
  // XCD then holds the same multiset of items).  Chosen where the order is
  // query-block-major: each round then spans every unit, and without the
  // dealing every XCD's L2 would fetch the K/V of all of them.  Kv-head-major
  // rounds already span one or two kv heads.
  const bool xcd_ok = persistent && plan->grid == NP && NP % fa::kXcds == 0 &&
                      ((long long)B * Hkv) % fa::kXcds == 0;
  plan->hkv_major = hkv;
  plan->xcd_map = (xcd_ok && !hkv) ? 1 : 0;
  // Work queue when every workgroup has many items: dealing them to free
  // workgroups evens out XCDs that run at different speeds, which pays for
  // the queue's fixed costs (an atomic per item, one at the launch's end)
  // only on long launches.  Its list runs heaviest query block first across
  // all heads (query-block-major, no XCD dealing): measured on the causal
  // B=1 Hq=128 Hkv=8 S=8192 shape, 0.5-1% faster than the kv-head-major
  // list, static or queued.
  if (dense && persistent && items >= (long long)kQueueMinItemsPerCTA * NP) {
    plan->queue = 1;
    plan->hkv_major = 0;
    plan->xcd_map = 0;
  }
  // tiles streamed and tiles needing the mask, per query block (x Hq*B)
  long long tiles = 0, masked = 0;
  const long long off = (long long)Sk - Sq;
  for (long long qb = 0; qb < nqb; ++qb) {
    const long long q0 = qb * BM;
    const long long qlast = (q0 + BM < Sq ? q0 + BM : Sq);  // one past the last row
    long long kv_end = Sk;
    long long free_t = Sk / BN;
    if (causal) {
      kv_end = qlast + off;
      if (kv_end < 0) kv_end = 0;
      if (kv_end > Sk) kv_end = Sk;
      long long f = q0 + off + 1;
      if (f < 0) f = 0;
      f /= BN;
      if (f < free_t) free_t = f;
    }
    const long long nt = (kv_end + BN - 1) / BN;
    tiles += nt;
    masked += nt > free_t ? nt - free_t : 0;
  }
  plan->kv_tiles = tiles * Hq * (long long)B;
  plan->masked_tiles = masked * Hq * (long long)B;
  // Key split of an under-filled launch: the smallest tiles-per-part T whose
  // parts still fit one workgroup per CU (the part count only falls as T
  // grows, and T = the longest item's tile count gives the unsplit items,
  // fewer than the CUs).  Taken when it cuts the longest item by at least
  // kSplitMinTiles tiles, which pays for the merge of the parts.
  if (dense && !persistent && items > 0) {
    // the last query block has the most keys (all blocks alike when not causal)
    const long long max_nt = block_tiles(nqb - 1, Sq, Sk, causal);
    long long lo = fa::kSplitMinTiles, hi = max_nt;
    if (lo < hi) {
      while (lo < hi) {
        const long long mid = lo + (hi - lo) / 2;
        if (split_parts(B, Hq, Sq, Sk, causal, mid) <= fa::kSplitMaxParts) hi = mid;
        else lo = mid + 1;
      }
      if (lo <= max_nt - fa::kSplitMinTiles) {
        plan->split_tiles = (int)lo;
        plan->grid = (int)split_parts(B, Hq, Sq, Sk, causal, lo);
      }
    }
  }
  return FA_OK;
}

// A caller's launch plan for these sizes: the automatic plan with the
// schedule choices (persistent, hkv_major, xcd_map) taken from `want`.
// Choices that do not fit the sizes are rejected.
fa_status_t apply_plan(const fa_fwd_plan_t* want, fa_fwd_plan_t* plan, int B, int Hq, int Hkv,
                       int Sq, int Sk, int causal) {
  if ((want->persistent != 0 && want->persistent != 1) ||
      (want->hkv_major != 0 && want->hkv_major != 1) || (want->xcd_map != 0 && want->xcd_map != 1) ||
      (want->queue != 0 && want->queue != 1) || want->split_tiles < 0)
    return FA_ERR_SHAPE;
  if (want->split_tiles > 0) {
    if (want->persistent || want->hkv_major || want->xcd_map || want->queue) return FA_ERR_SHAPE;
    const long long parts = split_parts(B, Hq, Sq, Sk, causal, want->split_tiles);
    if (parts > fa::kSplitMaxParts) return FA_ERR_SHAPE;
    plan->persistent = 0;
    plan->grid = (int)parts;
    plan->hkv_major = 0;
    plan->xcd_map = 0;
    plan->queue = 0;
    plan->split_tiles = want->split_tiles;
    return FA_OK;
  }
  plan->split_tiles = 0;
  const int NP = fa::kPersistentCTAs;
  const int persistent = want->persistent && plan->work_items > 0 ? 1 : 0;
  const int grid = persistent ? (plan->work_items < NP ? plan->work_items : NP) : plan->work_items;
  if (want->xcd_map && !(persistent && grid == NP && NP % fa::kXcds == 0 &&
                         ((long long)B * Hkv) % fa::kXcds == 0))
    return FA_ERR_SHAPE;
  if (want->queue && !persistent) return FA_ERR_SHAPE;
  plan->persistent = persistent;
  plan->grid = grid;
  plan->hkv_major = want->hkv_major;
  plan->xcd_map = want->xcd_map;
  plan->queue = want->queue;
  return FA_OK;
}

// Prefill workspace, one per (device, stream): the split and work-queue
// counters (zeroed here once; every launch leaves them at zero) and the split
// part records.  Kept until the process ends, as a stream's launches may
// still be in flight.
struct SplitWorkspace {
  int device;
  void* stream;
  void* ptr;
};
std::mutex g_split_mu;
std::vector<SplitWorkspace> g_split_ws;

hipError_t split_workspace(void* stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_split_mu);
  for (const SplitWorkspace& w : g_split_ws)
    if (w.device == dev && w.stream == stream) {
      *out = w.ptr;
      return hipSuccess;
    }
  void* ptr = nullptr;
  if ((e = hipMalloc(&ptr, fa::kSplitWorkspaceBytes)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(ptr, 0, fa::kSplitCounterBytes, static_cast<hipStream_t>(stream))) !=
      hipSuccess) {
    (void)hipFree(ptr);
    return e;
  }
  g_split_ws.push_back({dev, stream, ptr});
  *out = ptr;
  return hipSuccess;
}

fa_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale, int dtype,
                     void* stream, const fa_fwd_plan_t* want = nullptr) {
  fa_fwd_plan_t plan;
  fa_status_t ps = plan_prefill(B, Hq, Hkv, Sq, Sk, D, causal, &plan);
  if (ps != FA_OK) return ps;
  if (want && (ps = apply_plan(want, &plan, B, Hq, Hkv, Sq, Sk, causal)) != FA_OK) return ps;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  long long nq, nkv, nlse;
  if (!count4(B, Hq, Sq, D, &nq) || !count4(B, Hkv, Sk, D, &nkv) || !count4(B, Hq, Sq, 1, &nlse))
    return FA_ERR_SHAPE;
  if (nq > LLONG_MAX / 2 || nkv > LLONG_MAX / 2 || nlse > LLONG_MAX / 4) return FA_ERR_SHAPE;
  // one (batch, kv head) of K or V is addressed with 32-bit byte offsets
  if ((long long)Sk * D * 2 > INT_MAX) return FA_ERR_SHAPE;
  // pointers may be NULL only for empty tensors
  if (nq > 0 && (!q || !o)) return FA_ERR_NULL;
  if (nkv > 0 && (!k || !v)) return FA_ERR_NULL;
  for (const void* ptr : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(lse)})
    if (ptr && !aligned16(ptr)) return FA_ERR_ALIGN;
  const long long ob = nq * 2, kb = nkv * 2;
  if (overlaps(o, ob, q, ob) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb))
    return FA_ERR_ALIAS;
  if (lse && (overlaps(lse, nlse * 4, q, ob) || overlaps(lse, nlse * 4, k, kb) ||
              overlaps(lse, nlse * 4, v, kb) || overlaps(lse, nlse * 4, o, ob)))
    return FA_ERR_ALIAS;
  if (nq == 0) return FA_OK;  // nothing to compute

  fa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_bstride = (long long)Hq * Sq * D;
  p.kv_bstride = (long long)Hkv * Sk * D;
  p.cu_q = nullptr;
  p.cu_k = nullptr;
  p.total_q = 0;
  p.total_k = 0;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.gqa = Hq / Hkv;
  p.nqb = (Sq + fa::kPrefillBM - 1) / fa::kPrefillBM;
  p.work_items = plan.work_items;
  p.hkv_major = plan.hkv_major;
  p.persistent = plan.persistent;
  p.xcd_map = plan.xcd_map;
  fold_scale(scale, &p.c_log2, &p.q_sign);
  p.split_tiles = plan.split_tiles;
  p.split_cnt = nullptr;
  p.split_rec = nullptr;
  p.queue = nullptr;
  if (plan.split_tiles > 0 || plan.queue) {
    void* ws = nullptr;
    if (split_workspace(stream, &ws) != hipSuccess) return FA_ERR_HIP;
    p.split_cnt = static_cast<unsigned*>(ws);
    p.split_rec = reinterpret_cast<float*>(static_cast<char*>(ws) + fa::kSplitCounterBytes);
    if (plan.queue) p.queue = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + fa::kQueueOffset);
  }
  const hipError_t e = fa::launch_prefill(p, D, dtype, causal != 0, plan.grid,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t varlen_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_q, const int32_t* cu_k, int B, int Hq, int Hkv,
                        int total_q, int total_k, int max_sq, int max_sk, int D, int causal,
                        float scale, int dtype) {
  if (total_q < 0 || total_k < 0) return FA_ERR_SHAPE;
  // the launch plan of a dense batch of B sequences of the maximum lengths
  fa_fwd_plan_t plan;
  const fa_status_t ps = plan_prefill(B, Hq, Hkv, max_sq, max_sk, D, causal, &plan, false);
  if (ps != FA_OK) return ps;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  long long nq, nkv;
  if (!count4(total_q, Hq, D, 1, &nq) || !count4(total_k, Hkv, D, 1, &nkv)) return FA_ERR_SHAPE;
  if (nq > LLONG_MAX / 4 || nkv > LLONG_MAX / 2) return FA_ERR_SHAPE;
  // one sequence's K or V is addressed with 32-bit byte offsets
  if ((long long)max_sk * Hkv * D * 2 > INT_MAX) return FA_ERR_SHAPE;
  if (B > 0 && (!cu_q || !cu_k)) return FA_ERR_NULL;
  if (nq > 0 && (!q || !o)) return FA_ERR_NULL;
  if (nkv > 0 && (!k || !v)) return FA_ERR_NULL;
  for (const void* ptr : {q, k, v, static_cast<const void*>(o), static_cast<const void*>(lse)})
    if (ptr && !aligned16(ptr)) return FA_ERR_ALIGN;
  for (const void* ptr : {static_cast<const void*>(cu_q), static_cast<const void*>(cu_k)})
    if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3u) != 0) return FA_ERR_ALIGN;
  const long long ob = nq * 2, kb = nkv * 2, lb = (long long)total_q * Hq * 4, cb = (B + 1LL) * 4;
  if (overlaps(o, ob, q, ob) || overlaps(o, ob, k, kb) || overlaps(o, ob, v, kb) ||
      overlaps(o, ob, cu_q, cb) || overlaps(o, ob, cu_k, cb))
    return FA_ERR_ALIAS;
  if (lse && (overlaps(lse, lb, q, ob) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
              overlaps(lse, lb, o, ob) || overlaps(lse, lb, cu_q, cb) ||
              overlaps(lse, lb, cu_k, cb)))
    return FA_ERR_ALIAS;
  return FA_OK;
}

fa_status_t launch_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_q, const int32_t* cu_k, int B, int Hq, int Hkv,
                          int total_q, int total_k, int max_sq, int max_sk, int D, int causal,
                          float scale, int dtype, void* stream) {
  const fa_status_t st = varlen_impl(q, k, v, o, lse, cu_q, cu_k, B, Hq, Hkv, total_q, total_k,
                                     max_sq, max_sk, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  if (B == 0 || max_sq == 0 || total_q == 0) return FA_OK;
  fa_fwd_plan_t plan;
  plan_prefill(B, Hq, Hkv, max_sq, max_sk, D, causal, &plan, false);
  fa::PrefillParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_bstride = 0;
  p.kv_bstride = 0;
  p.cu_q = cu_q;
  p.cu_k = cu_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = max_sq;
  p.Sk = max_sk;
  p.gqa = Hq / Hkv;
  p.nqb = (max_sq + fa::kPrefillBM - 1) / fa::kPrefillBM;
  p.work_items = plan.work_items;
  p.hkv_major = plan.hkv_major;
  p.persistent = plan.persistent;
  // XCD dealing of whole kv heads (every kv head holds the same items) when
  // the launch is persistent over one workgroup per CU
  p.xcd_map = (plan.persistent && plan.grid == fa::kPersistentCTAs &&
               fa::kPersistentCTAs % fa::kXcds == 0 && Hkv % fa::kXcds == 0) ? 1 : 0;
  fold_scale(scale, &p.c_log2, &p.q_sign);
  p.split_tiles = 0;
  p.split_cnt = nullptr;
  p.split_rec = nullptr;
  p.queue = nullptr;
  if (plan.queue) {
    void* ws = nullptr;
    if (split_workspace(stream, &ws) != hipSuccess) return FA_ERR_HIP;
    p.queue = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + fa::kQueueOffset);
  }
  const hipError_t e = fa::launch_prefill(p, D, dtype, causal != 0, plan.grid,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Sq = 1 decode over a contiguous cache (page_table == nullptr) or a paged
// pool; all checks before any HIP call.
constexpr long long kMaxPagedCapacity = 1LL << 21;  // tokens a paged sequence may span
constexpr int kMaxDecodeSq = 32;                    // query tokens of one decode step

fa_status_t decode_impl(const void* q, const void* kc, const void* vc, const int32_t* valid_len,
                        const int32_t* page_table, int page_size, int pages_per_seq,
                        int num_pages, int capacity, void* o, int B, int Sq, int Hq, int Hkv,
                        int D, int causal, float scale, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream, bool launch = true) {
  const bool paged = page_size > 0;
  if (B < 0 || Hq < 1 || Hkv < 1 || capacity < 1) return FA_ERR_SHAPE;
  if (Sq < 1 || Sq > kMaxDecodeSq) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  long long nq, ncache, ntable = 0;
  if (!count4(B, Sq, Hq, D, &nq)) return FA_ERR_SHAPE;
  if (paged) {
    if (!count4(num_pages, page_size, Hkv, D, &ncache) || !count4(B, pages_per_seq, 1, 1, &ntable))
      return FA_ERR_SHAPE;
    // one page is addressed by 32-bit byte offsets from its base
    if ((long long)page_size * Hkv * D * 2 > INT_MAX) return FA_ERR_SHAPE;
  } else {
    if (!count4(B, capacity, Hkv, D, &ncache)) return FA_ERR_SHAPE;
    // one batch's cache is addressed by 32-bit byte offsets from its base
    if ((long long)capacity * Hkv * D * 2 > INT_MAX) return FA_ERR_SHAPE;
  }
  if (ncache > LLONG_MAX / 2 || ntable > LLONG_MAX / 4 || (long long)B * Hkv > INT_MAX / 64)
    return FA_ERR_SHAPE;
  if (B == 0) return FA_OK;
  if (!q || !kc || !vc || !valid_len || !o || (paged && !page_table)) return FA_ERR_NULL;
  for (const void* ptr : {q, kc, vc, static_cast<const void*>(o)})
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(valid_len) & 3u) != 0) return FA_ERR_ALIGN;
  if (paged && (reinterpret_cast<uintptr_t>(page_table) & 3u) != 0) return FA_ERR_ALIGN;
  const size_t need =
      fa::decode_workspace_layout(B, Sq, Hq, Hkv, D, capacity, nullptr, nullptr);
  if (!workspace || workspace_bytes < need ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return FA_ERR_WORKSPACE;
  const long long ob = nq * 2, cb = ncache * 2;
  if (overlaps(o, ob, q, ob) || overlaps(o, ob, kc, cb) || overlaps(o, ob, vc, cb) ||
      overlaps(o, ob, valid_len, (long long)B * 4) || overlaps(o, ob, workspace, (long long)need) ||
      overlaps(o, ob, page_table, ntable * 4))
    return FA_ERR_ALIAS;
  if (!launch) return FA_OK;  // checks only

  fa::DecodeParams p;
  p.q = q;
  p.k = kc;
  p.v = vc;
  p.valid_len = valid_len;
  p.o = o;
  size_t off_o = 0, off_ml = 0;
  fa::decode_workspace_layout(B, Sq, Hq, Hkv, D, capacity, &off_o, &off_ml);
  const fa::DecodePlan plan = fa::decode_plan(B, Sq, Hq, Hkv, D, capacity);
  char* ws = static_cast<char*>(workspace);
  p.flags = reinterpret_cast<unsigned*>(ws);
  p.part_o = reinterpret_cast<float*>(ws + off_o);
  p.part_ml = reinterpret_cast<float*>(ws + off_ml);
  p.page_table = paged ? page_table : nullptr;
  p.page_size = page_size;
  p.pages_per_seq = pages_per_seq;
  p.num_pages = num_pages;
  p.gqa = Hq / Hkv;
  p.sq = Sq;
  p.hpg = plan.hpg;
  p.causal = causal ? 1 : 0;
  p.nsplit = plan.nsplit;
  p.nmerge = plan.nmerge;
  p.merge_cols = plan.merge_cols;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.capacity = capacity;
  fold_scale(scale, &p.c_log2, &p.q_sign);
  const hipError_t e = fa::launch_decode(p, D, dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t paged_impl(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* page_table, const int32_t* valid_len, int page_size,
                       int pages_per_seq, int num_pages, void* o, int B, int Sq, int Hq, int Hkv,
                       int D, int causal, float scale, int dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (page_size < 32 || page_size % 32 != 0 || pages_per_seq < 1 || num_pages < 1)
    return FA_ERR_SHAPE;
  const long long capacity = (long long)pages_per_seq * page_size;
  if (capacity > kMaxPagedCapacity) return FA_ERR_SHAPE;
  return decode_impl(q, k_pages, v_pages, valid_len, page_table, page_size, pages_per_seq,
                     num_pages, (int)capacity, o, B, Sq, Hq, Hkv, D, causal, scale, dtype,
                     workspace, workspace_bytes, stream);
}

size_t bwd_workspace_bytes(long long rows) { return (size_t)((rows * 4 + 255) / 256 * 256); }

fa_status_t bwd_impl(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Sq < 0 || Sk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_FP16) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_SCALE;
  long long nq, nkv, rows;
  if (!count4(B, Hq, Sq, D, &nq) || !count4(B, Hkv, Sk, D, &nkv) || !count4(B, Hq, Sq, 1, &rows))
    return FA_ERR_SHAPE;
  if (nq > LLONG_MAX / 4 || nkv > LLONG_MAX / 4) return FA_ERR_SHAPE;
  // workgroup counts of the three launches fit a grid dimension
  if (rows / 32 + 1 > INT_MAX || (long long)B * Hq * ((Sq + 127) / 128) > INT_MAX ||
      (long long)B * Hkv * ((Sk + 127) / 128) > INT_MAX)
    return FA_ERR_SHAPE;
  if (nq > 0 && (!q || !o || !dout || !lse || !dq)) return FA_ERR_NULL;
  if (nkv > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  for (const void* ptr : {q, k, v, o, dout, static_cast<const void*>(dq),
                          static_cast<const void*>(dk), static_cast<const void*>(dv)})
    if (ptr && !aligned16(ptr)) return FA_ERR_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return FA_ERR_ALIGN;
  const size_t need = bwd_workspace_bytes(rows);
  if (rows > 0 && (!workspace || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
    return FA_ERR_WORKSPACE;
  const long long qb = nq * 2, kb = nkv * 2, lb = rows * 4;
  const void* ins[] = {q, k, v, o, dout, lse, workspace};
  const long long insz[] = {qb, kb, kb, qb, qb, lb, (long long)need};
  const void* outs[] = {dq, dk, dv};
  const long long outsz[] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ALIAS;
  }
  if (B == 0 || (Sq == 0 && Sk == 0)) return FA_OK;  // nothing to write
  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dsum = static_cast<float*>(workspace);
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.gqa = Hq / Hkv;
  fold_scale(scale, &p.c_log2, &p.q_sign);
  p.scale = scale;
  const hipError_t e =
      fa::launch_backward(p, D, dtype, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                          int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                          int max_seqlen_k, int D, int causal, float scale, int dtype,
                          void* stream) {
  return launch_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k,
                       max_seqlen_q, max_seqlen_k, D, causal, scale, dtype, stream);
}

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv,
                   int Sq, int Sk, int D, int causal, float scale, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, nullptr, B, Hq, Hkv, Sq, Sk, D, causal, scale, dtype, stream);
}

fa_status_t fa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                       int dtype, void* stream) {
  long long nlse;
  if (B >= 0 && Hq >= 1 && Sq >= 0 && count4(B, Hq, Sq, 1, &nlse) && nlse > 0 && !lse)
    return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, dtype, stream);
}

fa_status_t fa_fwd_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                        fa_fwd_plan_t* plan) {
  if (!plan) return FA_ERR_NULL;
  return plan_prefill(B, Hq, Hkv, Sq, Sk, D, causal, plan);
}

fa_status_t fa_fwd_planned(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                           int dtype, const fa_fwd_plan_t* plan, void* stream) {
  if (!plan) return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, causal, scale, dtype, stream, plan);
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int capacity) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || (D != 64 && D != 128) || capacity < 1) return 0;
  return fa::decode_workspace_layout(B, 1, Hq, Hkv, D, capacity, nullptr, nullptr);
}

size_t fa_decode_multi_workspace_bytes(int B, int Sq, int Hq, int Hkv, int D, int capacity) {
  if (B < 0 || Sq < 1 || Sq > kMaxDecodeSq || Hq < 1 || Hkv < 1 || Hq % Hkv ||
      (D != 64 && D != 128) || capacity < 1)
    return 0;
  return fa::decode_workspace_layout(B, Sq, Hq, Hkv, D, capacity, nullptr, nullptr);
}

fa_status_t fa_decode(const void* q, const void* kcache, const void* vcache,
                      const int32_t* valid_len, int capacity, void* o, int B, int Hq, int Hkv,
                      int D, int causal, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  // at Sq = 1 the bottom-right causal mask admits every valid token
  return decode_impl(q, kcache, vcache, valid_len, nullptr, 0, 0, 0, capacity, o, B, 1, Hq, Hkv,
                     D, causal, scale, dtype, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                              const int32_t* valid_len, int capacity, void* o, int B, int Hq,
                              int Hkv, int D, int causal, float scale, int dtype, void* stream) {
  // every check first, against a stand-in address for the built-in workspace
  // (its size is what matters here); then the one HIP call of the set-up
  void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
  fa_status_t st = decode_impl(q, kcache, vcache, valid_len, nullptr, 0, 0, 0, capacity, o, B, 1,
                               Hq, Hkv, D, causal, scale, dtype, stand_in,
                               fa::kDecodeScratchBytes, stream, false);
  if (st != FA_OK || B == 0) return st;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  return decode_impl(q, kcache, vcache, valid_len, nullptr, 0, 0, 0, capacity, o, B, 1, Hq, Hkv,
                     D, causal, scale, dtype, ws, fa::kDecodeScratchBytes, stream);
}

fa_status_t fa_decode_multi(const void* q, const void* kcache, const void* vcache,
                            const int32_t* valid_len, int capacity, void* o, int B, int Sq,
                            int Hq, int Hkv, int D, int causal, float scale, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, kcache, vcache, valid_len, nullptr, 0, 0, 0, capacity, o, B, Sq, Hq, Hkv,
                     D, causal, scale, dtype, workspace, workspace_bytes, stream);
}

fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* page_table, const int32_t* valid_len, int page_size,
                            int pages_per_seq, int num_pages, void* o, int B, int Hq, int Hkv,
                            int D, int causal, float scale, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return paged_impl(q, k_pages, v_pages, page_table, valid_len, page_size, pages_per_seq,
                    num_pages, o, B, 1, Hq, Hkv, D, causal, scale, dtype, workspace,
                    workspace_bytes, stream);
}

fa_status_t fa_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_table, const int32_t* valid_len,
                                  int page_size, int pages_per_seq, int num_pages, void* o, int B,
                                  int Sq, int Hq, int Hkv, int D, int causal, float scale,
                                  int dtype, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return paged_impl(q, k_pages, v_pages, page_table, valid_len, page_size, pages_per_seq,
                    num_pages, o, B, Sq, Hq, Hkv, D, causal, scale, dtype, workspace,
                    workspace_bytes, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq) {
  long long rows;
  if (B < 0 || Hq < 1 || Sq < 0 || !count4(B, Hq, Sq, 1, &rows)) return 0;
  return bwd_workspace_bytes(rows);
}

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
                   int Sk, int D, int causal, float scale, int dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Sq, Sk, D, causal, scale, dtype,
                  workspace, workspace_bytes, stream);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid or overflowing sizes";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head_dim must be 64 or 128, dtype bf16 or fp16";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale is not finite";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or too small (fa_decode_noalloc: the sizes need more than its built-in workspace)";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime refused the launch";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: the output overlaps an input";
    default: return "unknown fa status";
  }
}

}  // extern "C"
