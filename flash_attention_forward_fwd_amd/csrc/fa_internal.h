// Internal interface between the C-ABI front end (fa_api.cpp) and the HIP
// kernels (fa_prefill.hip, fa_decode.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// ---------------------------------------------------------------------------
// Prefill (dense forward)
// ---------------------------------------------------------------------------
#ifndef FA_PREFILL_WAVES
#define FA_PREFILL_WAVES 8
#endif
constexpr int kPrefillWaves = FA_PREFILL_WAVES;  // waves per workgroup, 32 query rows each
constexpr int kPrefillBM = 32 * kPrefillWaves;   // query rows per work item
#ifndef FA_PREFILL_BN
#define FA_PREFILL_BN 128
#endif
constexpr int kPrefillBN = FA_PREFILL_BN;        // keys per KV tile (64 or 128)
constexpr int kNumCUs = 256;                     // MI355X compute units
// two waves per SIMD: 8 waves per CU
constexpr int kPrefillCTAsPerCU = 8 / kPrefillWaves;
constexpr int kPersistentCTAs = kNumCUs * kPrefillCTAsPerCU;
// MI355X accelerator dies (XCDs), each with its own L2; workgroup i of a
// launch is dispatched to XCD i % kXcds
constexpr int kXcds = 8;

// Key-split schedule for launches with fewer work items than CUs: each item's
// key tiles are cut into parts of at most split_tiles tiles, one workgroup per
// part, and the item's last part to finish merges the others' partial results.
constexpr int kSplitMinTiles = 2;      // a part holds at least this many tiles
constexpr int kSplitMaxParts = kNumCUs; // workgroups of a split launch at most
// Workspace of a (device, stream): the split launches' per-item counters
// (arrivals, records written) and the persistent launches' work-queue
// counters (one ticket counter per item list, then a finished-workgroup
// counter), all zero between launches, then the split part records.
constexpr size_t kSplitCounterBytes = 4096;
constexpr size_t kQueueOffset = 2048;  // bytes from the workspace start
static_assert(kSplitMaxParts * 2 * sizeof(unsigned) <= kQueueOffset, "split counters fit");
static_assert(kQueueOffset + 16 * sizeof(unsigned) <= kSplitCounterBytes, "queue counters fit");
// fp32 record of one part: per wave and lane D/2 O values, then (m, l)
constexpr size_t split_record_bytes(int D) { return (size_t)kPrefillWaves * 64 * (D / 2 + 2) * 4; }
constexpr size_t kSplitWorkspaceBytes = kSplitCounterBytes + kSplitMaxParts * split_record_bytes(128);

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // nullptr unless the LSE variant runs
  long long q_bstride; // elements between batches of q / o  (Hq * Sq * D)
  long long kv_bstride;// elements between batches of k / v  (Hkv * Sk * D)
  // varlen (packed [total, H, D] tensors): device int32[B + 1] row offsets of
  // the sequences; nullptr for the dense layout.  Sq / Sk are then the
  // maximum sequence lengths.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  int B, Hq, Hkv, Sq, Sk;
  int gqa;             // Hq / Hkv
  int nqb;             // ceil(Sq / BM)
  int work_items;      // nqb * Hq * B
  int hkv_major;       // work-item order
  int persistent;      // grid-stride over work items
  // 1: the B * Hkv (batch, kv head) units are dealt to the XCDs (unit u to
  // XCD u % kXcds) and each XCD's workgroups stride over its own units'
  // items, so a kv head's K/V tiles are fetched into one L2 only.  Needs a
  // persistent grid of a multiple of kXcds workgroups and B * Hkv a multiple
  // of kXcds; hkv_major then orders each XCD's list unit-major.  Varlen
  // (compacted list): whole kv heads are dealt (Hkv a multiple of kXcds),
  // each XCD's list in block-major order.
  int xcd_map;
  float c_log2;        // |scale| * log2(e), or 1 when scale == 0
  int q_sign;          // +1, -1, or 0 (scale == 0): applied to q in registers
  // key split (dense, non-persistent, query-block-major): tiles per part, 0
  // for none; the grid is then the number of parts.  split_cnt: 2 counters
  // per work item, zero between launches; split_rec: one record per part.
  int split_tiles;
  unsigned* split_cnt;
  float* split_rec;
  // persistent launches: nullptr for the static round-robin over the item
  // list, else the work-queue counters (kXcds ticket counters, then the
  // finished-workgroup counter) that hand out items after each workgroup's
  // first
  unsigned* queue;
};

hipError_t launch_prefill(const PrefillParams& p, int D, int dtype, bool causal, int grid,
                          hipStream_t stream);

// ---------------------------------------------------------------------------
// Decode (Sq = 1 and few-token steps; split-KV merged inside the launch)
// ---------------------------------------------------------------------------
constexpr int kDecodeWaves = 4;
// split workgroups a decode launch aims for (one per CU)
#ifndef FA_DECODE_TARGET_WGS
#define FA_DECODE_TARGET_WGS 256
#endif
constexpr int kDecodeTargetWGs = FA_DECODE_TARGET_WGS;
constexpr int kDecodeChunk = 32;       // tokens per MFMA step
constexpr int kDecodeMaxGqa = 32;      // query heads sharing one kv head (MFMA N)
constexpr int kMinSplitChunks = 4;     // a split run holds at least this many chunks
constexpr int kMaxSplits = 256;        // split runs per unit at most
constexpr int kMaxMergers = 64;        // merger workgroups per launch at most

// Launch plan of a decode call: `units` (batch, kv head, head group) units of
// `cstride` record columns (query token x head), each split into at most
// `nsplit` runs whose records `nmerge` merger workgroups per unit combine
// (nsplit == 1: no records, no mergers).
struct DecodePlan {
  long long units;
  int hpg;       // query heads per head group
  int cstride;   // record columns: hpg * Sq
  int nsplit;
  int nmerge;
  int merge_cols;  // record columns per merger
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* valid_len;
  void* o;
  float* part_o;       // [units][nsplit][cstride][D] fp32 run records
  float* part_ml;      // [units][nsplit][cstride][2] fp32 (m in log2 domain, l)
  unsigned* flags;     // [units][nmerge][nsplit] run-complete flags, zero between calls
  // paged cache: device int32 [B][pages_per_seq] physical page of each
  // logical page of a pool [num_pages][page_size][Hkv][D]; nullptr for the
  // contiguous [B][capacity][Hkv][D] cache.  capacity = pages_per_seq *
  // page_size when paged.
  const int32_t* page_table;
  int page_size, pages_per_seq, num_pages;
  int B, Hq, Hkv, capacity;
  int gqa;
  int sq;              // query tokens per sequence (1 = plain decode), <= 32
  int hpg;             // query heads per head group: min(gqa, 32 / sq)
  int causal;          // bottom-right mask among the sq query tokens
  int nsplit;          // split runs per unit at most
  int nmerge;          // merger workgroups per unit (0 when nsplit == 1)
  int merge_cols;      // record columns each merger combines (1, 2 or 4)
  int lds_bytes;       // dynamic LDS of the launch (set by the launcher)
  float c_log2;
  int q_sign;
};

int decode_heads_per_group(int gqa, int sq);
DecodePlan decode_plan(int B, int Sq, int Hq, int Hkv, int D, int capacity);
// Workspace layout: the flags at offset 0 (kDecodeFlagBytes, split launches
// only), part_o at *off_o, part_ml at *off_ml (either pointer may be null);
// returns the total size.
constexpr size_t kDecodeFlagBytes = (size_t)kMaxMergers * kMaxSplits * 4;
size_t decode_workspace_layout(int B, int Sq, int Hq, int Hkv, int D, int capacity,
                               size_t* off_o, size_t* off_ml);
hipError_t launch_decode(const DecodeParams& p, int D, int dtype, hipStream_t stream);
// The built-in decode workspace of fa_decode_noalloc: its size, and its
// device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
hipError_t decode_scratch(void** ptr);

// ---------------------------------------------------------------------------
// Backward (dQ, dK, dV)
// ---------------------------------------------------------------------------
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;    // [B, Hq, Sq] natural-log row log-sum-exp of the forward
  float* dsum;         // [B, Hq, Sq] workspace: rowsum(dO * O)
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Sq, Sk;
  int gqa;
  float c_log2;        // |scale| * log2(e), or 1 when scale == 0
  int q_sign;          // +1, -1, or 0 (scale == 0), applied to q in the kernels
  float scale;
};

hipError_t launch_backward(const BwdParams& p, int D, int dtype, bool causal, hipStream_t stream);

}  // namespace fa
