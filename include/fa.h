/*
 * fa.h -- C ABI of the MI355X (gfx950) dense flash-attention forward library.
 *
 * Two operations, both from the pages:
 *
 *  fa_fwd     Dense attention forward ("prefill"):
 *               O = softmax(scale * Q K^T + mask) V
 *             computed tile by tile with a running max / running sum, so the
 *             Sq x Sk score matrix never reaches memory.  Forward only,
 *             bf16 or fp16 storage, head_dim 64 or 128, MHA or GQA.
 *             Page "Dense flash-attention prefill (gfx950 / MI355X)", intro
 *             and "Baked-in levers"; tessera PR page, flash_attn forward
 *             commit (S = scale*Q@K^T, causal/ragged mask, online softmax,
 *             O += P@V).  Causal masking is bottom-right aligned: key j is
 *             admissible for query i iff j <= i + (Sk - Sq) (decode PR page,
 *             PR description: "bottom-right causal").  A query row with no
 *             admissible key (causal with Sq > Sk, or Sk = 0) gets O = 0.
 *
 *  fa_decode  The Sq = 1 case over a contiguous token-major KV cache whose
 *             valid length lives on the device and is never read by the host
 *             (decode PR page, PR description: "device INT32 valid-length
 *             scalar", "contiguous token-major KV").  Cache entries at or past
 *             the valid length are never read, so NaN or garbage there cannot
 *             reach O (decode PR page, review: unused V-cache NaNs must not
 *             contaminate the output).  Long caches are split into runs whose
 *             partial results are merged by merger workgroups of the same
 *             launch (split-KV, which the decode PR page names as follow-up
 *             work); one launch per call.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are device pointers owned by the caller, contiguous,
 *    16-byte aligned, in the element type given by `dtype`.  The library never
 *    allocates, frees or synchronises, and never reads device memory on the
 *    host.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously on it; the call returns once enqueued.
 *  - Every argument check runs before any HIP call, so a rejected call has no
 *    side effect.  Launch failures are reported as FA_ERR_HIP.
 *  - `o` must not overlap any input.
 *  - Accumulation is fp32; P is rounded to the input type before the P*V
 *    product; O is rounded to the output type with round-to-nearest-even.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_BF16 = 0, /* bfloat16 storage */
  FA_FP16 = 1  /* IEEE binary16 storage */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* negative size, Hq % Hkv != 0, capacity < 1, size overflow */
  FA_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, dtype not bf16/fp16 */
  FA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  FA_ERR_SCALE = 5,       /* scale is NaN or infinite */
  FA_ERR_WORKSPACE = 6,   /* workspace NULL, misaligned or smaller than required */
  FA_ERR_HIP = 7,         /* the HIP runtime refused the launch */
  FA_ERR_ALIAS = 8        /* the output overlaps an input */
} fa_status_t;

/*
 * fa_fwd -- dense attention forward.
 *   q : [B, Hq,  Sq, D]   queries
 *   k : [B, Hkv, Sk, D]   keys
 *   v : [B, Hkv, Sk, D]   values
 *   o : [B, Hq,  Sq, D]   output (written)
 * Query head h reads kv head h / (Hq / Hkv) (contiguous GQA groups).
 * causal != 0 selects the bottom-right aligned causal mask.
 * scale multiplies the q.k dot products (1/sqrt(D) is the usual value).
 * B, Sq or Sk may be 0: B = 0 or Sq = 0 enqueues nothing; Sk = 0 writes O = 0.
 * One (batch, kv head) of K or V must fit 32-bit byte offsets:
 * Sk * D * 2 <= INT_MAX, else FA_ERR_SHAPE.
 * When the shape has fewer work items than the GPU has CUs, the keys of each
 * item are split over several workgroups (fa_fwd_plan reports split_tiles);
 * their partial results meet in a workspace.  With at least 12 items per CU,
 * the persistent workgroups take items from a work queue whose counters live
 * in the same workspace.  The library allocates it once per (device,
 * stream) on the first such call, 34.6 MB held until the process ends, so
 * that first call is not capturable in a HIP graph.  Every launch leaves its
 * counters at zero; calls on one stream reuse the workspace in order; a graph
 * captured with such a launch keeps using the workspace of the stream it was
 * captured on.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o,
                   int B, int Hq, int Hkv, int Sq, int Sk, int D,
                   int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_lse -- fa_fwd that also writes the natural-log row log-sum-exp
 *   lse : [B, Hq, Sq] float32, lse[b,h,i] = log sum_{j admissible} exp(scale*q_i.k_j),
 *         -inf for a row with no admissible key.
 * The per-row running max and running sum of the online softmax give it for
 * free; it is the quantity a split or cross-device merge of partial outputs
 * needs (decode PR page lists LSE as a follow-up; the tessera backward uses
 * it as L).
 */
fa_status_t fa_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int Hq, int Hkv, int Sq, int Sk, int D,
                       int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_varlen -- fa_fwd over a batch of sequences of different lengths,
 * packed along the token dimension (the packed varlen path, cu_seqlens_q/kv,
 * that the page "Dense flash-attention prefill (gfx950 / MI355X)" names
 * under TODO / follow-ups).
 *   q   : [total_q, Hq,  D]  queries of all sequences, back to back
 *   k   : [total_k, Hkv, D]  keys
 *   v   : [total_k, Hkv, D]  values
 *   o   : [total_q, Hq,  D]  output (written for the rows of every sequence)
 *   lse : NULL, or [Hq, total_q] float32: natural-log row log-sum-exp as in
 *         fa_fwd_lse (-inf for a row with no admissible key)
 *   cu_seqlens_q, cu_seqlens_k : device int32[B + 1]; sequence b owns query
 *         rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows
 *         [cu_seqlens_k[b], cu_seqlens_k[b+1]).  They are read on the device
 *         only.  Offsets are clamped to [0, total] and lengths to
 *         max_seqlen_q / max_seqlen_k, so malformed offsets give unspecified
 *         values but never an access outside the tensors.  Rows that belong
 *         to no sequence are not written.
 *   max_seqlen_q, max_seqlen_k : upper bounds of the sequence lengths; the
 *         launch is planned for a dense batch of B sequences of these lengths
 *         and work items past the end of a shorter sequence exit at once.
 * Within sequence b attention is that of fa_fwd with Sq = its query length
 * and Sk = its key length (bottom-right causal mask when causal != 0).
 * Limits: max_seqlen_k * Hkv * D * 2 <= INT_MAX, else FA_ERR_SHAPE.
 */
fa_status_t fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int B, int Hq, int Hkv, int total_q, int total_k,
                          int max_seqlen_q, int max_seqlen_k, int D,
                          int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_plan -- the launch plan fa_fwd would use for a shape (host only, no
 * HIP call).  Exposed so the schedule can be inspected and tested.
 */
typedef struct {
  int block_m;          /* query rows per work item */
  int block_n;          /* keys per KV tile */
  int work_items;       /* ceil(Sq / block_m) * Hq * B */
  int grid;             /* workgroups launched */
  int persistent;       /* 1 = grid-stride persistent launch */
  int hkv_major;        /* 1 = work items ordered kv-head-major, 0 = query-block-major */
  long long kv_tiles;   /* KV tiles streamed, summed over work items */
  long long masked_tiles; /* of those, tiles that need the mask */
  int xcd_map;          /* 1 = each XCD's workgroups take the items of the
                           (batch, kv head) units u with u % 8 == XCD, so a kv
                           head's K/V is fetched into one XCD's L2 only; chosen
                           for query-block-major persistent launches whose unit
                           count B * Hkv is a multiple of 8 */
  int split_tiles;      /* 0, or: the key tiles of each work item are cut into
                           ceil(tiles / split_tiles) parts of near-equal size,
                           one workgroup each (grid = number of parts), merged
                           in the launch; chosen for non-persistent launches
                           whose longest item can be cut to at most
                           tiles - 2 tiles per part within one workgroup per CU */
  int queue;            /* 1 = persistent launch whose workgroups take the items
                           after their first from a work queue (an atomic
                           ticket counter in the library's per-stream
                           workspace), so the list is dealt to whichever
                           workgroup is free; 0 = static round-robin.  Chosen
                           for persistent launches of 12 or more items per
                           workgroup, with the query-block-major order */
} fa_fwd_plan_t;

fa_status_t fa_fwd_plan(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                        fa_fwd_plan_t* plan);

/*
 * fa_fwd_planned -- fa_fwd (and fa_fwd_lse when lse is not NULL) with the
 * launch schedule chosen by the caller: `plan` holds the choices in its
 * persistent, hkv_major, xcd_map, queue (each 0 or 1) and split_tiles (>= 0)
 * fields; the other fields are ignored.  Without a split the schedule only decides
 * which workgroup computes which work item and in what order, so every such
 * choice gives bitwise the same result.  A split (split_tiles > 0) sums each
 * item in parts and merges them: the result then differs from the unsplit one
 * by rounding only, and is the same bits call after call for one split_tiles.
 * It exists to compare schedules.  Choices that do not fit the sizes -- a
 * field out of range, xcd_map without a persistent grid of one workgroup per
 * CU (256) and B * Hkv a multiple of 8, queue without a persistent grid, a
 * split together with persistent, hkv_major, xcd_map or queue, or a split of
 * more than 256 parts -- give FA_ERR_SHAPE.  Other arguments and errors as fa_fwd / fa_fwd_lse.
 */
fa_status_t fa_fwd_planned(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal,
                           float scale, int dtype, const fa_fwd_plan_t* plan, void* stream);

/*
 * fa_decode_workspace_bytes -- bytes of workspace fa_decode needs for these
 * sizes (0 on invalid sizes).  The workspace holds the fp32 partial results
 * of the split runs and one run-complete flag per (run, merger workgroup).
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int capacity);

/*
 * fa_decode -- single-token (Sq = 1) attention over a KV cache.
 *   q         : [B, Hq, D]                 query of the new token
 *   kcache    : [B, capacity, Hkv, D]      token-major key cache
 *   vcache    : [B, capacity, Hkv, D]      token-major value cache
 *   valid_len : int32[B] on the device; batch b attends to tokens
 *               [0, clamp(valid_len[b], 0, capacity)).  Never read on the host.
 *   o         : [B, Hq, D]                 output (written); 0 when the length is 0
 *   causal    : accepted for symmetry with fa_fwd; at Sq = 1 the bottom-right
 *               causal mask admits every valid token, so it changes nothing.
 *   workspace : device memory of at least fa_decode_workspace_bytes(...) bytes,
 *               256-byte aligned, zero-filled by the caller once when it is
 *               allocated.  Every call leaves its flags at zero again, so it
 *               can be reused call after call on one stream, also for other
 *               shapes whose size it covers.  Two calls in flight at once must
 *               not share a workspace.
 * Tokens at or past the valid length are never loaded.  The split plan is
 * made on the device from the valid length: a short length is handled by one
 * workgroup that writes O itself.  Repeated calls give identical bits.
 * One batch's cache must fit 32-bit byte offsets: capacity * Hkv * D * 2 <=
 * INT_MAX, else FA_ERR_SHAPE.
 */
fa_status_t fa_decode(const void* q, const void* kcache, const void* vcache,
                      const int32_t* valid_len, int capacity, void* o,
                      int B, int Hq, int Hkv, int D, int causal, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_noalloc -- fa_decode with no workspace argument and no allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *   Arguments, layouts, semantics and errors as fa_decode.  The workspace is
 *   a built-in device array of 8 MiB per GPU (every single-token decode
 *   shape needs at most about 4.2 MiB), held until the process ends; sizes
 *   that would need more are rejected with FA_ERR_WORKSPACE before any HIP
 *   call.  The first call on a device looks up the array's device address
 *   once (hipGetSymbolAddress); no call allocates or frees anything.
 *   The array starts zeroed and every completed call leaves its flags at zero
 *   again.  All calls on one GPU share the array: two calls that overlap in
 *   time on one GPU (different streams, or different host threads) race and
 *   give undefined results -- order them on one stream.
 */
fa_status_t fa_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                              const int32_t* valid_len, int capacity, void* o,
                              int B, int Hq, int Hkv, int D, int causal, float scale, int dtype,
                              void* stream);

/*
 * fa_decode_paged -- fa_decode over a paged KV cache (the decode PR page
 * names paged KV as follow-up work beyond its identity page table).
 *   k_pages, v_pages : [num_pages, page_size, Hkv, D] pool of pages, each
 *               page token-major like the contiguous cache
 *   page_table: device int32 [B, pages_per_seq]; token t of batch b is row
 *               t % page_size of page page_table[b][t / page_size].  Read on
 *               the device only, and only for pages holding valid tokens;
 *               entries are clamped to [0, num_pages), so a malformed table
 *               gives unspecified values but no access outside the pool.
 *   valid_len : device int32[B], clamped to [0, pages_per_seq * page_size]
 *   page_size : a multiple of 32 (a 32-token step never straddles pages)
 *   workspace : as for fa_decode, sized by fa_decode_workspace_bytes with
 *               capacity = pages_per_seq * page_size
 * Limits: pages_per_seq * page_size <= 2^21 tokens and
 * page_size * Hkv * D * 2 <= INT_MAX, else FA_ERR_SHAPE; the pool itself may
 * exceed 2 GiB.  Other arguments, errors and semantics as fa_decode; with an
 * identity page table over a pool that is the contiguous cache of batch 0
 * (B = 1) the result is bitwise that of fa_decode.
 */
fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* page_table, const int32_t* valid_len,
                            int page_size, int pages_per_seq, int num_pages, void* o,
                            int B, int Hq, int Hkv, int D, int causal, float scale, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-token (speculative) decode: Sq query tokens per sequence in one call
 * (the decode PR page leaves Sq > 1 decode as follow-up work).
 *   q, o : [B, Sq, Hq, D]; query token t of batch b sits at position
 *          L - Sq + t of its sequence (L = clamp(valid_len[b], 0, capacity)),
 *          i.e. the tokens being decoded are the last Sq valid ones.
 *   causal != 0: token t sees keys j <= L - Sq + t (bottom-right causal, the
 *          prefill mask with Sk = L); causal == 0: every j < L.  A token with
 *          no key to see (L - Sq + t < 0) gets O = 0.
 *   1 <= Sq <= 32.  Sq = 1 is fa_decode / fa_decode_paged exactly.
 *   workspace : at least fa_decode_multi_workspace_bytes(B, Sq, Hq, Hkv, D,
 *          capacity) bytes (capacity = pages_per_seq * page_size if paged),
 *          otherwise as for fa_decode.
 * The other arguments, limits and errors are those of fa_decode and
 * fa_decode_paged.
 */
size_t fa_decode_multi_workspace_bytes(int B, int Sq, int Hq, int Hkv, int D, int capacity);

fa_status_t fa_decode_multi(const void* q, const void* kcache, const void* vcache,
                            const int32_t* valid_len, int capacity, void* o,
                            int B, int Sq, int Hq, int Hkv, int D, int causal, float scale,
                            int dtype, void* workspace, size_t workspace_bytes, void* stream);

fa_status_t fa_decode_paged_multi(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* page_table, const int32_t* valid_len,
                                  int page_size, int pages_per_seq, int num_pages, void* o,
                                  int B, int Sq, int Hq, int Hkv, int D, int causal,
                                  float scale, int dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Backward pass: gradients of O = softmax(scale Q K^T + mask) V (tessera PR
 * page, flash_attn backward commit: the FA-2 backward as a pre-pass for
 * D = rowsum(O * dO), a dK/dV pass per key tile and a dQ pass per query tile).
 *   q, k, v   : the forward's inputs, layouts as fa_fwd
 *   o         : [B, Hq, Sq, D] the forward's output
 *   dout      : [B, Hq, Sq, D] gradient of the loss with respect to o
 *   lse       : [B, Hq, Sq] float32, the forward's row log-sum-exp (fa_fwd_lse)
 *   dq        : [B, Hq, Sq, D]  written
 *   dk, dv    : [B, Hkv, Sk, D] written; the query heads of a GQA group add
 *               into their kv head
 *   workspace : device memory of at least fa_bwd_workspace_bytes(B, Hq, Sq)
 *               bytes, 256-byte aligned (holds the row sums D; no zeroing needed)
 * causal, scale, dtype as fa_fwd.  Sq = 0 gives dK = dV = 0; Sk = 0 gives dQ = 0.
 * Errors: as fa_fwd, FA_ERR_WORKSPACE for a missing or small workspace, and
 * FA_ERR_ALIAS when an output overlaps an input, the workspace or another
 * output.  Runs as three kernels on `stream`; allocates nothing.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq);

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, float scale,
                   int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
