/*
 * attn_sink.h -- C ABI of the MI355X (gfx950) grouped-query attention library
 * with per-head attention sinks.
 *
 * The operation.  Page "GPT-OSS on Day 0" (perplexity.ai), section
 * "Attention: GQA with Attention Sinks": grouped-query attention in which
 * every query head owns one pre-trained sink value that takes part in the
 * softmax.  Section "Kernels for GPT-OSS / Sink Attention" of the same page:
 * the sink is an extra term before the softmax next to the Q.K^T products; the
 * softmax runs online with a running max m and scale d; m starts from the
 * head's sink instead of -inf; the work is spread over heads and over blocks
 * of the key length, and only the first block of a split carries the sink.
 * For one query row with visible keys j < n:
 *
 *     x_j = sm_scale * (q . k_j)
 *     w   = softmax([x_0 .. x_{n-1}, s_h])     (the sink is one more logit)
 *     out = sum_{j<n} w_j v_j                  (the sink has no value row)
 *
 * The sink is in the same natural-log units as x_j and is NOT multiplied by
 * sm_scale; s_h = -inf turns it off.  Query head h reads key/value head
 * h / group_size.  Page "Fast embeddings on GPUs", section "ROSE": ragged
 * (unpadded, packed) batches for prefill and a paged key/value cache for
 * decode.
 *
 * Conventions shared by every entry point:
 *   - every pointer argument is a DEVICE pointer except where stated; the
 *     caller owns every buffer and keeps it alive until the stream's work is
 *     done; the library allocates nothing and keeps no state;
 *   - calls only enqueue work on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream): no host synchronisation and no device-to-host
 *     copy, so the calls can be captured into a HIP graph;
 *   - the returned status is host-side: argument errors are detected before
 *     anything is enqueued; ATTN_SINK_ERR_LAUNCH reports a failed launch;
 *   - element type `dtype`: ATTN_SINK_F32 or ATTN_SINK_BF16 for q, k, v and
 *     out; sinks and split partials are always fp32;
 *   - head_dim must be 64 and page_size 16 (ATTN_SINK_ERR_UNSUPPORTED
 *     otherwise); every tensor pointer must be 16-byte aligned;
 *   - device-side integer contents (cumulative offsets, lengths, page ids)
 *     are clamped, never trusted: offsets are clamped to [0, total], lengths
 *     to [0, capacity], and a page id outside [0, num_pages) makes its page
 *     skipped, so bad contents give wrong numbers, never a memory fault.
 */
#ifndef ATTN_SINK_H
#define ATTN_SINK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_SINK_OK = 0,
    ATTN_SINK_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or flag */
    ATTN_SINK_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, page size, group */
    ATTN_SINK_ERR_LAUNCH = 3,      /* the HIP runtime refused the launch */
    ATTN_SINK_ERR_TOO_LARGE = 4    /* exceeds the static scratch buffer (no-alloc call) */
} attn_sink_status;

typedef enum { ATTN_SINK_F32 = 0, ATTN_SINK_BF16 = 1 } attn_sink_dtype;

/*
 * Ragged prefill (causal or not) with sinks.
 * Passage: "GPT-OSS on Day 0", sections "Attention: GQA with Attention
 * Sinks" and "Kernels for GPT-OSS / Sink Attention"; ragged layout from
 * "Fast embeddings on GPUs", section "ROSE".
 *
 *   q     [total_q,  Hkv*G, D] dtype, token-major (sequences packed)
 *   k, v  [total_kv, Hkv,   D] dtype
 *   sinks [Hkv*G] fp32, natural-log units; -inf allowed, +inf is not
 *   cu_seqlens_q, cu_seqlens_kv [batch+1] int32 prefix offsets
 *         (cu[0] = 0, non-decreasing, cu[batch] = total)
 *   max_seqlen_q: host-side upper bound on any sequence's query count; it
 *         sizes the grid, and query rows beyond it are not written
 *   group_size G in 1..64; num_kv_heads >= 1; head_dim = 64
 *   sm_scale > 0 and finite; causal in {0, 1}: causal masks are aligned to
 *         the bottom-right corner (row i sees keys j <= i + Lkv - Lq)
 *   out   [total_q, Hkv*G, D] dtype; a row with no visible key gets 0
 * q and out may be NULL when total_q == 0, k and v when total_kv == 0.
 * Each of q, k, v must be below 4 GiB (ATTN_SINK_ERR_UNSUPPORTED otherwise).
 */
int attn_sink_prefill(const void *q, const void *k, const void *v,
                      const float *sinks, const int32_t *cu_seqlens_q,
                      const int32_t *cu_seqlens_kv, int batch, int total_q,
                      int total_kv, int max_seqlen_q, int num_kv_heads,
                      int group_size, int head_dim, float sm_scale, int causal,
                      int dtype, void *out, void *stream);

/*
 * Split-KV ragged prefill: the partial states of each query row over S
 * chunks of its sequence's key range, for attn_sink_merge to combine.  For
 * few query tiles against long key ranges this fills the GPU.
 * Passage: "GPT-OSS on Day 0", section "Kernels for GPT-OSS / Sink
 * Attention" (blocks along the key length, the sink in the first only).
 *
 *   q, k, v, sinks, cu_seqlens_*, sizes, sm_scale, causal: as in
 *         attn_sink_prefill
 *   num_splits S in 1..65536: sequence b's Lkv keys are cut into chunks of
 *         ceil(ceil(Lkv/16)/S) whole 16-key units; chunk c of a query row
 *         holds the keys of chunk c that the row can see.  Chunk 0 carries
 *         the sink: an empty chunk 0 yields (s_h, 1, 0), an empty chunk
 *         c > 0 yields (-inf, 0, 0).
 *   partial_m, partial_d [total_q, Hkv*G, S] fp32 (m in natural-log units)
 *   partial_o            [total_q, Hkv*G, S, D] fp32, unnormalised
 *         (relative to m); (m, d, o) is one of many equivalent states, since
 *         any m with d and o taken relative to it merges to the same result:
 *         m + ln d and o / d are unique.
 * attn_sink_merge(partial_m, partial_d, partial_o, total_q, Hkv*G, S, ...)
 * then yields what attn_sink_prefill writes.
 */
int attn_sink_prefill_partials(const void *q, const void *k, const void *v,
                               const float *sinks, const int32_t *cu_seqlens_q,
                               const int32_t *cu_seqlens_kv, int batch,
                               int total_q, int total_kv, int max_seqlen_q,
                               int num_kv_heads, int group_size, int head_dim,
                               float sm_scale, int causal, int dtype,
                               int num_splits, float *partial_m,
                               float *partial_d, float *partial_o,
                               void *stream);

/*
 * Paged (chunked) prefill: several new query tokens per sequence against
 * the paged key/value cache that already holds them, optionally split along
 * the key length.
 * Passage: "Fast embeddings on GPUs", section "ROSE" (prefill over a paged
 * cache); "GPT-OSS on Day 0", section "Kernels for GPT-OSS / Sink
 * Attention" (one kernel design for prefill and decode; the split rule).
 *
 *   q          [total_q, Hkv*G, D] dtype, sequences packed (cu_seqlens_q)
 *   k_cache, v_cache, page_table, num_pages, page_size: as in
 *              attn_sink_decode_paged
 *   kv_lens    [batch] int32: keys in the cache, the new tokens' included,
 *              clamped to [0, max_pages_per_seq*page_size].  The Lq queries
 *              of a sequence are its last Lq positions: with causal = 1 row
 *              i sees keys j <= i + kv_len - Lq (bottom-right alignment).
 *   sinks, group_size (1..64), head_dim, sm_scale, max_seqlen_q: as in
 *              attn_sink_prefill
 *   num_splits S == 1: writes out [total_q, Hkv*G, D] dtype; partials may
 *              be NULL.  S > 1 (up to 65536): chunks of whole pages as in
 *              attn_sink_decode_paged, clipped to each row's visible keys;
 *              writes partial_m, partial_d [total_q, Hkv*G, S] and
 *              partial_o [total_q, Hkv*G, S, D] as attn_sink_prefill_partials
 *              does; out is not touched and may be NULL.
 * q and out may be NULL when total_q == 0; the caches when num_pages == 0.
 * Caches of any size are accepted: below 4 GiB pages are read at 32-bit
 * offsets from the cache base, from 4 GiB on through 64-bit page bases.
 */
int attn_sink_prefill_paged(const void *q, const void *k_cache,
                            const void *v_cache, const int32_t *page_table,
                            const int32_t *cu_seqlens_q, const int32_t *kv_lens,
                            const float *sinks, int batch, int total_q,
                            int max_seqlen_q, int max_pages_per_seq,
                            int num_pages, int num_kv_heads, int group_size,
                            int head_dim, int page_size, float sm_scale,
                            int causal, int dtype, int num_splits,
                            float *partial_m, float *partial_d,
                            float *partial_o, void *out, void *stream);

/*
 * Paged decode (one query token per sequence) with sinks, optionally split
 * along the key length.
 * Passage: "GPT-OSS on Day 0", section "Kernels for GPT-OSS / Sink
 * Attention" (split over key blocks, sink in the first block only); paged
 * cache from "Fast embeddings on GPUs", section "ROSE".
 *
 *   q          [batch, Hkv*G, D] dtype
 *   k_cache    [num_pages, Hkv, page_size, D] dtype (token-major pages)
 *   v_cache    [num_pages, Hkv, D, page_size] dtype (dim-major pages)
 *   page_table [batch, max_pages_per_seq] int32: physical page of each
 *              logical page; entries past ceil(kv_len/page_size) are unread
 *   kv_lens    [batch] int32, clamped to [0, max_pages_per_seq*page_size]
 *   sinks      [Hkv*G] fp32
 *   group_size G in 1..16; page_size = 16; head_dim = 64
 *   num_splits S >= 1: sequence b's np = ceil(kv_len/16) pages are cut into
 *              chunks of ppc = ceil(np/S) pages; chunk c covers tokens
 *              [c*ppc*16, min((c+1)*ppc*16, kv_len)).  Chunk 0 carries the
 *              sink; an empty chunk c > 0 yields (m, d, o) = (-inf, 0, 0).
 *   S == 1:    writes out [batch, Hkv*G, D] dtype; partials may be NULL.
 *              One launch: the workgroup of a (sequence, kv head) splits
 *              its pages over 16 waves and merges their states in LDS, so
 *              no partial state is written and no merge call is needed
 *              ("CuTeDSL at Perplexity", section "Grid synchronization",
 *              weighs a merge in the same launch against a second one).
 *   k_cache and v_cache may be NULL when num_pages == 0.
 *   S  > 1:    writes partial_m, partial_d [batch, Hkv*G, S] and
 *              partial_o [batch, Hkv*G, S, D] (fp32; m in natural-log
 *              units, o unnormalised relative to m); out is not touched and
 *              may be NULL -- attn_sink_merge finishes the job.
 */
int attn_sink_decode_paged(const void *q, const void *k_cache,
                           const void *v_cache, const int32_t *page_table,
                           const int32_t *kv_lens, const float *sinks,
                           int batch, int max_pages_per_seq, int num_pages,
                           int num_kv_heads, int group_size, int head_dim,
                           int page_size, float sm_scale, int dtype,
                           int num_splits, float *partial_m, float *partial_d,
                           float *partial_o, void *out, void *stream);

/*
 * Merge of split-KV partial states into the final output; the sink is
 * already inside chunk 0's state, so it is counted exactly once.
 * Passage: "GPT-OSS on Day 0", section "Kernels for GPT-OSS / Sink
 * Attention" (blocks along the key length, sink only in the first).
 *
 *   partial_m, partial_d [batch, num_q_heads, num_splits] fp32
 *   partial_o            [batch, num_q_heads, num_splits, head_dim] fp32
 *   out [batch, num_q_heads, head_dim], out_dtype (F32 or BF16, RNE)
 *   out = (sum_c o_c e^(m_c - M)) / (sum_c d_c e^(m_c - M)), M = max_c m_c;
 *   a row whose m_c are all -inf gets 0.
 */
int attn_sink_merge(const float *partial_m, const float *partial_d,
                    const float *partial_o, int batch, int num_q_heads,
                    int num_splits, int head_dim, int out_dtype, void *out,
                    void *stream);

/*
 * Split paged decode and merge in one call that allocates nothing: for
 * callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 *   Arguments as in attn_sink_decode_paged; out [batch, Hkv*G, D] dtype is
 *   always written.  With num_splits == 1 this is attn_sink_decode_paged.
 *   With num_splits > 1 the partial states go to a file-scope device array
 *   of 16 MiB inside the library instead of caller buffers, and the merge
 *   runs on `stream` right after the decode; the result is bit for bit
 *   that of attn_sink_decode_paged + attn_sink_merge.
 *   Limit: 4 * batch * Hkv*G * num_splits * (D + 2) bytes (plus alignment)
 *   must fit in 16 MiB, else ATTN_SINK_ERR_TOO_LARGE and nothing is
 *   enqueued.
 *   Each GPU holds one copy of the array for the life of the process, and
 *   every call on that GPU uses it: calls that may overlap on one GPU (on
 *   different streams, or from different threads) race and must be
 *   serialised by the caller.  Nothing in the array needs clearing: every
 *   call writes every partial state it later reads.  The first call on a
 *   device resolves the array's device address (hipGetSymbolAddress); no
 *   call allocates, frees or synchronises.
 */
int attn_sink_decode_paged_static(const void *q, const void *k_cache,
                                  const void *v_cache,
                                  const int32_t *page_table,
                                  const int32_t *kv_lens, const float *sinks,
                                  int batch, int max_pages_per_seq,
                                  int num_pages, int num_kv_heads,
                                  int group_size, int head_dim, int page_size,
                                  float sm_scale, int dtype, int num_splits,
                                  void *out, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *attn_sink_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SINK_H */
