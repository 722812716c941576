/*
 * paged_kv.h — C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * Two operations, as the pages state the problem:
 *
 *   paged_kv_write           scatter this step's new K/V rows into fixed-size physical blocks through a
 *                            slot mapping ("Paged Attention 基础 – 原理与实现进度", §3.2 status table:
 *                            block tables, slot mapping and context lengths as per-step metadata;
 *                            "Any plan for support paged attention?", tridao: the projections' contiguous
 *                            K/V blob is copied into blocks).
 *   paged_attention_forward  causal softmax(Q K^T * scale) V for every sequence over the K/V its block
 *                            table names ("Paged Attention 基础", §2 block-table figure and attention
 *                            steps 1-5; ADR 004 "Paged Attention Serving Integration", Decision 4: the
 *                            model writes K/V into blocks, then reads through the paged call with the
 *                            per-layer slice k_cache[i]; Consequences: prefill and decode share one
 *                            multi-token call).
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers marked (device) are HIP device addresses; (host) are host addresses.  The caller owns every
 *    buffer.  The library allocates no memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue work on it and return at once;
 *    no call synchronises the device.
 *  - The return value is a pkv_status.  A negative status means nothing was enqueued; the reason is in
 *    paged_kv_last_error().  All argument checks run on the host before any HIP call.
 *  - Element types: PKV_BF16 (bfloat16) or PKV_FP32 (float32); q, k, v, both caches and out share it.
 *  - Pool layout, per layer: block j starts at element j * block_stride of the cache base; inside a block
 *    rows are [block_size][num_kv_heads][head_dim] (token-major, heads, then channels; "Paged Attention
 *    基础", §4 comparison table, memory-layout row, with the layer axis taken out as ADR 004 slices it).
 *    block_stride = 0 means block_size * num_kv_heads * head_dim (a dense per-layer pool).  A larger
 *    stride addresses the layer-inside-block pool [num_blocks][layers][block_size][num_kv_heads][head_dim]
 *    of the same table: pass the base of layer l and block_stride = layers * block_size * H_kv * D.
 *  - A slot is a row of the pool: slot = physical_block * block_size + offset.
 *  - Supported set: head_dim in {64, 128}; block_size a power of two in [8, 256]; num_q_heads a multiple
 *    of num_kv_heads (query head h reads kv head h / (num_q_heads / num_kv_heads)); num_blocks *
 *    block_size < 2^31; every data pointer and block_stride * element size 16-byte aligned.
 *  - Contents of device metadata are trusted: a block id outside [0, num_blocks) among a sequence's first
 *    ceil(context_len / block_size) table entries, a slot outside the pool, q_len > context_len, a
 *    decreasing query_start_loc, or a slot repeated within one write are outside the supported inputs
 *    (behaviour undefined; the Python binding's validate=True mode checks them on the host first).
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes, misalignment */
  PKV_ERR_UNSUPPORTED = -2, /* outside the supported set above */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than paged_attention_workspace_size() */
  PKV_ERR_HIP = -4          /* a HIP launch or runtime call failed; message names it */
} pkv_status;

typedef enum { PKV_FP32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Version of this ABI (bumped on any signature or semantic change). */
int paged_kv_abi_version(void);

/* Message of the last failed call on the calling thread ("" after a successful call).  The string stays
 * valid until the next call into the library on that thread. */
const char* paged_kv_last_error(void);

/*
 * paged_kv_write — for every t < num_tokens with slot_mapping[t] >= 0:
 *     block = slot / block_size, offset = slot % block_size
 *     k_cache[block][offset][h][d] = k[t][h][d];  v_cache[block][offset][h][d] = v[t][h][d]
 * A negative slot writes nothing (a padding token or a prefix-cache hit).  Values are copied bit for bit.
 *
 *   k, v          (device) [num_tokens][num_kv_heads][head_dim], contiguous, read only
 *   slot_mapping  (device) [num_tokens] int32
 *   k_cache, v_cache (device) one layer's pool (layout above), written in place
 *   num_blocks    physical blocks in the pool (bounds the host checks; contents are not checked)
 *   dtype         pkv_dtype of k, v and the caches
 * num_tokens == 0 is a valid no-op.  Rows not named by a slot are never touched.
 */
int paged_kv_write(const void* k, const void* v, const int32_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
                   int64_t block_stride, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   void* stream);

/*
 * Bytes of device workspace paged_attention_forward needs for these sizes (0 for PKV_FP32, which needs
 * none).  max_q_len_hint as in paged_attention_forward.  Returns 0 and sets the last error on invalid
 * arguments.
 */
size_t paged_attention_workspace_size(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                      int32_t max_q_len_hint);

/*
 * paged_attention_forward — for each sequence s with n = query_start_loc[s+1] - query_start_loc[s] new
 * query tokens and L = context_lens[s] cached tokens (this step's tokens included, so n <= L), query i
 * (0 <= i < n) is the token at position L - n + i and attends keys 0 .. L - n + i (bottom-right causal
 * alignment):
 *     out[query_start_loc[s] + i][h] = softmax_p(scale * q[.][h] . K_s[p][h/G]) V_s[p][h/G]
 * where K_s, V_s are the first L rows of the concatenation, in table order, of the physical blocks
 * block_tables[s][0 .. ceil(L/block_size)-1].  Physical blocks may be shared between sequences (prefix
 * caching); table entries past ceil(L/block_size) and pool rows past L are never read.
 *
 *   out           (device) [total_q][num_q_heads][head_dim], written
 *   q             (device) [total_q][num_q_heads][head_dim], contiguous
 *   k_cache, v_cache (device) one layer's pool (layout above), read only
 *   block_tables  (device) [num_seqs][max_blocks_per_seq] int32, row-major
 *   context_lens  (device) [num_seqs] int32
 *   query_start_loc (device) [num_seqs + 1] int32, query_start_loc[0] == 0, query_start_loc[num_seqs]
 *                 == total_q; a sequence with n == 0 is skipped
 *   scale         multiplies Q K^T before the mask and the softmax (natural exponential); must be
 *                 finite and > 0 (a softmax temperature), else PKV_ERR_INVALID_ARG
 *   max_q_len_hint  an upper bound on n over the batch, or <= 0 if unknown (picks the row tile)
 *   workspace     (device) scratch of at least paged_attention_workspace_size() bytes, 256-byte aligned;
 *                 its contents need no initialisation and are meaningless after the call.  Calls that
 *                 share one workspace must be ordered (same stream or synchronised).
 * Accumulation is in float32; PKV_BF16 outputs are rounded to nearest even.  num_seqs == 0 or total_q
 * == 0 is a valid no-op.
 */
int paged_attention_forward(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, const int32_t* query_start_loc,
                            int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                            int32_t max_q_len_hint, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Tuning and measurement (per calling thread; they change how work is divided, never the result beyond
 * float32 summation order):
 *   partition_keys  > 0: split each tile's context into partitions of this many keys (rounded up to a
 *                   multiple of 128); 0 = chosen per call from the lengths on the device.
 *   target_items    > 0: aim the automatic choice at this many (tile, kv head, partition) work items;
 *                   0 = default.
 *   tile_kind       0 = automatic: 1 when max_q_len_hint * (num_q_heads / num_kv_heads) <= 128,
 *                   else 2; 1 = 128-row tiles (16 rows per wave); 2 = 256-row tiles (32 rows per wave).
 */
int paged_attention_set_tuning(int32_t partition_keys, int32_t target_items, int32_t tile_kind);

/*
 * When both events are non-NULL (hipEvent_t), paged_attention_forward records start_event just before
 * and stop_event just after its main attention kernel on `stream`, so the kernel's own duration can be
 * read with hipEventElapsedTime.  Pass NULL, NULL to stop.  Per calling thread.
 */
int paged_attention_set_profile_events(void* start_event, void* stop_event);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PAGED_KV_H */
