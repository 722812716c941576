/*
 * paged_kv.h — C ABI of the MI355X (gfx950) paged KV-cache library.
 *
 * Two operations, as the pages state the problem, and the cache manager they need:
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
 *   paged_attention_forward_prefix  the same result when a range of sequences shares its first blocks
 *                            (the pages' prefix caching, §1 problem 3 and the §2 figure where two
 *                            sequences start with one physical block): the shared keys are attended once
 *                            for all sharers' query rows together.
 *   pkv_cm_* / paged_kv_copy_blocks  host cache manager (block allocator, block tables, slot mapping,
 *                            shared blocks with copy on write) and its device block copy (declared below).
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers marked (device) are HIP device addresses; (host) are host addresses.  The caller owns every
 *    buffer.  The library allocates no memory and keeps no pointer after a call returns (its one buffer
 *    of its own is paged_attention_forward_noalloc's fixed scratch, below).
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
 *    ceil(context_len / block_size) table entries, a slot outside the pool, a decreasing
 *    query_start_loc, or a slot repeated within one write are outside the supported inputs (behaviour
 *    undefined; the Python binding's validate=True mode checks them on the host first).  A sequence the
 *    attention call rejects on the device -- q_len > context_len, a negative context_len, or context_len >
 *    max_blocks_per_seq * block_size -- reads nothing and gets NaN in every output row, when its own
 *    query_start_loc range lies inside [0, total_q]; the other sequences are computed as usual.
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
  PKV_ERR_HIP = -4,         /* a HIP launch or runtime call failed; message names it */
  PKV_ERR_NO_BLOCKS = -5    /* the cache manager has too few free blocks; nothing changed */
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
 *   block_tables  (device) [num_seqs][max_blocks_per_seq] int32, row-major; max_blocks_per_seq >= 1 and
 *                 max_blocks_per_seq * block_size < 2^29 (else PKV_ERR_INVALID_ARG / PKV_ERR_UNSUPPORTED)
 *   context_lens  (device) [num_seqs] int32
 *   query_start_loc (device) [num_seqs + 1] int32, query_start_loc[0] == 0, query_start_loc[num_seqs]
 *                 == total_q; a sequence with n == 0 is skipped
 *   scale         multiplies Q K^T before the mask and the softmax (natural exponential); must be
 *                 finite and > 0 (a softmax temperature), else PKV_ERR_INVALID_ARG
 *   max_q_len_hint  an upper bound on n over the batch, or <= 0 if unknown (picks the row tile)
 *   workspace     (device) scratch of at least paged_attention_workspace_size() bytes, 256-byte aligned;
 *                 its contents need no initialisation; after the call it holds the call's work plan, which
 *                 paged_attention_run may reuse.  Calls that share one workspace must be ordered (same
 *                 stream or synchronised).
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
 * paged_attention_write_forward — paged_kv_write(k_new, v_new, slot_mapping, num_tokens into k_cache,
 * v_cache) followed by paged_attention_forward(...) on the same pool: the same results (pools and output
 * bit-identical to the two calls), one launch fewer.  A decode step writes the step's new K/V rows and then
 * attends over them (flash-attention issue 660, the prefill/decode discussion; "Paged Attention 基础 –
 * 原理与实现进度", §3.2 status table: slot mapping); the work planner reads only the metadata, so it runs in
 * the same launch as the write (workgroup 0 plans, the others write) instead of after it.
 *   k_new, v_new, slot_mapping, num_tokens  as paged_kv_write's k, v, slot_mapping, num_tokens (num_tokens
 *                 == 0 writes nothing); the pool arguments (k_cache, v_cache, num_blocks, block_size,
 *                 block_stride, num_kv_heads, head_dim, dtype) serve both.
 *   everything else as paged_attention_forward.
 * Errors: those of paged_kv_write, then those of paged_attention_forward; on any error nothing is launched.
 * PKV_FP32 (no plan) and a call with no query rows write with a launch of their own.
 */
int paged_attention_write_forward(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                  int64_t num_tokens, void* out, const void* q, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                                  int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, int64_t block_stride, float scale,
                                  int32_t dtype, int32_t max_q_len_hint, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * paged_attention_run — paged_attention_forward on the work plan an earlier call left in `workspace`,
 * without planning again.  Every layer of a model step calls attention with its own k_cache[i], v_cache[i]
 * but the same block tables and lengths (ADR 004 "Paged Attention Serving Integration", Decision 4), and
 * the plan -- how the batch is cut into work items and partial rows -- depends on nothing else: call
 * paged_attention_forward for the step's first layer and paged_attention_run for the others, with the same
 * workspace, the same block_tables / context_lens / query_start_loc (contents included), the same sizes,
 * max_q_len_hint and tuning; out, q, k_cache, v_cache and scale may differ.  The result is then identical
 * to paged_attention_forward's with the same arguments.
 *  - Same arguments and errors as paged_attention_forward.
 *  - The plan records the call's shape (sizes, row-tile kind, workspace layout).  If the workspace holds no
 *    plan for this shape, nothing is computed and every output element is NaN.  The metadata's contents
 *    are not checked: with contents other than the plan's, the output is undefined, but every access stays
 *    inside the call's buffers and the workspace.
 *  - Calls sharing the workspace must be ordered (same stream or synchronised); the plan is the one the
 *    last paged_attention_forward or paged_attention_forward_prefix call on the workspace made.
 * PKV_FP32 has no plan and runs as paged_attention_forward.
 */
int paged_attention_run(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                        const int32_t* query_start_loc, int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                        int64_t block_stride, float scale, int32_t dtype, int32_t max_q_len_hint, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Size in bytes of the library's own device scratch used by paged_attention_forward_noalloc (32 MiB per
 * GPU).
 */
#define PKV_NOALLOC_SCRATCH_BYTES 33554432

/*
 * paged_attention_forward_noalloc — paged_attention_forward (same arguments and result, up to float32
 * summation order) without a workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation.  It calls no allocating
 * routine.  Its scratch (the per-call work plan and split-context partial rows) is a fixed buffer of
 * PKV_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, that each GPU holds from the library's first
 * use on it until the process ends.
 *
 *  - Size limit: the call's work records (a few hundred bytes per sequence and per 128 query rows of a
 *    kv head, see paged_attention_workspace_size) must fit the scratch with room to spare, else
 *    PKV_ERR_UNSUPPORTED and nothing is enqueued; what remains holds up to 131072 partial rows (about
 *    63000 at head_dim 128), fewer than with a full workspace, so long contexts may be split into fewer,
 *    longer partitions.
 *  - All calls on one GPU share that GPU's scratch, whatever the stream: calls that overlap on one GPU
 *    race (and give undefined output); order them on one stream or synchronise between them.  Each call
 *    initialises what it reads, so the previous call's leftovers never matter.
 *  - The first call on a device looks up the scratch's device address (hipGetSymbolAddress) with that
 *    device current; a failure there returns PKV_ERR_HIP.
 * PKV_FP32 needs no scratch and runs as paged_attention_forward.
 */
int paged_attention_forward_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, const int32_t* query_start_loc,
                                    int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                                    int32_t max_q_len_hint, void* stream);

/*
 * Bytes of device workspace paged_attention_forward_prefix needs (0 for PKV_FP32).  Returns 0 and sets
 * the last error on invalid arguments.
 */
size_t paged_attention_prefix_workspace_size(int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, int32_t dtype);

/*
 * paged_attention_forward_prefix — the result of paged_attention_forward (same arguments, same output up
 * to float32 summation order), for a batch where sequences prefix_begin .. prefix_end - 1 share the
 * physical blocks that hold their first prefix_tokens tokens (prefix caching, "Paged Attention 基础 –
 * 原理与实现进度", §1 problem 3 and the §2 figure).  Instead of every sharer reading the shared blocks
 * again, one pass attends all sharers' query rows to the shared keys at once (a dense contraction on the
 * matrix cores); each sharer's own pass covers only its keys after the prefix, and the two partial
 * softmax states (max, sum, unnormalised output) merge exactly as the split-context partitions do.
 *
 *   prefix_begin, prefix_end  0 <= prefix_begin <= prefix_end <= num_seqs (else PKV_ERR_INVALID_ARG);
 *                 an empty range or prefix_tokens == 0 runs the ordinary computation.
 *   prefix_tokens >= 0, a multiple of block_size and <= max_blocks_per_seq * block_size (else
 *                 PKV_ERR_INVALID_ARG).  The caller promises that block_tables[s][0 .. prefix_tokens /
 *                 block_size - 1] is the same for every s in the range (the sharing itself; the library
 *                 does not compare tables, and a violation gives undefined output, like other metadata
 *                 contents).  The device checks the rest and, if any sharer has a new token inside the
 *                 prefix (context_lens[s] - n < prefix_tokens), holds more rows than one 256-row tile
 *                 (n * num_q_heads / num_kv_heads > 256), or the extra work would not fit the workspace,
 *                 runs the ordinary computation instead.
 *   workspace     at least paged_attention_prefix_workspace_size() bytes, 256-byte aligned.
 * Everything else as paged_attention_forward (which picks the row tile from max_q_len_hint; this call
 * always uses 256-row tiles).  PKV_FP32 runs the ordinary fp32 computation.
 */
int paged_attention_forward_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int64_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, int64_t block_stride, float scale, int32_t dtype,
                                   int32_t prefix_begin, int32_t prefix_end, int32_t prefix_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_run_prefix — paged_attention_forward_prefix on the work plan an earlier
 * paged_attention_forward_prefix call left in `workspace`, without planning again: for the layers after the
 * first of a model step whose batch shares a prefix (the same sharing in every layer, since every layer's
 * pool uses the same block tables; ADR 004 "Paged Attention Serving Integration", Decision 4).  Call
 * paged_attention_forward_prefix for the step's first layer and this for the others, with the same
 * workspace, metadata (contents included), sizes, prefix_begin / prefix_end / prefix_tokens and tuning; out,
 * q, k_cache, v_cache and scale may differ.  The result is then identical to paged_attention_forward_prefix's
 * with the same arguments.
 *  - Same arguments and errors as paged_attention_forward_prefix.
 *  - If the workspace holds no plan for this shape and prefix range (none, or one that paged_attention_forward
 *    or another range made), nothing is computed and every output element is NaN; otherwise as
 *    paged_attention_run.
 * PKV_FP32 has no plan and runs as paged_attention_forward.
 */
int paged_attention_run_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc, int32_t num_seqs,
                               int64_t total_q, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, int64_t block_stride, float scale,
                               int32_t dtype, int32_t prefix_begin, int32_t prefix_end, int32_t prefix_tokens,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_copy_blocks — for i < num_pairs: block dst_blocks[i] of both caches takes the contents of
 * block src_blocks[i] (this layer's block_size * num_kv_heads * head_dim elements, bit for bit).  The
 * device half of copy on write: run it with the (src, dst) pair pkv_cm_append reports, before writing the
 * new slots.  Pool geometry and checks as in paged_kv_write.
 *
 *   src_blocks, dst_blocks (device) [num_pairs] int32; ids outside [0, num_blocks) are skipped.  Pairs
 *                 run concurrently: no dst may be another pair's src or dst (the manager's pairs never are).
 *   num_pairs     0 is a no-op; at most 65535 (PKV_ERR_UNSUPPORTED above).
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, int64_t num_blocks, int32_t block_size,
                         int64_t block_stride, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         const int32_t* src_blocks, const int32_t* dst_blocks, int32_t num_pairs,
                         void* stream);

/*
 * Cache manager (host memory and host calls only; no HIP call, no device pointer).  It owns the mapping
 * from sequences to physical blocks: a block allocator, one block table per sequence id, the slot mapping
 * of new tokens, and blocks shared by several sequences ("Paged Attention 基础", §1 problems 1-3 and
 * §3.1 A: block allocator, block table, slot mapping; §2 figure: sequences A [7, 3] and B [7, 9] share
 * block 7; ADR 004, Decision 5 and Consequences: one update call for fresh and growing sequences,
 * free(seq_id), add_prefix / try_get_prefix_blocks).
 *
 *  - Allocation takes the lowest-numbered free block.  A block is shared by reference counting: each
 *    sequence and each registered prefix listing it holds one reference; it is free again at zero.
 *  - Every call either completes or changes nothing (PKV_ERR_NO_BLOCKS, PKV_ERR_INVALID_ARG).
 *  - A manager is not thread-safe; it is owned by its creator and released with pkv_cm_destroy.
 */
typedef struct pkv_cache_manager pkv_cache_manager;

/* A manager over num_blocks blocks of block_size tokens, all free.  NULL (last error set) on
 * num_blocks < 1, block_size < 1, or num_blocks * block_size >= 2^31. */
pkv_cache_manager* pkv_cm_create(int32_t num_blocks, int32_t block_size);
void pkv_cm_destroy(pkv_cache_manager* manager);

/* Free blocks; -1 for a NULL manager. */
int32_t pkv_cm_num_free(const pkv_cache_manager* manager);

/* Tokens held by seq_id; -1 if unknown. */
int32_t pkv_cm_seq_len(const pkv_cache_manager* manager, int64_t seq_id);

/*
 * Append num_tokens tokens at the end of seq_id (created if new): the update call of a prefill or decode
 * step.  Takes the blocks the new length needs; slots_out (host, [num_tokens]) receives the pool row of
 * each new position in order (block_table[pos / block_size] * block_size + pos % block_size), ready for
 * paged_kv_write.  If the last block is partly filled and shared, it is first replaced by a fresh copy:
 * cow_out (host, [2]) receives (src, dst) — copy block src to dst with paged_kv_copy_blocks before
 * writing — else (-1, -1).  PKV_ERR_NO_BLOCKS when the free blocks do not suffice.
 */
int pkv_cm_append(pkv_cache_manager* manager, int64_t seq_id, int32_t num_tokens, int32_t* slots_out,
                  int32_t* cow_out);

/* Release seq_id: each of its blocks loses one reference. */
int pkv_cm_free(pkv_cache_manager* manager, int64_t seq_id);

/* child (new) starts as parent's copy, sharing every block (one more reference each). */
int pkv_cm_fork(pkv_cache_manager* manager, int64_t parent, int64_t child);

/* Register the blocks holding the first num_tokens tokens of seq_id (1 <= num_tokens <= its length)
 * under key; the registry keeps one reference, so they outlive the sequence.  The key must be new. */
int pkv_cm_add_prefix(pkv_cache_manager* manager, uint64_t key, int64_t seq_id, int32_t num_tokens);

/* A new seq_id starts with the prefix registered under key (shared blocks); *tokens_out = its length,
 * or 0 (and nothing created) when the key is unknown. */
int pkv_cm_attach_prefix(pkv_cache_manager* manager, uint64_t key, int64_t seq_id, int32_t* tokens_out);

/* Release the registry's references of key. */
int pkv_cm_drop_prefix(pkv_cache_manager* manager, uint64_t key);

/*
 * Per-step metadata for a batch: block_tables_out (host, [num_seqs][max_blocks_per_seq], row-major)
 * receives each sequence's blocks padded with -1, context_lens_out (host, [num_seqs]) its length.
 * Fails, writing nothing, if a sequence is unknown or holds more than max_blocks_per_seq blocks.
 */
int pkv_cm_build_tables(const pkv_cache_manager* manager, const int64_t* seq_ids, int32_t num_seqs,
                        int32_t max_blocks_per_seq, int32_t* block_tables_out, int32_t* context_lens_out);

/*
 * Tuning and measurement (per calling thread; they change how work is divided, never the result beyond
 * float32 summation order):
 *   partition_keys  > 0: split each tile's context into partitions of this many keys (rounded up to a
 *                   multiple of 64); 0 = chosen per call from the lengths on the device.
 *   target_items    > 0: aim the automatic choice at this many (tile, kv head, partition) work items;
 *                   0 = default (about 576 items, with partitions of at least 2048 keys as long as the
 *                   call keeps two items per workgroup of the attention grid; a call with partitions of
 *                   2048 keys or more ends each split tile on shorter late pieces).
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
