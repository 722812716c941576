// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Keys staged in LDS per stage of the attention main loop: 8 waves x 8 keys.  Partitions are multiples
// of it.
constexpr int kStageKeys = 64;
constexpr int kThreads = 256;
// paged_kv_write's grid: at most this many workgroups of kThreads lanes, striding over 16-byte chunks with a
// 32-bit index, so a call may move at most INT32_MAX - kWriteGridLanes chunks.
constexpr int kWriteMaxBlocks = 8192;
constexpr int kWriteGridLanes = kWriteMaxBlocks * kThreads;
// Row-tile kinds of the bf16 attention, chosen per sequence by the planner.  Kind 1: 128-row tiles, 8 waves
// of 16 rows (two waves per SIMD), for sequences whose q_len x group rows fit one tile (decode, speculative
// decode).  Kind 2: 256-row tiles, 8 waves of 32 rows (two waves per SIMD, 32 x 32 MFMA tiles), for long
// query chunks.
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
// The attention kernels are compiled for exactly this many waves per SIMD (amdgpu_waves_per_eu), so the
// compiler may give each wave up to 512 / kAttnWavesPerSimd registers (every build takes more than 128,
// counting accumulation registers): kAttnWavesPerSimd * 4 SIMDs / kAttnWaves workgroups fit on a CU.
constexpr int kAttnWavesPerSimd = 2;
constexpr int tile_rows_of(int kind) { return kind == 1 ? 128 : 256; }
constexpr int kMaxTileRows = tile_rows_of(2);
// Tile kind of a sequence with `rows` = q_len x group rows per kv head; `forced` (1 or 2) overrides it.
__host__ __device__ inline int tile_kind_for(int rows, int forced) {
  return forced > 0 ? forced : (rows <= tile_rows_of(1) ? 1 : 2);
}
// Upper bound on the automatic work-item target (items = units x kv heads).
constexpr int kMaxItems = 4096;
// Automatic target: 576 items (about 2.25 per workgroup of the persistent grid).  With late pieces ending
// the queue, longer bulk partitions are cheaper: the speculative batch (32 sequences over 8K-32K keys) takes
// 439-441 us at 512-576 against 449-451 us at 768; decode, the mixed step and the shared-prefix batch are
// unchanged within noise (decode's partitions are set by kSoftMinPartition).
constexpr int kDefaultItems = 576;
constexpr int kMinPartition = 256;
// With the automatic item target, partitions are lengthened up to this many keys as long as the call
// keeps PlanParams::min_items items: every item costs a pipeline fill and an epilogue, so fewer, longer
// items are faster while there are enough of them to balance the grid.
constexpr int kSoftMinPartition = 2048;
// A call is left unsplit when its unsplit items number at most one per workgroup and the longest context is at
// most kNoSplitSlackNum / kNoSplitSlackDen times the average work per workgroup.
constexpr int kNoSplitSlackNum = 13;
constexpr int kNoSplitSlackDen = 10;

// Workspace header words.
enum HeaderWord {
  kHdrUnits = 0,
  kHdrQueue = 1,
  kHdrPartition = 2,      // partition length of tiles with at most kSmallTileRows rows (before late pieces)
  kHdrTiles = 3,
  kHdrBadSeqs = 4,
  kHdrPartitionWide = 5,  // partition length of taller tiles
  // Shared-prefix pass (0 rows when off): the prefix sequence's first query token, token count, context
  // (prefix length - 1 + token count, so every prefix key is visible to every row), key end (the prefix
  // length), block-table row, partition length and partition count.
  kHdrPrefQ0 = 6,
  kHdrPrefN = 7,
  kHdrPrefL = 8,
  kHdrPrefKeys = 9,
  kHdrPrefTable = 10,
  kHdrPrefPartition = 11,
  kHdrPrefParts = 12,
  // The call shape the plan was made for (PlanParams::sig): a call that runs on an existing plan checks it.
  kHdrSig0 = 13,
  kHdrSig1 = 14,
  kHdrSig2 = 15,
};
// Tiles with more rows than this (long query chunks) are split only over long contexts: their partial
// rows cost as much to write and merge as a good share of the keys they would save reading, and there are
// already many of them.  Their partition is at least kWidePartitionMin keys.
constexpr int kSmallTileRows = 64;
constexpr int kWidePartitionMin = 4096;
// Late pieces.  In a call whose small tiles are split into long partitions (P >= kLateMinPartition keys), each
// split small tile's last kLateNum / kLateDen of keys become pieces of max(P / 4, kLatePieceMin) keys.  Sorted
// longest first, they are the queue's last items, so that the workgroups' last items are short and they
// finish closer together: the speculative batch 457 -> 442 us (at 768 items, P 7104), the mixed step's 56
// decodes alone 171.6 -> 167.8 us (P about 3900); decode (P 2048) and the whole mixed step are unchanged.
constexpr int kLateMinPartition = 2048;
constexpr int kLateNum = 3;
constexpr int kLateDen = 20;
constexpr int kLatePieceMin = 1024;

// Device work plan, all in the caller's workspace.  A unit is (sequence, row tile, context partition);
// every unit is processed once per kv head.
struct PlanBuffers {
  int* hdr;         // [16]
  int* seq_tiles;   // [num_seqs]  scratch
  int4* tile_rec;   // [tile_cap]  {sequence, tile, first partial row or -1, number of partitions}
  int2* tile_q;     // [tile_cap]  the tile's sequence's {first query token, query tokens}, as planned
  // [unit_cap][2]: {sequence, tile, first key of the partition, first partial row or -1 if unsplit}, then the
  // sequence's {first query token, query tokens, context length} and the tile kind (1 or 2) | the partition's
  // key count << 2, so that an item needs no further dependent metadata load
  int4* units;
  float2* part_ml;  // [prow_cap]  running max (log2 units) and sum per partial row
  float* part_acc;  // [prow_cap * head_dim] unnormalised partial outputs
  // [total_q] for query tokens of the shared-prefix sequences: {sequence, first partial row of its
  // shared-prefix partitions, its rows, its first query token}
  int4* tok_info;
};

// Shared-prefix pass.  Sequences [prefix_begin, prefix_end) share the blocks holding their first
// prefix_tokens tokens.  The plan adds one prefix sequence (index num_seqs in the unit records) whose
// query tokens are all of theirs and whose keys are the prefix, all visible to every row; each member's
// own units cover keys [prefix_tokens, kmax), and the prefix sequence's partitions write partial rows
// into extra partitions of the members' tiles, which split_reduce_kernel merges with the rest.
struct PrefixParams {
  int begin;
  int end;
  int tokens;  // 0 = no shared-prefix pass
};

// Partial rows of a split unit u (tile with `rows` rows): [u.w, u.w + H_kv * rows), kv head g's rows at
// u.w + g * rows.
constexpr int kPartialRowCap = 1 << 17;

struct PlanParams {
  const int* context_lens;
  const int* query_start_loc;
  int num_seqs;
  int64_t total_q;
  int group;          // num_q_heads / num_kv_heads
  int num_kv_heads;
  int tile_kind;      // 0: per sequence (tile_kind_for); 1 or 2: every sequence
  int max_context;    // max_blocks_per_seq * block_size: longer contexts are rejected on the device
  int target_items;
  int min_items;      // 0, or the item count that partitions may not be lengthened below (see kSoftMinPartition)
  int forced_partition;
  int unit_cap;
  int tile_cap;
  int prow_cap;
  PrefixParams prefix;
  PlanBuffers buf;
  int sig[3];  // call-shape signature, written to the header words kHdrSig0..2
  // Upper bound on the row tiles (the host's, from total_q, the group and the q-length hint): with more
  // sequences or tiles than one wave's 64 lanes, the planner runs on four waves, so that each of its walks
  // over the sequences and tiles is one round of memory loads rather than several.
  int64_t tiles_bound;
};
// Threads of the planner's workgroup.
inline int plan_threads(const PlanParams& p) {
  return p.num_seqs > 64 || p.tiles_bound > 64 ? 256 : 64;
}

struct AttnParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int* block_tables;
  const int* context_lens;
  const int* query_start_loc;
  int max_blocks_per_seq;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int block_size_log2;
  int tile_kind;         // as PlanParams::tile_kind (the split reduce recovers each tile's height from it)
  int64_t num_blocks;
  int64_t block_stride;  // elements
  int64_t total_q;
  float scale;           // natural-exponent scale
  float scale_log2;      // scale * log2(e)
  PlanBuffers buf;
  // Signature of the call shape (PlanParams::sig).  The kernels run the plan in the workspace only if its
  // header carries the same words; otherwise the attention kernel does nothing and split_reduce_kernel fills
  // the whole output with NaN.
  int sig[3];
};

// Words of the plan header every work item needs, read once per workgroup (scalar loads) before the first
// item: the shared-prefix sequence's key count, table row and partition length.
struct PlanWords {
  int pre_keys, pre_table, pre_P;
};

struct KvWriteParams {
  const void* k;
  const void* v;
  const int* slot_mapping;
  void* k_cache;
  void* v_cache;
  int num_tokens;
  int chunks_per_row;       // 16-byte chunks in one token row (H_kv * D * elem / 16)
  int block_size_log2;
  int64_t num_slots;        // num_blocks * block_size
  int64_t block_stride_bytes;
};

struct CopyBlocksParams {
  void* k_cache;
  void* v_cache;
  const int* src;
  const int* dst;
  int64_t num_blocks;
  int64_t chunks_per_block;    // 16-byte chunks of one block of this layer
  int64_t block_stride_bytes;
};

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyBlocksParams& p, int num_pairs, hipStream_t stream);
hipError_t launch_plan(const PlanParams& p, hipStream_t stream);
// The plan and a K/V write (w.num_tokens may be 0) in one launch.
hipError_t launch_write_plan(const PlanParams& p, const KvWriteParams& w, hipStream_t stream);
// grid = persistent workgroups; each work item runs on the tile kind its unit carries, or (narrow_only) on the
// 16-row body, for plans made with tile kind 1 throughout.
hipError_t launch_attention(const AttnParams& p, int head_dim, bool narrow_only, int grid, hipStream_t stream);
hipError_t launch_split_reduce(const AttnParams& p, int head_dim, int tile_cap, hipStream_t stream);
hipError_t launch_attention_fp32(const AttnParams& p, int head_dim, hipStream_t stream);
// Workgroups per CU the bf16 attention kernel is built for (from its LDS footprint).
int attention_wgs_per_cu(int head_dim, bool narrow_only);

}  // namespace pkv
