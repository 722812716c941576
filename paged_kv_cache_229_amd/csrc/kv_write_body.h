// The slot-mapping scatter's per-chunk work, shared by the write kernel and the launch that plans and writes
// in one (attention_plan.hip).
//
// This step's K/V arrive as one contiguous blob [T][H_kv][D]; each row is copied into the pool row its slot
// names ("Any plan for support paged attention?" (flash-attention issue 660), tridao's comment on prefill
// K/V; "Paged Attention 基础 – 原理与实现进度", §3.2 status table: slot mapping).
// slot = physical_block * block_size + offset; a negative slot, or one past the pool, writes nothing.
#pragma once

#include "kernels.h"

namespace pkv {

// Moves 16-byte chunks first, first + stride, ... of the call: chunk idx is token idx / (2 cpr), its K row's
// chunks then its V row's.  Consecutive lanes take consecutive chunks of a row, so both the read of the blob
// and the write of a pool row are coalesced; the copy is bit exact.  32-bit index: the host keeps the chunk
// count plus one stride below 2^31.
__device__ inline void kv_write_chunks(const KvWriteParams& p, int first, int stride) {
  typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
  const int cpr = p.chunks_per_row;
  const int per_token = 2 * cpr;  // K row chunks, then V row chunks
  const int total = p.num_tokens * per_token;
  const int64_t row_bytes = static_cast<int64_t>(cpr) * 16;
  const int bs_mask = (1 << p.block_size_log2) - 1;
  for (int idx = first; idx < total; idx += stride) {
    const int t = idx / per_token;
    const int rem = idx - t * per_token;
    const bool is_v = rem >= cpr;
    const int c = is_v ? rem - cpr : rem;
    const int slot = p.slot_mapping[t];
    if (slot < 0 || slot >= p.num_slots) continue;
    const int64_t blk = slot >> p.block_size_log2;
    const int64_t off = slot & bs_mask;
    const char* src = static_cast<const char*>(is_v ? p.v : p.k) + t * row_bytes + c * 16;
    char* dst = static_cast<char*>(is_v ? p.v_cache : p.k_cache) + blk * p.block_stride_bytes +
                off * row_bytes + c * 16;
    *reinterpret_cast<u32x4w*>(dst) = *reinterpret_cast<const u32x4w*>(src);
  }
}

}  // namespace pkv
