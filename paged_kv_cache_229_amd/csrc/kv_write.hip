// Slot-mapping scatter of new K/V rows into the paged pool.
//
// The projections hand over this step's K/V as one contiguous blob [T][H_kv][D]; each row is copied
// into the pool row its slot names ("Any plan for support paged attention?" (flash-attention issue 660),
// tridao's comment on prefill K/V; "Paged Attention 基础 – 原理与实现进度", §3.2 status table: slot
// mapping).  slot = physical_block * block_size + offset; a negative slot writes nothing.
//
// Pure data movement: each lane moves one 16-byte chunk, consecutive lanes walk consecutive chunks of a
// row, so both the read of the blob and the write of a pool row are fully coalesced.  The copy is bit
// exact.
#include "kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads) kv_write_kernel(const KvWriteParams p) {
  const int cpr = p.chunks_per_row;
  const int per_token = 2 * cpr;  // K row chunks, then V row chunks
  const int total = p.num_tokens * per_token;
  const int64_t row_bytes = static_cast<int64_t>(cpr) * 16;
  const int bs_mask = (1 << p.block_size_log2) - 1;
  // 32-bit index: the host keeps total + one grid stride below 2^31.
  for (int idx = blockIdx.x * kThreads + threadIdx.x; idx < total; idx += gridDim.x * kThreads) {
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
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& p, hipStream_t stream) {
  if (p.num_tokens == 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(p.num_tokens) * 2 * p.chunks_per_row;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > kWriteMaxBlocks) blocks = kWriteMaxBlocks;
  hipLaunchKernelGGL(kv_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                     p);
  return hipGetLastError();
}

}  // namespace pkv
