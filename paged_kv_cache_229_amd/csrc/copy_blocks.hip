// Whole-block copies inside a pool, the device half of copy on write: block dst[i] of both caches takes
// the contents of block src[i] (this layer's block_size x num_kv_heads x head_dim elements, bit for bit).
// A paged cache needs such copy kernels beside attention ("Any plan for support paged attention?",
// tridao and curry-zzl: the cache manager copies and updates the pages).
//
// One lane per 16-byte chunk, consecutive lanes along the block: coalesced reads and writes.  Grid: x over
// the chunks of a block, y over the pairs.  Block ids outside [0, num_blocks) are skipped.
#include "kernels.h"

namespace pkv {
namespace {

__global__ void __launch_bounds__(kThreads) copy_blocks_kernel(const CopyBlocksParams p) {
  const int pair = blockIdx.y;
  const int64_t src = p.src[pair];
  const int64_t dst = p.dst[pair];
  if (src < 0 || dst < 0 || src >= p.num_blocks || dst >= p.num_blocks) return;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (c >= p.chunks_per_block) return;
  const uint4* const ks = reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_cache) + src * p.block_stride_bytes);
  const uint4* const vs = reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_cache) + src * p.block_stride_bytes);
  uint4* const kd = reinterpret_cast<uint4*>(static_cast<char*>(p.k_cache) + dst * p.block_stride_bytes);
  uint4* const vd = reinterpret_cast<uint4*>(static_cast<char*>(p.v_cache) + dst * p.block_stride_bytes);
  kd[c] = ks[c];
  vd[c] = vs[c];
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksParams& p, int num_pairs, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>((p.chunks_per_block + kThreads - 1) / kThreads), static_cast<unsigned>(num_pairs));
  hipLaunchKernelGGL(copy_blocks_kernel, g, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
