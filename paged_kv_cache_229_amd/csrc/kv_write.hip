// Slot-mapping scatter of new K/V rows into the paged pool (the per-chunk work is kv_write_chunks in
// kv_write_body.h).  Pure data movement, one lane per 16-byte chunk, bit exact.
#include "kv_write_body.h"

namespace pkv {
namespace {

__global__ void __launch_bounds__(kThreads) kv_write_kernel(const KvWriteParams p) {
  kv_write_chunks(p, blockIdx.x * kThreads + threadIdx.x, gridDim.x * kThreads);
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
