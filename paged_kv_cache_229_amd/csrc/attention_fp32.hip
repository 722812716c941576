// Paged attention in float32 (inputs, accumulation and output), on the VALU.
//
// Same definition as the bf16 path ("Paged Attention 基础 – 原理与实现进度", §2 block-table figure and
// steps 1-5; bottom-right causal alignment for several new tokens per sequence), kept exact to float32
// for callers that need it: no reduced-precision operand anywhere.  One wave per (query token, query
// head); the wave takes 64 keys at a time, one key per lane for the dot products, then one channel per
// lane for the weighted sum of value rows, with an online softmax in between.
#include "kernels.h"

namespace pkv {
namespace {

template <int D>
__global__ void __launch_bounds__(64) attn_fp32_kernel(const AttnParams p) {
  constexpr int PER = D / 64;  // channels per lane
  __shared__ float qs[D];
  __shared__ float ps[64];

  const int tok = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int N = p.num_seqs;
  const int* qsl = p.query_start_loc;
  if (tok >= qsl[N]) return;
  int lo = 0, hi = N;  // qsl[lo] <= tok < qsl[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= tok) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = qsl[s];
  const int n = qsl[s + 1] - q0;
  const int L = p.context_lens[s];
  if (n <= 0) return;
  if (n > L || L > p.max_blocks_per_seq << p.block_size_log2) {
    // Rejected metadata (more new tokens than cached ones, or a context past the table): the row is NaN so
    // that the error shows in the result.
    float* orow = static_cast<float*>(p.out) + (static_cast<int64_t>(tok) * p.num_q_heads + h) * D;
#pragma unroll
    for (int c = 0; c < PER; ++c) orow[lane + 64 * c] = __builtin_nanf("");
    return;
  }
  const int i = tok - q0;
  const int lim = L - n + i;  // keys 0 .. lim
  const int g = h / p.group;
  const int bs_mask = (1 << p.block_size_log2) - 1;
  const int last_block = static_cast<int>(p.num_blocks - 1);
  const int* tbl = p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq;
  const float* kc = static_cast<const float*>(p.k_cache);
  const float* vc = static_cast<const float*>(p.v_cache);
  const float* qrow = static_cast<const float*>(p.q) + (static_cast<int64_t>(tok) * p.num_q_heads + h) * D;

#pragma unroll
  for (int c = 0; c < PER; ++c) qs[lane + 64 * c] = qrow[lane + 64 * c];
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;

  for (int base = 0; base <= lim; base += 64) {
    const int k = base + lane;
    float sc = -INFINITY;
    if (k <= lim) {
      const int phys = min(max(tbl[k >> p.block_size_log2], 0), last_block);
      const int64_t off = static_cast<int64_t>(phys) * p.block_stride +
                          (static_cast<int64_t>(k & bs_mask) * p.num_kv_heads + g) * D;
      const float* kr = kc + off;
      float dot = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(kr + d);
        dot = fmaf(qs[d], kv.x, dot);
        dot = fmaf(qs[d + 1], kv.y, dot);
        dot = fmaf(qs[d + 2], kv.z, dot);
        dot = fmaf(qs[d + 3], kv.w, dot);
      }
      sc = dot * p.scale;
    }
    float cm = sc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cm = fmaxf(cm, __shfl_xor(cm, o));
    const float mnew = fmaxf(m, cm);  // finite: key `base` is always visible here
    const float alpha = expf(m - mnew);
    const float pk = k <= lim ? expf(sc - mnew) : 0.f;
    float sum = pk;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    l = l * alpha + sum;
    m = mnew;
    __syncthreads();
    ps[lane] = pk;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] *= alpha;
    const int nk = min(64, lim + 1 - base);
    for (int j = 0; j < nk; ++j) {
      const int kj = base + j;
      const int phys = min(max(tbl[kj >> p.block_size_log2], 0), last_block);
      const float* vr = vc + static_cast<int64_t>(phys) * p.block_stride +
                        (static_cast<int64_t>(kj & bs_mask) * p.num_kv_heads + g) * D;
      const float w = ps[j];
#pragma unroll
      for (int c = 0; c < PER; ++c) acc[c] = fmaf(w, vr[lane + 64 * c], acc[c]);
    }
  }
  float* orow = static_cast<float*>(p.out) + (static_cast<int64_t>(tok) * p.num_q_heads + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int c = 0; c < PER; ++c) orow[lane + 64 * c] = acc[c] * inv;
}

}  // namespace

hipError_t launch_attention_fp32(const AttnParams& p, int head_dim, hipStream_t stream) {
  if (p.total_q == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(p.total_q), static_cast<unsigned>(p.num_q_heads));
  if (head_dim == 128) hipLaunchKernelGGL(attn_fp32_kernel<128>, grid, dim3(64), 0, stream, p);
  else hipLaunchKernelGGL(attn_fp32_kernel<64>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
