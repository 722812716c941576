// Paged attention, bf16 in / fp32 accumulate: the persistent kernel that runs every work item of a call.
//
// What is computed, per sequence and kv head, is "Paged Attention 基础 – 原理与实现进度", §2 (the
// block-table walk of steps 1-4 and the causal softmax(Q K^T * scale) V of step 5), for any number of new
// tokens per sequence (ADR 004 "Paged Attention Serving Integration", Consequences: prefill and decode share
// one call).  The planner (attention_plan.hip) lists units (sequence, row tile, context partition) longest
// first; every unit is one work item per kv head.  Each unit carries the row-tile kind the planner chose
// for its sequence:
//   kind 1, 128-row tiles on 16-row waves (attention_narrow.h): sequences whose q_len x group rows fit one
//          such tile -- decode, speculative decode, the decodes of a chunked-prefill batch;
//   kind 2, 256-row tiles on 32-row waves, 32 x 32 MFMA (attention_wide.h): long query chunks and the
//          shared-prefix sequence.
// One grid serves both, so a batch that mixes prefill chunks and decodes runs each on its own kind within a
// single launch.  Both bodies use the same LDS ring of 64-key stages and the same eight waves; the
// workgroup's LDS is sized for the larger of the two.  When the caller's q-length bound shows that every
// sequence fits a 128-row tile, the host plans 128-row tiles throughout and launches the build that holds
// only the 16-row body.
#include "attention_narrow.h"
#include "attention_wide.h"

namespace pkv {
namespace {

template <int D>
struct AttnSmem {
  static constexpr int NARROW = Geo<D, 1>::SMEM;
  static constexpr int WIDE = WideGeo<D, kWideHalves>::SMEM;
  static constexpr int BYTES = NARROW > WIDE ? NARROW : WIDE;
  static_assert(WideGeo<D, kWideHalves>::THREADS == kAttnThreads, "both bodies run on one workgroup shape");
};

// NARROW_ONLY: every unit runs the 16-row body (the host plans 128-row tiles for every sequence).  Built
// separately because the 16-row body alone needs far fewer registers (about 160) than the two bodies
// together, and decode-like batches, which only ever need it, run measurably faster without the other.
template <int D, bool NARROW_ONLY>
__global__ void __launch_bounds__(kAttnThreads)
__attribute__((amdgpu_waves_per_eu(kAttnWavesPerSimd, kAttnWavesPerSimd)))
attn_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16)))
  unsigned char smem[NARROW_ONLY ? Geo<D, 1>::SMEM : AttnSmem<D>::BYTES];
  __shared__ int s_item;
  const int tid = threadIdx.x;
  const int Hkv = p.num_kv_heads;
  // The plan header through scalar loads, once: the planner wrote it before this launch and nothing here
  // writes these words (only the queue counter beside them changes, through vector atomics).  Read per item
  // instead, they would be vector loads, and each item would wait a memory round trip before its copies.
  const CONST_AS int* const hdr = (const CONST_AS int*)p.buf.hdr;
  // A plan made for another call shape is not run (split_reduce_kernel then fills the output with NaN).
  const bool plan_ok = hdr[kHdrSig0] == p.sig[0] && hdr[kHdrSig1] == p.sig[1] && hdr[kHdrSig2] == p.sig[2];
  const int total_items = plan_ok ? hdr[kHdrUnits] * Hkv : 0;
  const PlanWords pw{hdr[kHdrPrefKeys], hdr[kHdrPrefTable], hdr[kHdrPrefPartition]};
  // Workgroup w starts on item w without a claim (the first claims of all workgroups at once would queue on
  // one counter); each later item is claimed while the current one finishes (after its last stage), so the
  // atomic's latency hides behind the epilogue, and the queue hands out gridDim.x, gridDim.x + 1, ...
  int next_item = 0;
  for (int item = blockIdx.x;;) {
    if (item >= total_items) break;
    const int unit = item / Hkv;
    const int g = item - unit * Hkv;
    if (NARROW_ONLY) {
      narrow_item<D>(p, pw, smem, unit, g, next_item);
    } else {
      // The unit's row-tile kind (low bits of word 7 of its record), through a scalar load.
      const int kind = ((const CONST_AS int*)p.buf.units)[8 * unit + 7] & 3;
      if (kind == 2) wide_item<D, kWideHalves>(p, pw, smem, unit, g, next_item);
      else narrow_item<D>(p, pw, smem, unit, g, next_item);
    }
    if (tid == 0) s_item = next_item;
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();
  }
}

}  // namespace

int attention_wgs_per_cu(int head_dim, bool narrow_only) {
  // Registers: kAttnWavesPerSimd waves per SIMD.  LDS: 160 KiB per CU; a workgroup holds the 4-stage K/V
  // ring (reused for the merges) plus a word.  (The runtime's occupancy query counts only the
  // architectural registers, and overstates this for builds that also use accumulation registers.)
  constexpr int by_regs = kAttnWavesPerSimd * 4 / kAttnWaves;
  static_assert(by_regs >= 1, "a workgroup fits a CU");
  const int smem = narrow_only ? (head_dim == 128 ? Geo<128, 1>::SMEM : Geo<64, 1>::SMEM)
                               : (head_dim == 128 ? AttnSmem<128>::BYTES : AttnSmem<64>::BYTES);
  const int by_lds = (160 * 1024) / (smem + 64);
  const int wgs = by_lds < by_regs ? by_lds : by_regs;
  return wgs < 1 ? 1 : wgs;
}

hipError_t launch_attention(const AttnParams& p, int head_dim, bool narrow_only, int grid, hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(kAttnThreads);
  if (narrow_only) {
    if (head_dim == 128) hipLaunchKernelGGL((attn_kernel<128, true>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((attn_kernel<64, true>), g, b, 0, stream, p);
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((attn_kernel<128, false>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((attn_kernel<64, false>), g, b, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
