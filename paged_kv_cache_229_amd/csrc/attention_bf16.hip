// Paged attention, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// What is computed (per sequence s, kv head g): the sequence's K/V are the first L rows of its physical
// blocks taken in block-table order ("Paged Attention 基础 – 原理与实现进度", §2 block-table figure,
// steps 1-4); each new query token i (the last n positions) attends keys 0 .. L-n+i with
// softmax(Q K^T * scale) V (same figure, step 5; the scale is the softmax_scale of zhaoyang-star's comment
// on flash-attention issue 660 "Any plan for support paged attention?").  Several tokens per sequence
// (ADR 004 "Paged Attention Serving Integration", Consequences: prefill and decode share one call) and
// grouped kv heads (the same comment: MQA/GQA) are handled by one kernel.
//
// How (gfx950 design, not a translation of any kernel the pages name):
//  * Work item = (unit, kv head) from the device plan; a persistent grid pops items from a queue.  The
//    rows of an item are (query token, head of g's group) pairs, so all G heads sharing kv head g read
//    each K/V byte once.
//  * K/V stream through LDS 128 keys at a time.  Each of the 4 waves loads 32 keys with 16-byte lanes,
//    one uniform block-table lookup per wave-wide load (a wave-wide load never crosses a block since
//    block_size >= keys per load), so every load instruction reads whole 256-byte (D=128) rows.  The next
//    128 keys are loaded into registers while the current ones are used.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16 (keys as M, rows as N):
//    each lane then owns one row (lane % 16) for every key it holds, so row max / row sum need only two
//    cross-lane exchanges, and the probabilities already sit in the B-operand layout of O^T = V^T P^T.
//    The 32 keys of one PV step are taken in the order the S^T fragments deliver them; V is written to
//    LDS transposed in that same order, so each V^T operand is one 16-byte LDS read.
//  * Online softmax in log2 units (scale * log2 e folded into the score scale), exp2 on the VALU.
//  * Waves split a tile's rows when it has many (prefill), or the keys when it has few (decode); in the
//    latter case the waves' partial softmax states are merged through LDS at the end.
//  * A tile whose context was split into partitions writes (acc, m, l) per row; split_reduce_kernel
//    merges them.  Unsplit tiles write the normalised bf16 output directly.
#include "kernels.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzles that keep the fragment reads of both LDS tiles free of bank conflicts.
template <int D>
__device__ inline int k_swizzle(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
__device__ inline int v_swizzle(int d) { return (d & 15) ^ ((d >> 3) & 15); }

template <int D, int NTW>
struct Geo {
  static constexpr int CPK = D / 8;          // 16-byte chunks per K/V row of one head
  static constexpr int KPL = 64 / CPK;       // keys covered by one wave-wide 16-byte load
  static constexpr int NLOAD = 32 / KPL;     // such loads per lane, per tensor, per stage
  static constexpr int DC = D / 32;          // 32-channel steps of the QK contraction
  static constexpr int DT = D / 16;          // 16-channel output tiles
  static constexpr int WROWS = 16 * NTW;     // rows one wave owns
  static constexpr int RT = 4 * WROWS;       // rows per tile
  static constexpr int KBYTES = kStageKeys * D * 2;
  static constexpr int LDS = 2 * KBYTES;     // K tile + V^T tile
  static constexpr int MERGE_SLOT = DT * 256 + 32;  // floats per (wave, n-tile) in the merge buffer
  static_assert(3 * NTW * MERGE_SLOT * 4 <= LDS, "merge buffer must fit the stage buffer");
};

template <int D, int NTW>
__global__ void __launch_bounds__(kThreads) attn_bf16_kernel(const AttnParams p) {
  using T = Geo<D, NTW>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];
  __shared__ int s_item;
  unsigned char* const Ks = smem;
  unsigned char* const Vt = smem + T::KBYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Hq = p.num_q_heads;
  const int total_items = p.buf.hdr[kHdrUnits] * Hkv;
  const int P = p.buf.hdr[kHdrPartition];
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int last_block = static_cast<int>(p.num_blocks - 1);
  const __bf16* const kc = static_cast<const __bf16*>(p.k_cache);
  const __bf16* const vc = static_cast<const __bf16*>(p.v_cache);
  const __bf16* const qg = static_cast<const __bf16*>(p.q);
  __bf16* const og = static_cast<__bf16*>(p.out);
  const float sl2 = p.scale_log2;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(p.buf.hdr + kHdrQueue, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();
    if (item >= total_items) break;

    const int unit = item / Hkv;
    const int g = item - unit * Hkv;
    const int4 u = p.buf.units[unit];
    const int s = u.x, tile = u.y, part = u.z, nparts = u.w;
    const int q0 = p.query_start_loc[s];
    const int n = p.query_start_loc[s + 1] - q0;
    const int L = p.context_lens[s];
    const int row0 = tile * T::RT;
    const int rows_here = min(T::RT, n * G - row0);
    const int kmax = L - n + (row0 + rows_here - 1) / G + 1;
    const int kb = part * P;
    const int ke = min(kmax, kb + P);
    const int WR = rows_here <= T::WROWS ? 1 : (rows_here <= 2 * T::WROWS ? 2 : 4);
    const int WK = 4 / WR;
    const int wr = wave / WK;
    const int wk = wave - wr * WK;
    const int my_row0 = row0 + wr * T::WROWS;
    const int* const tbl = p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq;

    // Query fragments: B operand of S^T = K Q^T.  Lane holds row l16, channels 32*dc + 8*g4 + [0, 8).
    bf16x8 qf[NTW][T::DC];
    int lim[NTW];  // last visible key of the lane's row within this partition (-1: padding row)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int r = my_row0 + nt * 16 + l16;
      if (r < row0 + rows_here) {
        const int i = r / G;
        const int hh = r - i * G;
        const __bf16* qp = qg + ((static_cast<int64_t>(q0 + i) * Hq + g * G + hh) * D + 8 * g4);
#pragma unroll
        for (int dc = 0; dc < T::DC; ++dc) qf[nt][dc] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 32 * dc));
        lim[nt] = min(L - n + i, ke - 1);
      } else {
#pragma unroll
        for (int dc = 0; dc < T::DC; ++dc) qf[nt][dc] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        lim[nt] = -1;
      }
    }

    f32x4 acc[NTW][T::DT];
    float m[NTW], lsum[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      m[nt] = -INFINITY;
      lsum[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int nst = (ke - kb + kStageKeys - 1) / kStageKeys;
    u32x4 kreg[T::NLOAD], vreg[T::NLOAD];

    // Block-table entries for one stage: lane i (< NLOAD) fetches the physical block of this wave's
    // i-th wave-wide load.  Fetched a stage ahead so the data loads never wait on a table lookup.
    auto fetch_table = [&](int st) -> int {
      const int i = lane < T::NLOAD ? lane : T::NLOAD - 1;
      const int kk0 = min(kb + st * kStageKeys + 32 * wave + T::KPL * i, ke - 1);
      return tbl[kk0 >> bs_log2];
    };
    // Wave w loads keys [32w, 32w+32) of stage st.  Keys at or past ke are clamped to row ke-1 of the
    // same block (a wave-wide load never spans two blocks); their scores are masked, so the duplicate
    // rows carry probability 0 and rows past the context are never read.
    auto issue = [&](int st, int tv) {
      const int kbase = kb + st * kStageKeys + 32 * wave;
#pragma unroll
      for (int i = 0; i < T::NLOAD; ++i) {
        const int phys = min(max(__builtin_amdgcn_readlane(tv, i), 0), last_block);
        const int kk = min(kbase + T::KPL * i + lane / T::CPK, ke - 1);
        const int64_t e = static_cast<int64_t>(phys) * p.block_stride +
                          (static_cast<int64_t>(kk & bs_mask) * Hkv + g) * D + (lane % T::CPK) * 8;
        kreg[i] = *reinterpret_cast<const u32x4*>(kc + e);
        vreg[i] = *reinterpret_cast<const u32x4*>(vc + e);
      }
    };

    int tv = fetch_table(0);
    issue(0, tv);
    if (nst > 1) tv = fetch_table(1);
    for (int st = 0; st < nst; ++st) {
      __syncthreads();  // every wave is done reading the previous stage
#pragma unroll
      for (int i = 0; i < T::NLOAD; ++i) {
        const int key = 32 * wave + T::KPL * i + lane / T::CPK;
        const int c = lane % T::CPK;
        *reinterpret_cast<u32x4*>(Ks + key * (D * 2) + ((c ^ k_swizzle<D>(key)) << 4)) = kreg[i];
        // V^T: key kk of the 32-key step goes to position 8*((kk&15)>>2) + (kk&3) + 4*(kk>>4), which is
        // where the S^T fragments of the two 16-key halves put its probability.
        const int kk = key & 31;
        const int chunk = (wave << 2) + ((kk & 15) >> 2);
        const int jj = (kk & 3) + ((kk >> 4) << 2);
        const bf16x8 vb = as_bf16x8(vreg[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 8 * c + e;
          *reinterpret_cast<__bf16*>(Vt + d * 256 + ((chunk ^ v_swizzle(d)) << 4) + jj * 2) = vb[e];
        }
      }
      __syncthreads();
      if (st + 1 < nst) {
        issue(st + 1, tv);
        if (st + 2 < nst) tv = fetch_table(st + 2);
      }

      const int kstage = kb + st * kStageKeys;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((c % WK) != wk || kstage + 32 * c >= ke) continue;
        // S^T for keys 32c + [0, 32): two 16-key M tiles.
        f32x4 sacc[NTW][2];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) sacc[nt][0] = sacc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int key = 32 * c + 16 * mt + l16;
#pragma unroll
          for (int dc = 0; dc < T::DC; ++dc) {
            const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(
                Ks + key * (D * 2) + (((4 * dc + g4) ^ k_swizzle<D>(key)) << 4)));
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) sacc[nt][mt] = mfma16x16x32(kf, qf[nt][dc], sacc[nt][mt]);
          }
        }
        // Online softmax; lane holds keys kabs0 + 16*mt + j of row l16.
        const int kabs0 = kstage + 32 * c + 4 * g4;
        bf16x8 pf[NTW];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          float sv[8];
          float cm = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x = sacc[nt][mt][j] * sl2;
              const float y = (kabs0 + 16 * mt + j <= lim[nt]) ? x : -INFINITY;
              sv[mt * 4 + j] = y;
              cm = fmaxf(cm, y);
            }
          }
          cm = fmaxf(cm, __shfl_xor(cm, 16));
          cm = fmaxf(cm, __shfl_xor(cm, 32));
          const float mnew = fmaxf(m[nt], cm);
          const float mref = mnew == -INFINITY ? 0.f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m[nt] - mref);
          float ps = 0.f;
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8) {
            const float pv = __builtin_amdgcn_exp2f(sv[k8] - mref);
            ps += pv;
            pf[nt][k8] = static_cast<__bf16>(pv);
          }
          lsum[nt] = lsum[nt] * alpha + ps;
          m[nt] = mnew;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) acc[nt][dt] *= alpha;
        }
        // O^T += V^T P^T over the 32 keys.
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
          const int d = 16 * dt + l16;
          const bf16x8 vf = as_bf16x8(*reinterpret_cast<const u32x4*>(
              Vt + d * 256 + ((((c << 2) + g4) ^ v_swizzle(d)) << 4)));
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[nt][dt] = mfma16x16x32(vf, pf[nt], acc[nt][dt]);
        }
      }
    }

#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      lsum[nt] += __shfl_xor(lsum[nt], 16);
      lsum[nt] += __shfl_xor(lsum[nt], 32);
    }

    if (WK > 1) {  // waves that split the keys merge their softmax states through LDS
      __syncthreads();
      float* const mb = reinterpret_cast<float*>(smem);
      if (wk > 0) {
        float* const base = mb + ((wr * (WK - 1) + (wk - 1)) * NTW) * T::MERGE_SLOT;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          float* const b = base + nt * T::MERGE_SLOT;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(b + dt * 256 + lane * 4) = acc[nt][dt];
          if (g4 == 0) {
            b[T::DT * 256 + 2 * l16] = m[nt];
            b[T::DT * 256 + 2 * l16 + 1] = lsum[nt];
          }
        }
      }
      __syncthreads();
      if (wk == 0) {
        for (int o = 1; o < WK; ++o) {
          const float* const base = mb + ((wr * (WK - 1) + (o - 1)) * NTW) * T::MERGE_SLOT;
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            const float* const b = base + nt * T::MERGE_SLOT;
            const float mo = b[T::DT * 256 + 2 * l16];
            const float lo = b[T::DT * 256 + 2 * l16 + 1];
            const float mnew = fmaxf(m[nt], mo);
            const float mref = mnew == -INFINITY ? 0.f : mnew;
            const float a = __builtin_amdgcn_exp2f(m[nt] - mref);
            const float bb = __builtin_amdgcn_exp2f(mo - mref);
            lsum[nt] = lsum[nt] * a + lo * bb;
            m[nt] = mnew;
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
              acc[nt][dt] = acc[nt][dt] * a + *reinterpret_cast<const f32x4*>(b + dt * 256 + lane * 4) * bb;
          }
        }
      }
    }

    if (wk == 0) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int r = my_row0 + nt * 16 + l16;
        if (r >= row0 + rows_here) continue;
        if (nparts == 1) {
          const int i = r / G;
          const int hh = r - i * G;
          const float inv = 1.f / lsum[nt];
          __bf16* const o = og + ((static_cast<int64_t>(q0 + i) * Hq + g * G + hh) * D + 4 * g4);
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) {
            bf16x4 v;
            v[0] = static_cast<__bf16>(acc[nt][dt][0] * inv);
            v[1] = static_cast<__bf16>(acc[nt][dt][1] * inv);
            v[2] = static_cast<__bf16>(acc[nt][dt][2] * inv);
            v[3] = static_cast<__bf16>(acc[nt][dt][3] * inv);
            *reinterpret_cast<bf16x4*>(o + 16 * dt) = v;
          }
        } else {
          const int64_t prow = static_cast<int64_t>(item) * T::RT + (r - row0);
          float* const pa = p.buf.part_acc + prow * D + 4 * g4;
#pragma unroll
          for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(pa + 16 * dt) = acc[nt][dt];
          if (g4 == 0) p.buf.part_ml[prow] = make_float2(m[nt], lsum[nt]);
        }
      }
    }
  }
}

}  // namespace

int attention_bf16_wgs_per_cu(int head_dim, int tile_kind) {
  (void)tile_kind;
  // 160 KiB of LDS per CU; the stage buffer is 2 * 128 keys * head_dim * 2 bytes.
  const int lds = 2 * kStageKeys * head_dim * 2 + 64;
  int wgs = (160 * 1024) / lds;
  return wgs > 4 ? 4 : wgs;
}

hipError_t launch_attention_bf16(const AttnParams& p, int head_dim, int tile_kind, int grid,
                                 hipStream_t stream) {
  const dim3 g(static_cast<unsigned>(grid)), b(kThreads);
  if (head_dim == 128) {
    if (tile_kind == 2) hipLaunchKernelGGL((attn_bf16_kernel<128, 2>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, 1>), g, b, 0, stream, p);
  } else {
    if (tile_kind == 2) hipLaunchKernelGGL((attn_bf16_kernel<64, 2>), g, b, 0, stream, p);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, 1>), g, b, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
