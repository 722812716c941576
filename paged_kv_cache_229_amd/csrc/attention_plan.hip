// Device-side work plan and split-context reduction for paged attention.
//
// The host never reads context_lens or query_start_loc (that would need a device-to-host sync), so the
// decomposition into work is made here, on the device, in one small workgroup:
//
//   unit = (sequence s, row tile t, context partition p), processed once per kv head.
//
// The rows of (s, kv head g) are the pairs (query token i, query head of g's group), row = i * G + h',
// so a tile holds several tokens' worth of grouped heads and the keys it loads serve all of them.  Row
// tile t covers rows [t*RT, min(rows, (t+1)*RT)); its last token sees keys [0, kmax).  A tile whose kmax
// exceeds the partition length P is split into ceil(kmax / P) partitions; P is picked so the whole call
// has about `target_items` (unit, kv head) items, enough to fill 256 compute units several times over,
// and then lengthened until the split tiles' partial rows fit the workspace.  Units are listed longest
// first (counting sort on their 64-key stage count) so that the attention kernel's static, snake-ordered
// assignment of items to workgroups stays balanced.
//
// Each partition of a split tile leaves (acc, m, l) per row; split_reduce_kernel merges them:
//     M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (m in log2 units: the main kernel folds log2(e) into the score scale).
//
// The method's softmax is "Paged Attention 基础 – 原理与实现进度", §2 step 5; splitting the key range and
// merging the partial softmax sums gives the same result up to float32 rounding order.
#include "kernels.h"

namespace pkv {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kSortBuckets = 1024;

__device__ inline bool seq_ok(int q_lo, int q_hi, int context_len, int64_t total_q, int max_context) {
  return q_lo >= 0 && q_hi >= q_lo && q_hi <= total_q && context_len >= q_hi - q_lo &&
         context_len <= max_context;
}

// One past the last key the tile's last row may see.
__device__ inline int tile_kmax(int context_len, int n, int group, int rows, int rows_per_tile, int t) {
  const int last_row = min(rows, (t + 1) * rows_per_tile) - 1;
  return context_len - n + last_row / group + 1;
}

// Stage-count bucket of a unit, longest first.
__device__ inline int sort_bucket(int keys) {
  const int stages = (keys + kStageKeys - 1) / kStageKeys;
  return kSortBuckets - 1 - min(stages, kSortBuckets - 1);
}

// Exclusive prefix sum over the workgroup (wave scans, then a scan of the wave totals);
// *total receives the sum of all values.  `sm` holds kPlanWaves + 1 entries.
__device__ long long block_exclusive_scan(long long v, long long* total, long long* sm) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  long long incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long x = __shfl_up(incl, off);
    if (lane >= off) incl += x;
  }
  if (lane == 63) sm[wave] = incl;
  __syncthreads();
  if (t == 0) {
    long long run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const long long x = sm[w];
      sm[w] = run;
      run += x;
    }
    sm[kPlanWaves] = run;
  }
  __syncthreads();
  const long long excl = sm[wave] + incl - v;
  *total = sm[kPlanWaves];
  __syncthreads();
  return excl;
}

__device__ long long block_max(long long v, long long* sm) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<long long>(__shfl_xor(v, off)));
  if (lane == 0) sm[wave] = v;
  __syncthreads();
  long long r = sm[0];
  for (int w = 1; w < kPlanWaves; ++w) r = max(r, sm[w]);
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(const PlanParams p) {
  __shared__ long long sm[kPlanWaves + 1];
  __shared__ int bucket[kSortBuckets];
  const int t = threadIdx.x;
  const int N = p.num_seqs;
  const int per = (N + kPlanThreads - 1) / kPlanThreads;
  const int s0 = min(N, t * per);
  const int s1 = min(N, s0 + per);
  const int RT = p.rows_per_tile;
  const int G = p.group;
  const int* qsl = p.query_start_loc;

  long long work = 0, tiles = 0, bad = 0, maxk = 0;
  for (int s = s0; s < s1; ++s) {
    const int lo = qsl[s], hi = qsl[s + 1], L = p.context_lens[s];
    const int n = hi - lo;
    int nt = 0;
    if (!seq_ok(lo, hi, L, p.total_q, p.max_context)) {
      ++bad;
    } else if (n > 0) {
      const int rows = n * G;
      nt = (rows + RT - 1) / RT;
      for (int tt = 0; tt < nt; ++tt) {
        const int km = tile_kmax(L, n, G, rows, RT, tt);
        work += km;
        maxk = max(maxk, static_cast<long long>(km));
      }
    }
    p.buf.seq_tiles[s] = nt;
    tiles += nt;
  }
  long long total_work, total_tiles, total_bad;
  block_exclusive_scan(work, &total_work, sm);
  block_exclusive_scan(bad, &total_bad, sm);
  const long long tile_off = block_exclusive_scan(tiles, &total_tiles, sm);
  const long long max_kmax = block_max(maxk, sm);

  if (total_tiles > p.tile_cap) {  // inconsistent metadata: do nothing
    if (t == 0) {
      p.buf.hdr[kHdrUnits] = 0;
      p.buf.hdr[kHdrQueue] = 0;
      p.buf.hdr[kHdrPartition] = kStageKeys;
      p.buf.hdr[kHdrTiles] = 0;
      p.buf.hdr[kHdrBadSeqs] = -1;
    }
    return;
  }

  long long P;
  if (p.forced_partition > 0) {
    P = (p.forced_partition + kStageKeys - 1) / kStageKeys * kStageKeys;
  } else {
    const long long items = total_work * p.num_kv_heads;
    const long long want = (items + p.target_items - 1) / p.target_items;
    P = (want + kStageKeys - 1) / kStageKeys * kStageKeys;
    if (P < kMinPartition) P = kMinPartition;
  }

  // Partitions per tile and partial rows per split tile, for partition length P.
  long long units_total = 0, prows_total = 0, prow_off = 0;
  for (;;) {
    long long units = 0, prows = 0;
    for (int s = s0; s < s1; ++s) {
      const int nt = p.buf.seq_tiles[s];
      if (nt == 0) continue;
      const int lo = qsl[s], n = qsl[s + 1] - lo, L = p.context_lens[s];
      const int rows = n * G;
      for (int tt = 0; tt < nt; ++tt) {
        const long long np = (tile_kmax(L, n, G, rows, RT, tt) + P - 1) / P;
        units += np;
        if (np > 1) prows += np * min(RT, rows - tt * RT) * p.num_kv_heads;
      }
    }
    block_exclusive_scan(units, &units_total, sm);
    prow_off = block_exclusive_scan(prows, &prows_total, sm);
    if ((units_total <= p.unit_cap && prows_total <= p.prow_cap) || P >= max_kmax) break;
    P *= 2;
  }

  // Counting sort of the units by stage count, longest first: histogram, bucket offsets, scatter.
  for (int i = t; i < kSortBuckets; i += kPlanThreads) bucket[i] = 0;
  __syncthreads();
  for (int s = s0; s < s1; ++s) {
    const int nt = p.buf.seq_tiles[s];
    if (nt == 0) continue;
    const int lo = qsl[s], n = qsl[s + 1] - lo, L = p.context_lens[s];
    const int rows = n * G;
    for (int tt = 0; tt < nt; ++tt) {
      const int km = tile_kmax(L, n, G, rows, RT, tt);
      const int np = static_cast<int>((km + P - 1) / P);
      for (int pp = 0; pp < np; ++pp) {
        const int keys = static_cast<int>(min(static_cast<long long>(km) - pp * P, P));
        atomicAdd(&bucket[sort_bucket(keys)], 1);
      }
    }
  }
  __syncthreads();
  {
    const long long c = t < kSortBuckets ? bucket[t] : 0;
    long long dummy;
    const long long off = block_exclusive_scan(c, &dummy, sm);
    if (t < kSortBuckets) bucket[t] = static_cast<int>(off);
  }
  __syncthreads();

  long long tb = tile_off, pr = prow_off;
  for (int s = s0; s < s1; ++s) {
    p.buf.tile_base[s] = static_cast<int>(tb);
    const int nt = p.buf.seq_tiles[s];
    if (nt == 0) continue;
    const int lo = qsl[s], n = qsl[s + 1] - lo, L = p.context_lens[s];
    const int rows = n * G;
    for (int tt = 0; tt < nt; ++tt) {
      const int km = tile_kmax(L, n, G, rows, RT, tt);
      const int np = static_cast<int>((km + P - 1) / P);
      const int rows_t = min(RT, rows - tt * RT);
      const int pb0 = np > 1 ? static_cast<int>(pr) : -1;
      p.buf.tile_rec[tb] = make_int4(s, tt, pb0, np);
      ++tb;
      for (int pp = 0; pp < np; ++pp) {
        const int keys = static_cast<int>(min(static_cast<long long>(km) - pp * P, P));
        const int slot = atomicAdd(&bucket[sort_bucket(keys)], 1);
        const int pb = np > 1 ? static_cast<int>(pr + static_cast<long long>(pp) * rows_t * p.num_kv_heads)
                              : -1;
        p.buf.units[slot] = make_int4(s, tt, pp, pb);
      }
      if (np > 1) pr += static_cast<long long>(np) * rows_t * p.num_kv_heads;
    }
  }
  if (t == 0) {
    p.buf.tile_base[N] = static_cast<int>(total_tiles);
    p.buf.hdr[kHdrUnits] = static_cast<int>(units_total);
    p.buf.hdr[kHdrQueue] = 0;
    p.buf.hdr[kHdrPartition] = static_cast<int>(P);
    p.buf.hdr[kHdrTiles] = static_cast<int>(total_tiles);
    p.buf.hdr[kHdrBadSeqs] = static_cast<int>(total_bad);
  }
}

// One thread per (row, 4 channels) of a split tile: workgroup (tile, kv head, block of rows).  Tiles with
// a single partition were finished by the main kernel and are skipped.  Partition pp of a split tile with
// `rows` rows keeps kv head g's row r at partial row pb0 + pp * rows * H_kv + g * rows + r.  The
// partitions are folded in one pass with a running maximum, loads unrolled so they overlap.
template <int D>
__global__ void __launch_bounds__(kThreads) split_reduce_kernel(const AttnParams p) {
  constexpr int D4 = D / 4;
  constexpr int RPW = kThreads / D4;  // rows per workgroup
  const int tile_idx = blockIdx.x;
  const int g = blockIdx.y;
  if (tile_idx >= p.buf.hdr[kHdrTiles]) return;
  const int4 rec = p.buf.tile_rec[tile_idx];
  const int np = rec.w;
  if (np <= 1) return;
  const int s = rec.x, tile = rec.y, pb0 = rec.z;
  const int q0 = p.query_start_loc[s];
  const int n = p.query_start_loc[s + 1] - q0;
  const int G = p.group;
  const int RT = p.rows_per_tile;
  const int row0 = tile * RT;
  const int rows_here = min(RT, n * G - row0);
  const int rl = blockIdx.z * RPW + threadIdx.x / D4;
  if (rl >= rows_here) return;
  const int d0 = (threadIdx.x % D4) * 4;
  const int64_t part_stride = static_cast<int64_t>(rows_here) * p.num_kv_heads;
  const int64_t row_base = pb0 + static_cast<int64_t>(g) * rows_here + rl;
  float M = -INFINITY, den = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 4
  for (int pp = 0; pp < np; ++pp) {
    const int64_t prow = row_base + pp * part_stride;
    const float2 ml = p.buf.part_ml[prow];
    const float4 a = *reinterpret_cast<const float4*>(p.buf.part_acc + prow * D + d0);
    const float mnew = fmaxf(M, ml.x);
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float s_old = __builtin_amdgcn_exp2f(M - mref);
    const float s_new = __builtin_amdgcn_exp2f(ml.x - mref);
    den = den * s_old + ml.y * s_new;
    a0 = a0 * s_old + a.x * s_new;
    a1 = a1 * s_old + a.y * s_new;
    a2 = a2 * s_old + a.z * s_new;
    a3 = a3 * s_old + a.w * s_new;
    M = mnew;
  }
  const float inv = 1.f / den;
  const int r = row0 + rl;
  const int i = r / G;
  const int hh = r - i * G;
  __bf16* o = static_cast<__bf16*>(p.out) +
              ((static_cast<int64_t>(q0 + i) * p.num_q_heads + g * G + hh) * D + d0);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 v;
  v[0] = static_cast<__bf16>(a0 * inv);
  v[1] = static_cast<__bf16>(a1 * inv);
  v[2] = static_cast<__bf16>(a2 * inv);
  v[3] = static_cast<__bf16>(a3 * inv);
  *reinterpret_cast<bf16x4*>(o) = v;
}

}  // namespace

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const AttnParams& p, int head_dim, int tile_cap, hipStream_t stream) {
  if (tile_cap <= 0) return hipSuccess;
  const int rows_per_wg = kThreads / (head_dim / 4);
  const dim3 grid(static_cast<unsigned>(tile_cap), static_cast<unsigned>(p.num_kv_heads),
                  static_cast<unsigned>((kMaxTileRows + rows_per_wg - 1) / rows_per_wg));
  if (head_dim == 128) {
    hipLaunchKernelGGL(split_reduce_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(split_reduce_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
