// Device-side work plan and split-context reduction for paged attention.
//
// The host never reads context_lens or query_start_loc (that would need a device-to-host sync), so the
// decomposition into work is made here, on the device, by one workgroup (one wave up to 64 sequences and tiles):
//
//   unit = (sequence s, row tile t, context partition p), processed once per kv head.
//
// The rows of (s, kv head g) are the pairs (query token i, query head of g's group), row = i * G + h',
// so a tile holds several tokens' worth of grouped heads and the keys it loads serve all of them.  A
// sequence's tiles are 128 rows high when its rows fit one such tile, else 256 (tile_kind_for; the unit
// record carries the kind, which picks the item body of the attention kernel).  Row tile t covers rows
// [t*RT, min(rows, (t+1)*RT)); its last token sees keys [0, kmax).  A tile whose kmax
// exceeds its partition length is split into ceil(kmax / length) partitions.  Tiles of at most
// kSmallTileRows rows (decode-like work) use P, picked so the whole call has about `target_items`
// (unit, kv head) items, enough to fill 256 compute units several times over, but no shorter than
// kSoftMinPartition keys while the call keeps two items per workgroup of the persistent grid; taller tiles
// (long query chunks) use max(P, kWidePartitionMin).  P is then lengthened until the split tiles' partial
// rows fit the workspace.  Units are listed longest first (counting sort on their 64-key stage count), the
// order in which the attention kernel's workgroups claim them from one queue, so that the short ones fill
// the end.
//
// Each partition of a split tile leaves (acc, m, l) per row; split_reduce_kernel merges them:
//     M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// (m in log2 units: the main kernel folds log2(e) into the score scale).
//
// The method's softmax is "Paged Attention 基础 – 原理与实现进度", §2 step 5; splitting the key range and
// merging the partial softmax sums gives the same result up to float32 rounding order.
#include "fastdiv.h"
#include "kernels.h"
#include "kv_write_body.h"

namespace pkv {
namespace {

// One workgroup plans the whole call (one wave for up to 64 sequences and tiles, four waves beyond: each walk
// over the sequences or tiles is then one round of memory loads per thread): every step is
// a per-thread loop over sequences s = tid, tid + THREADS, ... followed by a reduction or scan (DPP
// inside each wave, then the wave totals through LDS).  Each sequence's
// (new tokens, context, tiles) is read from global memory once and kept in LDS (for the first
// kSeqCache sequences; later ones are read again), and all arithmetic is 32-bit: 64-bit division is a
// long software routine on this GPU.
constexpr int kSortBuckets = 1024;
constexpr int kSeqCache = 2048;

__device__ inline bool seq_ok(int q_lo, int q_hi, int context_len, int64_t total_q, int max_context) {
  return q_lo >= 0 && q_hi >= q_lo && q_hi <= total_q && context_len >= q_hi - q_lo &&
         context_len <= max_context;
}

// One past the last key tile t's last row may see (rows are token * G + head, so the row's token is
// row / G).  When G divides the tile height every tile but the last ends on a token boundary and no
// division is needed; the last tile's last row is the last token, which sees all L keys.
struct TileGeom {
  int G, RT, tokens_per_tile;  // tokens_per_tile = RT / G when G divides RT, else 0
  int kind, rt_log2;
  __device__ int tiles(int rows) const { return (rows + RT - 1) >> rt_log2; }
  __device__ int kmax(int L, int n, int rows, int t) const {
    const int end = (t + 1) * RT;
    if (end >= rows) return L;
    if (tokens_per_tile > 0) return L - n + (t + 1) * tokens_per_tile;
    return L - n + (end - 1) / G + 1;
  }
};

// A tile's own partitions (keys [k0, km)): nb partitions of len keys over [k0, kbulk), then late pieces of at
// most `piece` keys over [kbulk, km); n in all.  len, piece and kbulk - k0 are multiples of kStageKeys, so every
// partition starts on a stage boundary counted from k0.
struct OwnParts {
  int k0, km, len, nb, kbulk, piece, n;
  __device__ void range(int pp, int& kb, int& kl) const {
    if (pp < nb) {
      kb = k0 + pp * len;
      kl = min(len, kbulk - kb);
    } else {
      kb = kbulk + (pp - nb) * piece;
      kl = min(piece, km - kb);
    }
  }
};

// Stage-count bucket of a unit, longest first.  A stage of a 256-row tile (32-row waves, bound by the matrix
// cores) takes about twice as long as a stage of a 128-row tile (16-row waves, bound by the copies), so the
// former count double (weight 2): units are ordered by estimated time, not key count.
__device__ inline int sort_bucket(int keys, int weight) {
  const int stages = weight * ((keys + kStageKeys - 1) / kStageKeys);
  return kSortBuckets - 1 - min(stages, kSortBuckets - 1);
}
__device__ inline int kind_weight(int kind) { return kind == 2 ? 2 : 1; }

// Wave-wide inclusive prefix sum with DPP lane moves (no LDS traffic): running sums within each row of 16
// lanes by shifts of 1, 2, 4 and 8, then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then lane 31's running sum into rows 2 and 3 (row_bcast:31).  Lanes whose source is outside the row or
// masked off add 0.
__device__ inline int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return v;
}

__device__ inline int wave_sum(int v) { return __builtin_amdgcn_readlane(wave_inclusive_scan(v), 63); }

__device__ inline int wave_max(int v) {
  // Values are >= 0, so lanes without a source may contribute 0.
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// Workgroup-wide versions (every thread calls them; `red` holds kPlanWaves ints of LDS).
template <int WAVES>
__device__ inline int block_sum(int v, int* red) {
  const int w = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) t += red[i];
  __syncthreads();
  return t;
}

template <int WAVES>
__device__ inline int block_max(int v, int* red) {
  const int w = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) t = max(t, red[i]);
  __syncthreads();
  return t;
}

template <int WAVES>
__device__ inline int block_exclusive_scan(int v, int* total, int* red) {
  const int incl = wave_inclusive_scan(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) red[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) {
    const int x = red[i];
    before += i < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// The planner: one workgroup of THREADS threads builds the call's work plan in the workspace.
template <int THREADS>
__device__ __forceinline__ void plan_body(const PlanParams& p) {
  constexpr int kPlanThreads = THREADS;
  constexpr int kPlanWaves = THREADS / 64;
  constexpr int kBucketsPerThread = kSortBuckets / THREADS;
  // Sorting scratch: kSortBuckets counters for longest-first order; to interleave the two tile classes, also
  // per-class stage counts (twice: one copy hands out the ranks of the key histogram, the other those of the
  // scatter) and work offsets.
  __shared__ int sortbuf[7 * kSortBuckets];
  int* const bucket = sortbuf;
  __shared__ int4 seqc[kSeqCache];  // (n, L, tiles, first query token) per sequence
  const int tid = threadIdx.x;
  __shared__ int red[kPlanWaves];
  const int N = p.num_seqs;
  const int G = p.group;
  const int Hkv = p.num_kv_heads;
  const int* const qsl = p.query_start_loc;
  const int* const ctx = p.context_lens;
  // Tile geometry of each kind; a sequence takes the one tile_kind_for gives its rows.
  const TileGeom geo1{G, tile_rows_of(1), tile_rows_of(1) % G == 0 ? tile_rows_of(1) / G : 0, 1, 7};
  const TileGeom geo2{G, tile_rows_of(2), tile_rows_of(2) % G == 0 ? tile_rows_of(2) / G : 0, 2, 8};
  static_assert(tile_rows_of(1) == 1 << 7 && tile_rows_of(2) == 1 << 8, "tile heights");
  auto geom = [&](int rows) -> TileGeom { return tile_kind_for(rows, p.tile_kind) == 1 ? geo1 : geo2; };
  // Per-thread partial counts only ever meet caps below 2^17; saturating them at 2^22 keeps every
  // workgroup sum (256 threads) in 32 bits.
  constexpr int kSat = 1 << 22;

  // (n, L, tiles) of sequence s; tiles is 0 for empty or invalid sequences.
  auto seq = [&](int s, int& n, int& L) -> int {
    if (s < kSeqCache) {
      const int4 c = seqc[s];
      n = c.x;
      L = c.y;
      return c.z;
    }
    const int lo = qsl[s];
    n = qsl[s + 1] - lo;
    L = ctx[s];
    return p.buf.seq_tiles[s];
  };

  // Stage (first query, one past the last query, context) of the cached sequences in LDS; unrolled so
  // that many loads are in flight at once.
#pragma unroll 8
  for (int s = tid; s < min(N, kSeqCache); s += kPlanThreads) seqc[s] = make_int4(qsl[s], qsl[s + 1], ctx[s], 0);

  // Tiles per sequence, key work (in 64-key stages), longest context.
  int work = 0, bad = 0, maxk = 0;
  for (int s = tid; s < N; s += kPlanThreads) {
    int lo, hi, L;
    if (s < kSeqCache) {
      const int4 c = seqc[s];
      lo = c.x;
      hi = c.y;
      L = c.z;
    } else {
      lo = qsl[s];
      hi = qsl[s + 1];
      L = ctx[s];
    }
    const int n = hi - lo;
    int nt = 0;
    if (!seq_ok(lo, hi, L, p.total_q, p.max_context)) {
      ++bad;
    } else if (n > 0) {
      const int rows = n * G;
      const TileGeom geo = geom(rows);
      nt = geo.tiles(rows);
      for (int t = 0; t < nt; ++t) work = min(work + (geo.kmax(L, n, rows, t) + kStageKeys - 1) / kStageKeys, kSat);
      maxk = max(maxk, L);  // the last tile's last row sees all L keys
    }
    if (s < kSeqCache) seqc[s] = make_int4(n, L, nt, lo);
    else p.buf.seq_tiles[s] = nt;
  }
  const long long total_work = static_cast<long long>(block_sum<kPlanWaves>(work, red)) * kStageKeys;
  const int total_bad = block_sum<kPlanWaves>(bad, red);
  const int max_kmax = block_max<kPlanWaves>(maxk, red);

  // First tile record of every sequence, in sequence order.
  int total_tiles = 0;
  for (int base = 0; base < N; base += kPlanThreads) {
    const int s = base + tid;
    int n, L;
    const int nt = s < N ? seq(s, n, L) : 0;
    int sum;
    const int first = total_tiles + block_exclusive_scan<kPlanWaves>(nt, &sum, red);
    // Tile list: record (sequence, tile) of every tile once, so that the passes below run one thread per
    // tile rather than one per sequence (a long chunk has many tiles).  The records are completed (first
    // partial row, partitions) once P is known.
    if (first + nt <= p.tile_cap)
      for (int t = 0; t < nt; ++t) p.buf.tile_rec[first + t] = make_int4(s, t, -1, 0);
    total_tiles += sum;
    if (total_tiles > p.tile_cap) break;
  }
  __syncthreads();  // (also a workgroup-scope fence: the tile records are visible to every thread)

  if (total_tiles > p.tile_cap) {  // inconsistent metadata: do nothing
    if (tid == 0) {
      p.buf.hdr[kHdrUnits] = 0;
      p.buf.hdr[kHdrQueue] = 0;
      p.buf.hdr[kHdrPartition] = kStageKeys;
      p.buf.hdr[kHdrPartitionWide] = kStageKeys;
      p.buf.hdr[kHdrTiles] = 0;
      p.buf.hdr[kHdrBadSeqs] = -1;
      p.buf.hdr[kHdrPrefN] = 0;
      p.buf.hdr[kHdrSig0] = p.sig[0];
      p.buf.hdr[kHdrSig1] = p.sig[1];
      p.buf.hdr[kHdrSig2] = p.sig[2];
    }
    return;
  }

  // Partition length of small tiles: about target_items items in all, a multiple of the stage, at least
  // kMinPartition (kSoftMinPartition while that leaves min_items items), and never longer than needed for
  // the longest context.  Taller tiles use Pw >= P.
  const int pmax = max(kMinPartition, (max_kmax + kStageKeys - 1) / kStageKeys * kStageKeys);
  int P;
  if (p.forced_partition > 0) {
    P = min((p.forced_partition + kStageKeys - 1) / kStageKeys * kStageKeys, pmax);
  } else {
    const long long items = total_work * Hkv;
    const long long want = (items + p.target_items - 1) / p.target_items;
    P = static_cast<int>(min(static_cast<long long>(pmax), (want + kStageKeys - 1) / kStageKeys * kStageKeys));
    P = max(P, kMinPartition);
    if (p.min_items > 0) {
      const long long soft = min(static_cast<long long>(kSoftMinPartition), items / p.min_items / kStageKeys * kStageKeys);
      P = max(P, static_cast<int>(min(soft, static_cast<long long>(pmax))));
      // No split at all when the unsplit tiles already give each workgroup of the grid (min_items / 2) at
      // most one item and the longest is within kNoSplitSlack of the per-workgroup average: the makespan is
      // then that longest item, while splitting would add fills, partial rows and their merge to every
      // workgroup (measured: 256 MQA decodes over 2K-3K keys take 52 us unsplit vs 60 us split).  Spread
      // lengths or more items than workgroups are better balanced by partitions (decode batches, long
      // speculative contexts).  Not used with the shared-prefix pass, which partitions its own way.
      const long long grid = p.min_items / 2;
      if (p.prefix.tokens <= 0 && static_cast<long long>(total_tiles) * Hkv <= grid &&
          static_cast<long long>(max_kmax) * grid * kNoSplitSlackDen <= kNoSplitSlackNum * total_work * Hkv)
        P = pmax;
    }
  }
  auto wide_len = [&](int P_) { return p.forced_partition > 0 ? P_ : min(max(P_, kWidePartitionMin), pmax); };

  // Shared-prefix pass: on only when every member sequence is valid, fits one tile and has all of its new
  // tokens after the prefix, and when the extra units and partial rows fit; otherwise the ordinary plan.
  const int pb = p.prefix.begin, pe = p.prefix.end, ptok = p.prefix.tokens;
  bool pref = ptok > 0 && pb >= 0 && pe > pb && pe <= N;
  int vq0 = 0, vn = 0, tiles_v = 0, npv = 0, Pv = 0;
  if (pref) {
    int viol = 0;
    for (int s = pb + tid; s < pe; s += kPlanThreads) {
      int n, L;
      const int nt = seq(s, n, L);
      if (n < 0 || (n > 0 && (nt != 1 || L - n < ptok))) ++viol;
    }
    viol = block_sum<kPlanWaves>(viol, red);
    vq0 = qsl[pb];
    vn = qsl[pe] - vq0;
    pref = viol == 0 && vn > 0;
    if (pref) {
      tiles_v = geo2.tiles(vn * G);  // the prefix sequence always runs on 256-row tiles
      if (p.forced_partition > 0) {
        Pv = P;
      } else {
        // About one prefix item per two workgroups of the attention grid (min_items / 2 workgroups; a stage of
        // these 256-row tiles takes about twice as long as one of the members' 128-row tiles), partitions of
        // at least 256 keys.  Measured on 256 members over a 2048-key prefix (32 tiles): 3-4 partitions per
        // tile give 36-37 us of kernel time, 8 partitions 42 us (and twice the partial rows), 2 partitions 46 us.
        const int pre_items = p.min_items > 0 ? max(1, p.min_items / 4) : 128;
        const int want = min(max(1, (pre_items + tiles_v * Hkv - 1) / (tiles_v * Hkv)), max(1, ptok / 256));
        Pv = ((ptok + want - 1) / want + kStageKeys - 1) / kStageKeys * kStageKeys;
      }
      npv = (ptok + Pv - 1) / Pv;
      const long long min_prows = static_cast<long long>(1 + npv) * vn * G * Hkv;
      pref = static_cast<long long>(tiles_v) * npv <= p.unit_cap - p.tile_cap && min_prows <= p.prow_cap;
    }
    if (!pref) vn = tiles_v = npv = 0;
  }
  const int units_v = tiles_v * npv;

  // Partitions of tile record rec for partition lengths (P_, Pw_).  Its own key range starts at k0 (after the
  // prefix for members of the shared-prefix pass); returns all partitions of the tile including the prefix
  // ones.  Also gives the tile's rows and kind weight.  Late pieces (kLateMinPartition): a split small tile
  // of a call with long partitions ends on pieces of max(P_ / 4, kLatePieceMin) keys covering the last
  // kLateNum / kLateDen of its keys, so that the queue ends on short items.
  const bool late_on = p.forced_partition <= 0 && !pref;
  auto tile_parts = [&](const int4 rec, int P_, int Pw_, const FastDiv& dp, const FastDiv& dw, OwnParts& op,
                        int& rows_t, int& wt) -> int {
    int n, L;
    const int s = rec.x, t = rec.y;
    seq(s, n, L);
    const int rows = n * G;
    const TileGeom geo = geom(rows);
    wt = kind_weight(geo.kind);
    rows_t = min(geo.RT, rows - t * geo.RT);
    op.km = geo.kmax(L, n, rows, t);
    const bool member = pref && s >= pb && s < pe;
    op.k0 = member ? ptok : 0;
    const bool small = rows_t <= kSmallTileRows;
    op.len = small ? P_ : Pw_;
    const int keys = op.km - op.k0;
    op.kbulk = op.km;
    op.piece = op.len;
    if (late_on && small && P_ >= kLateMinPartition && keys > P_) {
      op.piece = max(P_ / 4 / kStageKeys * kStageKeys, kLatePieceMin);
      // Every partition starts a whole number of stages after k0: the copies resolve one block-table entry per
      // group of keys, which must not straddle a block.
      const int late = static_cast<int>(static_cast<long long>(keys) * kLateNum / kLateDen);
      op.kbulk = op.k0 + (keys - late) / kStageKeys * kStageKeys;
    }
    op.nb = small ? dp.ceil_div(op.kbulk - op.k0) : dw.ceil_div(op.kbulk - op.k0);
    op.n = op.nb + (op.km - op.kbulk + op.piece - 1) / op.piece;
    return op.n + (member ? npv : 0);
  };

  // Lengthen P until the units and the split tiles' partial rows fit the workspace.
  int units_total = 0, units_wide = 0;  // units in all, and units of 256-row tiles (the prefix sequence's included)
  for (;;) {
    const int Pw = wide_len(P);
    const FastDiv divp(P), divw(Pw);
    int units = 0, prows = 0, wide = 0;
    for (int tau = tid; tau < total_tiles; tau += kPlanThreads) {
      OwnParts op;
      int rows_t, wt;
      const int np = tile_parts(p.buf.tile_rec[tau], P, Pw, divp, divw, op, rows_t, wt);
      units = min(units + op.n, kSat);
      if (wt == 2) wide = min(wide + op.n, kSat);
      if (np > 1) prows = min(prows + min(np * rows_t, kSat) * Hkv, kSat);
    }
    units_total = block_sum<kPlanWaves>(units, red) + units_v;
    units_wide = block_sum<kPlanWaves>(wide, red) + units_v;
    const int prows_total = block_sum<kPlanWaves>(prows, red);
    if ((units_total <= p.unit_cap && prows_total <= p.prow_cap) || P >= max_kmax) break;
    P = P > pmax / 2 ? pmax : 2 * P;
  }

  const int Pw = wide_len(P);
  const FastDiv divp(P), divw(Pw);
  // Complete the tile records: first partial row of every split tile, in tile (= sequence) order.
  {
    int run = 0;
    for (int base = 0; base < total_tiles; base += kPlanThreads) {
      const int tau = base + tid;
      int pr = 0, np = 0;
      int4 rec = make_int4(0, 0, -1, 0);
      if (tau < total_tiles) {
        rec = p.buf.tile_rec[tau];
        OwnParts op;
        int rows_t, wt;
        np = tile_parts(rec, P, Pw, divp, divw, op, rows_t, wt);
        if (np > 1) pr = np * rows_t * Hkv;
      }
      int sum;
      const int first = run + block_exclusive_scan<kPlanWaves>(pr, &sum, red);
      if (tau < total_tiles) {
        p.buf.tile_rec[tau] = make_int4(rec.x, rec.y, np > 1 ? first : -1, np);
        // The sequence's query range as planned, for split_reduce_kernel (which then never reads the call's
        // query_start_loc, so a later call on this plan stays inside the planned partial rows).
        int n, L;
        seq(rec.x, n, L);
        p.buf.tile_q[tau] = make_int2(rec.x < kSeqCache ? seqc[rec.x].w : qsl[rec.x], n);
      }
      run += sum;
    }
  }

  // Order of the units.  Longest first on the stage count weighted by kind_weight (a counting sort), unless the
  // call has both tile classes with at least one item per workgroup of the grid each: units of 128-row tiles
  // (the 16-row body, paced by the K/V copies) and of 256-row tiles (the 32-row body, bound by the matrix
  // cores) are then interleaved -- each unit's key is the fraction of its class's work (longest first within
  // the class) that precedes it, quantised to kSortBuckets steps, and the units are counting-sorted on it --
  // so that throughout the call some workgroups compute long query chunks while others stream K/V, instead of
  // every workgroup computing chunks first (HBM idle) and streaming last (HBM saturated, each workgroup
  // slower).  Each class still ends on its shortest units.  A class with few items (the shared-prefix pass's
  // equally long prefix units) is not spread out: an even spread would start some of them last.
  const long long grid_wgs = p.min_items > 0 ? p.min_items / 2 : 256;
  const bool interleave = static_cast<long long>(units_total - units_wide) * Hkv >= grid_wgs &&
                          static_cast<long long>(units_wide) * Hkv >= grid_wgs;
  int* const cnt = sortbuf + kSortBuckets;       // [2][kSortBuckets] units per class and stage bucket
  int* const cumw = sortbuf + 3 * kSortBuckets;  // [2][kSortBuckets] class work before each stage bucket
  int* const cnt2 = sortbuf + 5 * kSortBuckets;  // [2][kSortBuckets] copy of cnt
  // Exact integer keys (the histogram and the scatter compute them separately and must agree bit for bit):
  // key = floor(x * kSortBuckets / W) for class work x <= W, with x and W shifted right alike so that the
  // product stays below 2^31, and the division by the class's W through FastDiv.
  int wshift0 = 0, wshift1 = 0;
  FastDiv wdiv0(2), wdiv1(2);
  // Merge key of the unit of class c, stage bucket b, rank r within the bucket.
  auto merge_key = [&](int c, int b, int r) -> int {
    const int stages = kSortBuckets - 1 - b;
    const long long x = cumw[c * kSortBuckets + b] + static_cast<long long>(r) * stages * kind_weight(c + 1);
    const int xs = static_cast<int>(x >> (c == 0 ? wshift0 : wshift1)) * kSortBuckets;
    return min(kSortBuckets - 1, (c == 0 ? wdiv0 : wdiv1).floor_div(xs));
  };
  if (interleave) {
    for (int i = tid; i < 3 * kSortBuckets; i += kPlanThreads) sortbuf[i] = 0;  // key counters and cnt[][]
    __syncthreads();
    for (int tau = tid; tau < total_tiles; tau += kPlanThreads) {
      OwnParts op;
      int rows_t, wt;
      tile_parts(p.buf.tile_rec[tau], P, Pw, divp, divw, op, rows_t, wt);
      for (int pp = 0; pp < op.n; ++pp) {
        int kb, kl;
        op.range(pp, kb, kl);
        atomicAdd(&cnt[(wt == 2) * kSortBuckets + sort_bucket(kl, 1)], 1);
      }
    }
    for (int i = tid; i < units_v; i += kPlanThreads) {
      const int k = (i % npv) * Pv;
      atomicAdd(&cnt[kSortBuckets + sort_bucket(min(ptok - k, Pv), 1)], 1);
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int mine = 0;
#pragma unroll
      for (int i = 0; i < kBucketsPerThread; ++i) {
        const int b = tid * kBucketsPerThread + i;
        mine += cnt[c * kSortBuckets + b] * (kSortBuckets - 1 - b) * kind_weight(c + 1);
      }
      int total;
      int off = block_exclusive_scan<kPlanWaves>(mine, &total, red);
#pragma unroll
      for (int i = 0; i < kBucketsPerThread; ++i) {
        const int b = tid * kBucketsPerThread + i;
        cumw[c * kSortBuckets + b] = off;
        cnt2[c * kSortBuckets + b] = cnt[c * kSortBuckets + b];
        off += cnt[c * kSortBuckets + b] * (kSortBuckets - 1 - b) * kind_weight(c + 1);
      }
      const int sh = max(0, 32 - __builtin_clz(static_cast<unsigned>(max(total, 1))) - 21);
      const FastDiv dv(max(total >> sh, 2));
      if (c == 0) {
        wshift0 = sh;
        wdiv0 = dv;
      } else {
        wshift1 = sh;
        wdiv1 = dv;
      }
    }
    __syncthreads();
    // Merge-key histogram (bucket[] counts keys): the scatter's walk over the units, with ranks handed out by
    // cnt2, so that every (class, stage bucket, rank) is counted once, as the scatter will place it.
    for (int tau = tid; tau < total_tiles; tau += kPlanThreads) {
      OwnParts op;
      int rows_t, wt;
      tile_parts(p.buf.tile_rec[tau], P, Pw, divp, divw, op, rows_t, wt);
      for (int pp = 0; pp < op.n; ++pp) {
        int kb, kl;
        op.range(pp, kb, kl);
        const int c = wt == 2, b = sort_bucket(kl, 1);
        atomicAdd(&bucket[merge_key(c, b, atomicSub(&cnt2[c * kSortBuckets + b], 1) - 1)], 1);
      }
    }
    for (int i = tid; i < units_v; i += kPlanThreads) {
      const int b = sort_bucket(min(ptok - (i % npv) * Pv, Pv), 1);
      atomicAdd(&bucket[merge_key(1, b, atomicSub(&cnt2[kSortBuckets + b], 1) - 1)], 1);
    }
    __syncthreads();
  } else {
    // Counting sort of the units by weighted stage count, longest first: histogram, bucket offsets, scatter.
#pragma unroll
    for (int i = 0; i < kBucketsPerThread; ++i) bucket[tid * kBucketsPerThread + i] = 0;
    __syncthreads();
    for (int tau = tid; tau < total_tiles; tau += kPlanThreads) {
      OwnParts op;
      int rows_t, wt;
      tile_parts(p.buf.tile_rec[tau], P, Pw, divp, divw, op, rows_t, wt);
      for (int pp = 0; pp < op.n; ++pp) {
        int kb, kl;
        op.range(pp, kb, kl);
        atomicAdd(&bucket[sort_bucket(kl, wt)], 1);
      }
    }
    for (int i = tid; i < units_v; i += kPlanThreads) {
      const int k = (i % npv) * Pv;
      atomicAdd(&bucket[sort_bucket(min(ptok - k, Pv), kind_weight(2))], 1);
    }
    __syncthreads();
  }
  {
    int c[kBucketsPerThread];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kBucketsPerThread; ++i) {
      c[i] = bucket[tid * kBucketsPerThread + i];
      mine += c[i];
    }
    int dummy;
    int off = block_exclusive_scan<kPlanWaves>(mine, &dummy, red);
#pragma unroll
    for (int i = 0; i < kBucketsPerThread; ++i) {
      bucket[tid * kBucketsPerThread + i] = off;
      off += c[i];
    }
  }
  __syncthreads();
  // Slot of the next unit of class c (1: 256-row tiles) in stage bucket b (unweighted stage count).
  auto place = [&](int c, int b) -> int {
    if (!interleave)  // the weighted stage count's bucket, as in the histogram
      return atomicAdd(&bucket[kSortBuckets - 1 - min((kSortBuckets - 1 - b) * kind_weight(c + 1), kSortBuckets - 1)], 1);
    const int r = atomicSub(&cnt[c * kSortBuckets + b], 1) - 1;  // ranks count down: no clearing
    return atomicAdd(&bucket[merge_key(c, b, r)], 1);
  };

  for (int tau = tid; tau < total_tiles; tau += kPlanThreads) {
    const int4 rec = p.buf.tile_rec[tau];
    OwnParts op;
    int rows_t, wt;
    const int np = tile_parts(rec, P, Pw, divp, divw, op, rows_t, wt);
    const int pr = rec.z;
    int4 sq;  // the sequence's first query token, query tokens and context, and its tile kind
    if (rec.x < kSeqCache) {
      const int4 c = seqc[rec.x];
      sq = make_int4(c.w, c.x, c.y, tile_kind_for(c.x * G, p.tile_kind));
    } else {
      const int lo = qsl[rec.x];
      const int n = qsl[rec.x + 1] - lo;
      sq = make_int4(lo, n, ctx[rec.x], tile_kind_for(n * G, p.tile_kind));
    }
    for (int pp = 0; pp < op.n; ++pp) {
      int kb, kl;
      op.range(pp, kb, kl);
      const int slot = place(wt == 2, sort_bucket(kl, 1));
      p.buf.units[2 * slot] = make_int4(rec.x, rec.y, kb, np > 1 ? pr + pp * rows_t * Hkv : -1);
      p.buf.units[2 * slot + 1] = make_int4(sq.x, sq.y, sq.z, sq.w | (kl << 2));
    }
    if (np > op.n) {
      // member of the shared-prefix pass (one tile): its query tokens find their prefix partial rows here
      const int s = rec.x;
      const int q_lo = qsl[s];
      const int n = rows_t / G;
      const int4 info = make_int4(s, pr + op.n * rows_t * Hkv, rows_t, q_lo);
      for (int i = 0; i < n; ++i) p.buf.tok_info[q_lo - vq0 + i] = info;
    }
  }
  for (int i = tid; i < units_v; i += kPlanThreads) {
    const int tv = i / npv;
    const int k = (i - tv * npv) * Pv;
    const int slot = place(1, sort_bucket(min(ptok - k, Pv), 1));
    p.buf.units[2 * slot] = make_int4(N, tv, k, -1);
    p.buf.units[2 * slot + 1] = make_int4(vq0, vn, ptok - 1 + vn, 2 | (min(Pv, ptok - k) << 2));
  }
  if (tid == 0) {
    p.buf.hdr[kHdrUnits] = units_total;
    p.buf.hdr[kHdrQueue] = 0;
    p.buf.hdr[kHdrPartition] = P;
    p.buf.hdr[kHdrPartitionWide] = Pw;
    p.buf.hdr[kHdrTiles] = total_tiles;
    p.buf.hdr[kHdrBadSeqs] = total_bad;
    p.buf.hdr[kHdrPrefQ0] = vq0;
    p.buf.hdr[kHdrPrefN] = vn;
    p.buf.hdr[kHdrPrefL] = ptok - 1 + vn;
    p.buf.hdr[kHdrPrefKeys] = ptok;
    p.buf.hdr[kHdrPrefTable] = pb;
    p.buf.hdr[kHdrPrefPartition] = Pv;
    p.buf.hdr[kHdrPrefParts] = npv;
    p.buf.hdr[kHdrSig0] = p.sig[0];
    p.buf.hdr[kHdrSig1] = p.sig[1];
    p.buf.hdr[kHdrSig2] = p.sig[2];
  }
}

template <int THREADS>
__global__ void __launch_bounds__(THREADS) plan_kernel(const PlanParams p) {
  plan_body<THREADS>(p);
}

// The plan and this step's K/V write in one launch: workgroup 0 plans, the others scatter the new K/V rows.
// They are independent (the planner reads only the metadata; only the attention kernel reads what the write
// stores), and each alone is about one launch's fixed cost.
template <int THREADS>
__global__ void __launch_bounds__(THREADS) write_plan_kernel(const PlanParams p, const KvWriteParams w) {
  if (blockIdx.x == 0) {
    plan_body<THREADS>(p);
    return;
  }
  kv_write_chunks(w, static_cast<int>(blockIdx.x - 1) * THREADS + static_cast<int>(threadIdx.x),
                  static_cast<int>(gridDim.x - 1) * THREADS);
}

// bf16 NaN rows for the sequences a plan rejected (q_len > context, negative context, context past the table):
// bad metadata shows in the result without a host check.  A sequence whose query range itself is inconsistent
// owns no rows and is left alone.  Called by every thread of one workgroup (THREADS threads, whole waves); each
// wave takes its own sequences and a wave-wide loop fills the rows of each rejected one.
template <int THREADS, int D>
__device__ void fill_rejected_rows(const AttnParams& p) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v nan8 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};  // eight bf16 NaNs
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int N = p.num_seqs;
  const int max_context = p.max_blocks_per_seq << p.block_size_log2;
  const int row_chunks = p.num_q_heads * D * 2 / 16;
  for (int base = tid - lane; base < N; base += THREADS) {
    const int s = base + lane;
    int lo = 0, hi = 0;
    bool poison = false;
    if (s < N) {
      lo = p.query_start_loc[s];
      hi = p.query_start_loc[s + 1];
      poison = lo >= 0 && hi > lo && hi <= p.total_q && !seq_ok(lo, hi, p.context_lens[s], p.total_q, max_context);
    }
    unsigned long long m = __builtin_amdgcn_ballot_w64(poison);
    while (m) {
      const int b = __builtin_ctzll(m);
      m &= m - 1;
      const int blo = __builtin_amdgcn_readlane(lo, b);
      const int bhi = __builtin_amdgcn_readlane(hi, b);
      u32x4v* const o = static_cast<u32x4v*>(p.out) + static_cast<int64_t>(blo) * row_chunks;
      const int64_t chunks = static_cast<int64_t>(bhi - blo) * row_chunks;
      for (int64_t c = lane; c < chunks; c += 64) o[c] = nan8;
    }
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
  const int block = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  // The attention kernel has finished (stream order): reset its item queue, so that a later call may run on
  // this plan again.
  if (block == 0 && threadIdx.x == 0) p.buf.hdr[kHdrQueue] = 0;
  if (p.buf.hdr[kHdrSig0] != p.sig[0] || p.buf.hdr[kHdrSig1] != p.sig[1] || p.buf.hdr[kHdrSig2] != p.sig[2]) {
    // The workspace holds no plan for this call's shape (the attention kernel did nothing): the whole output
    // becomes NaN, grid-strided.
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v nan8 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    const int64_t chunks = p.total_q * p.num_q_heads * D * 2 / 16;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z * kThreads;
    for (int64_t c = static_cast<int64_t>(block) * kThreads + threadIdx.x; c < chunks; c += nthreads)
      static_cast<u32x4v*>(p.out)[c] = nan8;
    return;
  }
  if (block == 0 && p.buf.hdr[kHdrBadSeqs] > 0) fill_rejected_rows<kThreads, D>(p);
  if (tile_idx >= p.buf.hdr[kHdrTiles]) return;
  const int4 rec = p.buf.tile_rec[tile_idx];
  const int np = rec.w;
  if (np <= 1) return;
  const int tile = rec.y, pb0 = rec.z;
  const int2 tq = p.buf.tile_q[tile_idx];
  const int q0 = tq.x;
  const int n = tq.y;
  const int G = p.group;
  const int RT = tile_rows_of(tile_kind_for(n * G, p.tile_kind));
  const int row0 = tile * RT;
  const int rows_here = min(RT, n * G - row0);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int d0 = (threadIdx.x % D4) * 4;
  const int64_t part_stride = static_cast<int64_t>(rows_here) * p.num_kv_heads;
  // Workgroup z merges row groups z, z + gridDim.z, ... of RPW rows each.
  for (int rl = blockIdx.z * RPW + threadIdx.x / D4; rl < rows_here; rl += gridDim.z * RPW) {
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
    bf16x4 v;
    v[0] = static_cast<__bf16>(a0 * inv);
    v[1] = static_cast<__bf16>(a1 * inv);
    v[2] = static_cast<__bf16>(a2 * inv);
    v[3] = static_cast<__bf16>(a3 * inv);
    *reinterpret_cast<bf16x4*>(o) = v;
  }
}

}  // namespace

hipError_t launch_plan(const PlanParams& p, hipStream_t stream) {
  if (plan_threads(p) == 256) hipLaunchKernelGGL(plan_kernel<256>, dim3(1), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(plan_kernel<64>, dim3(1), dim3(64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_write_plan(const PlanParams& p, const KvWriteParams& w, hipStream_t stream) {
  if (w.num_tokens == 0) return launch_plan(p, stream);
  const int threads = plan_threads(p);
  // The write's workgroups cover at most kWriteGridLanes lanes, as in launch_kv_write (the host's bound on
  // the chunk count leaves one such stride of room below 2^31).
  const int64_t chunks = static_cast<int64_t>(w.num_tokens) * 2 * w.chunks_per_row;
  int64_t blocks = (chunks + threads - 1) / threads;
  if (blocks > kWriteGridLanes / threads) blocks = kWriteGridLanes / threads;
  const dim3 grid(static_cast<unsigned>(1 + blocks));
  if (threads == 256) hipLaunchKernelGGL(write_plan_kernel<256>, grid, dim3(256), 0, stream, p, w);
  else hipLaunchKernelGGL(write_plan_kernel<64>, grid, dim3(64), 0, stream, p, w);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const AttnParams& p, int head_dim, int tile_cap, hipStream_t stream) {
  if (tile_cap <= 0) return hipSuccess;
  // One workgroup per (tile, kv head, quarter of a 128-row tile's row groups; a 256-row tile's workgroups
  // take twice the rows): most tiles are not split and their workgroups return at once, so the grid is kept
  // small rather than one workgroup per row group.
  const int rows_per_wg = kThreads / (head_dim / 4);
  const int z = (tile_rows_of(1) + 4 * rows_per_wg - 1) / (4 * rows_per_wg);
  const dim3 grid(static_cast<unsigned>(tile_cap), static_cast<unsigned>(p.num_kv_heads), static_cast<unsigned>(z));
  if (head_dim == 128) {
    hipLaunchKernelGGL(split_reduce_kernel<128>, grid, dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(split_reduce_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pkv
