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
// This item body serves row tiles of 128 rows (decode, speculative decode, and any sequence whose q_len x
// group rows fit one such tile); taller tiles (long query chunks) go to the body in attention_wide.h, which
// runs the same pipeline on 32 x 32 MFMA tiles.  attention.hip runs both in one persistent kernel and picks
// the body per work item from the unit's tile kind.
//
// How (gfx950 design, not a translation of any kernel the pages name):
//  * Work item = (unit, kv head) from the device plan; a persistent grid pops items from a queue.  The
//    rows of an item are (query token, head of g's group) pairs, so all G heads sharing kv head g read
//    each K/V byte once.
//  * K/V stream HBM -> LDS with global_load_lds (no register staging) into a 4-deep ring of 64-key
//    stages: while one stage is consumed, up to three are in flight.  Each wave fetches 8 keys of a
//    stage, one uniform physical block per wave-wide load (block_size >= keys per load), each load
//    instruction covering whole 256-byte (D=128) rows.  Block-table entries come through scalar loads
//    issued a stage ahead, so the data loads never wait on a lookup.
//  * In LDS both tiles are row-major [key][D] with the 16-byte chunks of row k XOR-swizzled by k, which
//    keeps the fragment reads conflict-free.  The swizzle is applied on the way in by choosing which lane
//    loads which chunk (the DMA writes lane l's 16 bytes at offset 16*l).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16 (16 keys as M, 16 rows
//    as N): each lane owns one row (lane % 16) for the 8 keys it holds of a 32-key chunk, so row max and
//    row sum need two cross-lane exchanges per chunk, and the probabilities already sit in the B-operand
//    layout of O^T += V^T P^T (v_mfma_f32_16x16x32_bf16, 32 keys as K, taken in the order the S^T
//    fragments deliver them).  The matching V^T operand (8 keys of one channel per lane) is read from the
//    row-major V tile with two ds_read_b64_tr_b16.
//  * Online softmax in log2 units (scale * log2 e folded into the score scale), exp2 on the VALU.
//  * Waves split a tile's rows when it has many (prefill, speculative decode), or the keys when it has
//    few (decode); in the latter case the waves' softmax states are merged through LDS at the end.
//  * A tile whose context was split into partitions writes (acc, m, l) per row; split_reduce_kernel
//    merges them.  Unsplit tiles write the normalised bf16 output directly.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "kernels.h"

namespace pkv {
namespace {

template <int D, int NTW>
struct Geo {
  static constexpr int CPK = D / 8;          // 16-byte chunks per K/V row of one head
  static constexpr int KPL = 64 / CPK;       // keys covered by one wave-wide 16-byte load
  static constexpr int NW = kAttnWaves;     // waves per workgroup
  static constexpr int KPW = kStageKeys / NW;  // keys each wave fetches per stage
  static constexpr int NL = KPW / KPL;       // wave-wide loads per wave, per tensor, per stage
  static constexpr int DC = D / 32;          // 32-channel steps of the QK contraction
  static constexpr int DT = D / 16;          // 16-channel output tiles
  static constexpr int WROWS = 16 * NTW;     // rows one wave owns
  static constexpr int RT = NW * WROWS;      // rows per tile
  static_assert(NTW != 1 || RT == tile_rows_of(1), "the plan and the kernel agree on the tile height");
  static constexpr int ROWB = 2 * D;         // bytes of one key row in LDS
  static constexpr int TILEB = kStageKeys * ROWB;
  static constexpr int STAGEB = 2 * TILEB;   // K tile + V tile
  static constexpr int NBUF = 4;  // ring_slot() orders exactly four slots
  static constexpr int LDS = NBUF * STAGEB;
  static constexpr int MERGE_SLOT = DT * 256 + 32;  // floats per (wave, n-tile) in the merge buffer
  static constexpr int MERGE_BYTES = NW * NTW * MERGE_SLOT * 4;
  static constexpr int SMEM = LDS > MERGE_BYTES ? LDS : MERGE_BYTES;  // ring, later reused for the merge
  static_assert(NL >= 1 && KPW % KPL == 0, "stage split");
  static_assert((STAGEB & (STAGEB - 1)) == 0, "a slot base is whole bits above every offset inside a slot");
};

// One work item (unit, kv head g) on 16-row waves.  Every thread of the workgroup calls it; `smem` is the
// workgroup's ring (at least Geo<D, NTW>::SMEM bytes of LDS); thread 0 claims the next item into
// `next_item` once the item's last stage is consumed.
template <int D, int NTW = 1>
__device__ __forceinline__ void narrow_item(const AttnParams& p, const PlanWords& pw, unsigned char* smem,
                                            int unit, int g, int& next_item) {
  using T = Geo<D, NTW>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Hq = p.num_q_heads;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int last_block = static_cast<int>(p.num_blocks - 1);
  const __bf16* const kc = static_cast<const __bf16*>(p.k_cache);
  const __bf16* const vc = static_cast<const __bf16*>(p.v_cache);
  const __bf16* const qg = static_cast<const __bf16*>(p.q);
  __bf16* const og = static_cast<__bf16*>(p.out);
  const float sl2 = p.scale_log2;
  // LDS byte address of the ring (DMA destinations are given as LDS addresses).
  const unsigned lds_ring = static_cast<unsigned>(reinterpret_cast<size_t>((LDS_AS unsigned char*)smem));

  // Lane-constant parts of the fragment addresses.
  // V^T operand via ds_read_b64_tr_b16: in each 16-lane group the 16 lanes point at 4 keys x 4 groups of
  // 4 channels; lane i of group g4 points at key 4*g4 + i/4, channels 4*(i%4) .. +3 of the 16-channel tile.
  const int tr_key = 4 * g4 + (l16 >> 2);
  const int tr_half = (l16 & 1) << 3;       // byte offset inside the 16-byte chunk
  const int tr_chunk = (l16 & 3) >> 1;      // chunk offset inside the 16-channel tile
  // Byte offsets of the lane's fragment reads in the ring, for key group 0; other key groups (+16, +32,
  // +48 keys) add a constant, because the swizzle depends on the key modulo 16 only.  They include the
  // current stage's slot: stage st sits in slot ring_slot(st) (0, 1, 3, 2), so one XOR per register moves
  // them on to the next stage.
  int koff[T::DC];  // K: key l16, 16-byte chunk 4*dc + g4 (A operand of S^T = K Q^T)
  int voff[T::DT];  // V: transpose-read row of tile dt (A operand of O^T += V^T P^T)
#pragma unroll
  for (int dc = 0; dc < T::DC; ++dc) koff[dc] = l16 * T::ROWB + (((4 * dc + g4) ^ k_swizzle<D>(l16)) << 4);
#pragma unroll
  for (int dt = 0; dt < T::DT; ++dt)
    voff[dt] = T::TILEB + tr_key * T::ROWB + tr_half + (((2 * dt + tr_chunk) ^ k_swizzle<D>(tr_key)) << 4);
  // bf16 ones: A operand that turns an MFMA over P^T into the row sums of P.
  bf16x8 ones;
#pragma unroll
  for (int t = 0; t < 8; ++t) ones[t] = static_cast<__bf16>(1.f);
  const float inv_sl2 = 1.f / sl2;

  {
    // The plan's arrays are read-only here: scalar loads (constant address space) keep these reads off
    // the vector-memory counter.
    const CONST_AS int* const urec = (const CONST_AS int*)p.buf.units + 8 * unit;
    const int s = urec[0], tile = urec[1], kb = urec[2], pbase = urec[3];
    const int q0 = urec[4];  // the sequence's first query token, query tokens and context, from the plan
    const int n = urec[5];
    const int L = urec[6];
    const int row0 = tile * T::RT;
    const int rows_here = min(T::RT, n * G - row0);
    const int kmax = L - n + (row0 + rows_here - 1) / G + 1;
    const int ke = min(kmax, kb + (urec[7] >> 2));  // the partition's key count, from the plan
    const int WR = rows_here <= T::WROWS ? 1
                   : rows_here <= 2 * T::WROWS ? 2
                   : rows_here <= 4 * T::WROWS ? 4 : 8;
    const int WK = T::NW / WR;
    // Wave w (on SIMD w % 4) takes row group w % WR and key group w / WR: the waves that compute one stage's
    // chunks (two key groups, all row groups) then sit on different SIMDs.
    const int wk = wave / WR;
    const int wr = wave - wk * WR;
    const int my_row0 = row0 + wr * T::WROWS;
    // 16-row n-tiles of this wave that hold rows of the item (0 when the last row group is empty).
    const int ntv = min(NTW, (row0 + rows_here - my_row0 + 15) >> 4);
    // Last visible key of the wave's first row: chunks ending at or before it need no mask for any row
    // of the wave (rows are ordered by query token, whose visible range only grows).
    const int lim0 = min(L - n + my_row0 / G, ke - 1);
    // Last visible key of the wave's last row: later chunks are masked for the whole wave and skipped.
    const int limw = min(L - n + (min(my_row0 + 16 * ntv, row0 + rows_here) - 1) / G, ke - 1);
    const CONST_AS int* const tbl =
        (const CONST_AS int*)(p.block_tables + static_cast<int64_t>(s) * p.max_blocks_per_seq);
    const int nst = (ke - kb + kStageKeys - 1) / kStageKeys;

    // Physical blocks of this wave's NL loads of stage st (scalar loads; keys past ke clamp to ke-1).
    auto fetch_table = [&](int st, int* phys) {
#pragma unroll
      for (int i = 0; i < T::NL; ++i) {
        const int kfirst = min(kb + st * kStageKeys + T::KPW * wave + T::KPL * i, ke - 1);
        phys[i] = tbl[kfirst >> bs_log2];
      }
    };
    // Wave w fetches keys [KPW*w, KPW*(w+1)) of stage st into ring slot ring_slot(st).  Keys at or past ke are
    // clamped to row ke-1 of the same block (a wave-wide load never spans two blocks); their scores are
    // masked, so those rows carry probability 0, and rows past the context are never read.
    auto issue = [&](int st, const int* phys) {
      unsigned char* const kdst = smem + ring_slot(st) * T::STAGEB;
      const int key0 = kb + st * kStageKeys + T::KPW * wave;
#pragma unroll
      for (int i = 0; i < T::NL; ++i) {
        const int key_local = T::KPW * wave + T::KPL * i + lane / T::CPK;
        const int kk = min(key0 + T::KPL * i + lane / T::CPK, ke - 1);
        const int ph = min(max(phys[i], 0), last_block);
        const int c = (lane % T::CPK) ^ k_swizzle<D>(key_local);
        const int64_t e = static_cast<int64_t>(ph) * p.block_stride +
                          (static_cast<int64_t>(kk & bs_mask) * Hkv + g) * D + c * 8;
        const unsigned dk = lds_ring + static_cast<unsigned>((kdst - smem) + (T::KPW * wave + T::KPL * i) * T::ROWB);
        dma16(kc + e, dk);
        dma16(vc + e, dk + T::TILEB);
      }
    };

    int tb0[T::NL], tb1[T::NL], tb2[T::NL], tbn[T::NL];
    fetch_table(0, tb0);
    if (nst > 1) fetch_table(1, tb1);
    if (nst > 2) fetch_table(2, tb2);
    if (nst > 3) fetch_table(3, tbn);

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

    // The query fragments must be in registers before the stage copies are issued: the compiler does not
    // count the copies, so any wait it placed for q inside the loop would drain them every stage.
    wait_vmem<0>();
    issue(0, tb0);
    if (nst > 1) issue(1, tb1);
    if (nst > 2) issue(2, tb2);

    f32x4 acc[NTW][T::DT];
    f32x4 lacc[NTW];   // row sums of P, accumulated by MFMA (all four entries equal)
    float m[NTW];      // reference maximum of the row's scaled scores (log2 units)
    float thr[NTW];    // raw score above which m must move: (m + kLazyRescale) / (scale log2 e)
    float nmr[NTW];    // -m, or 0 while m is -inf
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      m[nt] = -INFINITY;
      thr[nt] = -INFINITY;
      nmr[nt] = 0.f;
      lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One 32-key chunk (keys kc0 + [0, 32) at rows 32c .. 32c+31 of the stage tiles) for the wave's first
    // NA n-tiles.  kp / vp: the lane's K / V read addresses in the current stage for key group 0.
    auto chunk = [&](auto na_tag, const unsigned char* const* kp, const unsigned char* const* vp, int c,
                     int kc0) __attribute__((always_inline)) {
      constexpr int NA = decltype(na_tag)::value;
      // S^T for keys 32c + 16mt + [0, 16), mt = 0, 1.
      f32x4 sacc[NA][2];
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) sacc[nt][0] = sacc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int dc = 0; dc < T::DC; ++dc) {
          const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(kp[dc] + (32 * c + 16 * mt) * T::ROWB));
#pragma unroll
          for (int nt = 0; nt < NA; ++nt) sacc[nt][mt] = mfma_qk(kf, qf[nt][dc], sacc[nt][mt]);
        }
      }
      // V^T operands of this chunk, read now so that their LDS latency hides behind the softmax.
      bf16x8 vf[T::DT];
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[dt] + 32 * c * T::ROWB));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp[dt] + (32 * c + 16) * T::ROWB));
        vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      // Online softmax over the 32 keys; the lane holds keys kc0 + 4*g4 + 16*mt + [0, 4) of row l16.
      // Raw scores are compared (the scale is positive) and the scale is applied inside the exponent.
      float sv[NA][8];
#pragma unroll
      for (int nt = 0; nt < NA; ++nt)
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) sv[nt][k8] = sacc[nt][k8 >> 2][k8 & 3];
      if (kc0 + 31 > lim0) {  // the chunk reaches past some row's last visible key
        const int kl = kc0 + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < NA; ++nt)
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8)
            sv[nt][k8] = (kl + 16 * (k8 >> 2) + (k8 & 3) <= lim[nt]) ? sv[nt][k8] : -INFINITY;
      }
      // Lane-local maxima; only when one exceeds its row's threshold are the rows' maxima formed and the
      // references moved (rare after the first chunk).
      float lm[NA];
      bool grow = false;
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) {
        float x = sv[nt][0];
#pragma unroll
        for (int k8 = 1; k8 < 8; ++k8) x = fmaxf(x, sv[nt][k8]);
        lm[nt] = x;
        grow |= x > thr[nt];
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) {
          const float mnew = fmaxf(m[nt], row_max4(lm[nt]) * sl2);
          if (mnew != -INFINITY) {
            const float alpha = __builtin_amdgcn_exp2f(m[nt] - mnew);
            lacc[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) acc[nt][dt] *= alpha;
            m[nt] = mnew;
            nmr[nt] = -mnew;
            thr[nt] = (mnew + kLazyRescale) * inv_sl2;
          }
        }
      }
      bf16x8 pf[NA];
#pragma unroll
      for (int nt = 0; nt < NA; ++nt)
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8)
          pf[nt][k8] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[nt][k8], sl2, nmr[nt])));
      // O^T += V^T P^T over the 32 keys (v_mfma_f32_16x16x32_bf16): the contraction index 8*g4 + t is key
      // 4*g4 + t of the first 16-key half for t < 4 and of the second half for t >= 4, which is where the
      // S^T fragments put the probabilities; one transpose read per half gives the matching V^T operand.
      // The row sums of the same bf16 probabilities come from one more MFMA against ones.
#pragma unroll
      for (int nt = 0; nt < NA; ++nt) lacc[nt] = mfma_qk(ones, pf[nt], lacc[nt]);
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int nt = 0; nt < NA; ++nt) acc[nt][dt] = mfma_qk(vf[dt], pf[nt], acc[nt][dt]);
    };

    for (int st = 0; st < nst; ++st) {
      // Stage st has landed once at most the later stages' loads are outstanding.
      const int later = min(2, nst - 1 - st);
      if (later == 2) wait_vmem<4 * T::NL>();
      else if (later == 1) wait_vmem<2 * T::NL>();
      else wait_vmem<0>();
      __syncthreads();  // all waves' loads of stage st landed; all waves done with stage st-1

      const unsigned char* kp[T::DC];
      const unsigned char* vp[T::DT];
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) kp[dc] = smem + koff[dc];
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) vp[dt] = smem + voff[dt];
      const int kstage = kb + st * kStageKeys;
      // Two 32-key chunks per stage; chunk number st*2+c goes to the key-group (st*2+c) % WK.  The copy of
      // stage st + 3 refills the slot of stage st - 1, free since the barrier; it goes out after the first
      // chunk, so that the waves computing that chunk start right after the barrier.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kc0 = kstage + 32 * c;
        if (((st * 2 + c) % WK) == wk && kc0 <= limw) {
          if (NTW > 1 && ntv == NTW) chunk(std::integral_constant<int, NTW>{}, kp, vp, c, kc0);
          else if (ntv > 0) chunk(std::integral_constant<int, 1>{}, kp, vp, c, kc0);
        }
        if (c == 0 && st + 3 < nst) issue(st + 3, tbn);
      }
      if (st + 4 < nst) fetch_table(st + 4, tbn);
      // On to the next stage's slot: ring_slot(st) ^ ring_slot(st + 1) is bit 0 for even st, bit 1 for odd.
      const int flip = (st & 1) ? 2 * T::STAGEB : T::STAGEB;
#pragma unroll
      for (int dc = 0; dc < T::DC; ++dc) koff[dc] ^= flip;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) voff[dt] ^= flip;
    }

    // (workgroup w's first item was item w: the queue hands out the items from gridDim.x on)
    if (tid == 0) next_item = static_cast<int>(gridDim.x) + atomicAdd(p.buf.hdr + kHdrQueue, 1);

    float lsum[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) lsum[nt] = lacc[nt][0];

    // Writes d-tile dt of the lane's row in n-tile nt: the normalised bf16 output, or for a split tile
    // the partial (acc, and with_ml: m and l).
    auto emit = [&](int nt, int dt, f32x4 a, float mm, float ll, bool with_ml) __attribute__((always_inline)) {
      const int r = my_row0 + nt * 16 + l16;
      if (r >= row0 + rows_here) return;
      if (pbase < 0) {
        const int i = r / G;
        const int hh = r - i * G;
        const float inv = 1.f / ll;
        bf16x4 v;
        v[0] = static_cast<__bf16>(a[0] * inv);
        v[1] = static_cast<__bf16>(a[1] * inv);
        v[2] = static_cast<__bf16>(a[2] * inv);
        v[3] = static_cast<__bf16>(a[3] * inv);
        *reinterpret_cast<bf16x4*>(og + ((static_cast<int64_t>(q0 + i) * Hq + g * G + hh) * D + 4 * g4 + 16 * dt)) = v;
      } else {
        const int64_t prow = static_cast<int64_t>(pbase) + g * rows_here + (r - row0);
        *reinterpret_cast<f32x4*>(p.buf.part_acc + prow * D + 4 * g4 + 16 * dt) = a;
        if (with_ml && g4 == 0) p.buf.part_ml[prow] = make_float2(mm, ll);
      }
    };

    if (WK == 1) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) emit(nt, dt, acc[nt][dt], m[nt], lsum[nt], dt == 0);
    } else {
      // The WK waves of a row group split the keys: each publishes its (acc, m, l) in LDS, then wave
      // (wr, wk) combines d-tiles wk, wk + WK, ... of all WK states, so the merge is spread over the waves.
      __syncthreads();  // every wave is done with the ring
      float* const mb = reinterpret_cast<float*>(smem);
      float* const grp = mb + (wr * WK * NTW) * T::MERGE_SLOT;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (nt >= ntv) break;  // only n-tiles with rows are merged
        float* const b = grp + (wk * NTW + nt) * T::MERGE_SLOT;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) *reinterpret_cast<f32x4*>(b + dt * 256 + lane * 4) = acc[nt][dt];
        if (g4 == 0) {
          b[T::DT * 256 + 2 * l16] = m[nt];
          b[T::DT * 256 + 2 * l16 + 1] = lsum[nt];
        }
      }
      __syncthreads();
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if (nt >= ntv) break;
        const float* const st0 = grp + nt * T::MERGE_SLOT + T::DT * 256 + 2 * l16;  // (m, l) of partner 0
        float M = -INFINITY;
        for (int o = 0; o < WK; ++o) M = fmaxf(M, st0[o * NTW * T::MERGE_SLOT]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f;
        for (int o = 0; o < WK; ++o) {
          const float* const so = st0 + o * NTW * T::MERGE_SLOT;
          Lsum += so[1] * __builtin_amdgcn_exp2f(so[0] - Mr);
        }
        for (int dt = wk; dt < T::DT; dt += WK) {
          f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int o = 0; o < WK; ++o) {
            const float* const so = st0 + o * NTW * T::MERGE_SLOT;
            a += *reinterpret_cast<const f32x4*>(grp + (o * NTW + nt) * T::MERGE_SLOT + dt * 256 + lane * 4) *
                 __builtin_amdgcn_exp2f(so[0] - Mr);
          }
          emit(nt, dt, a, M, Lsum, dt == 0);
        }
      }
    }
  }
}


}  // namespace
}  // namespace pkv
