// Paged attention for long query chunks, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Same computation as the 16-row item body (attention_narrow.h): per sequence s and kv head g, the sequence's
// K/V are the first L rows of its physical blocks in block-table order ("Paged Attention 基础 – 原理与实现
// 进度", §2 block-table figure, steps 1-4), and each new query token i (the last n positions) attends keys
// 0 .. L-n+i with softmax(Q K^T * scale) V (same figure, step 5).  Used for row tiles of 256 (query token,
// grouped head) rows, i.e. prefill and chunked-prefill work, and for the shared-prefix sequence of
// paged_attention_forward_prefix.  attention.hip runs this item body and the 16-row one in one kernel.
//
// How (gfx950 design):
//  * Each wave owns 32 rows of the tile per 32 x 32 half (v_mfma_f32_32x32x16_bf16, twice the sustained
//    rate of the 16 x 16 x 32 form on MI355X): eight waves of one half (two per SIMD), or four waves of
//    two halves, where every K or V fragment read from LDS feeds both halves.
//  * K/V arrive in LDS through the same 4-deep ring of 64-key stages as the 16-row kernel (each wave
//    copies 64 / waves keys of a stage, 8 with eight waves; block-table entries through scalar loads a
//    stage ahead), under this kernel's own chunk swizzle (wide_swizzle), which keeps its V transpose
//    reads free of bank conflicts.
//  * S^T = K Q^T: A = K (32 keys x 16 channels, one 16-byte read per lane), B = Q^T from registers.
//    Lane l holds row l % 32 and keys 8i + 4(l/32) + [0, 4), i < 4, of each 32-key chunk, so the row's
//    maximum and sum need one exchange of the wave halves.
//  * O^T += V^T P^T in two 16-key steps; the lane's own probabilities are the B operand in the order
//    16s + 8(t/4) + 4(l/32) + t%4, and two ds_read_b64_tr_b16 per step give V^T in that order.
//  * Lazy online softmax as in the 16-row kernel (reference maximum moves only on growth beyond 2^8);
//    row sums add the bf16 probabilities pairwise with v_dot2_f32_bf16, i.e. the values the PV MFMAs use.
//  * The two waves sharing a SIMD (w and w + 4) run at different issue priorities, so their matrix and
//    vector phases stagger instead of coinciding after every stage barrier.
//  * Tiles with few rows (decode-like units of a mixed batch) split the keys among the waves, whose states
//    are merged through LDS; split partitions write (acc, m, l) for split_reduce_kernel.
#pragma once

#include <type_traits>

#include "device_util.h"
#include "kernels.h"

namespace pkv {
namespace {

// Halves (32-row MFMA tiles) per wave of the built kernel: 1 = eight waves of 32 rows (two per SIMD),
// 2 = four waves of 64 rows (one per SIMD).
constexpr int kWideHalves = 1;

// 16-byte-chunk swizzle of LDS row `key` for this kernel's reads.  For D = 128 (16 chunks per row) the two
// low bits of the key pick the upper two bits of the chunk mask and the next two bits the lower two: the
// four keys that one half-wave's V transpose read covers (4 chunks each) then land on 16 distinct chunks,
// and K's 16-byte reads (16 keys per 16 lanes, one chunk each) stay on distinct chunks too.  The plain
// key-as-mask swizzle puts those four keys on the same four chunks (a 4-way bank conflict).
template <int D>
__device__ inline int wide_swizzle(int key) {
  return D == 128 ? (((key & 3) << 2) | ((key >> 2) & 3)) : ((key >> 1) & 7);
}

template <int D, int NH>
struct WideGeo {
  static constexpr int CPK = D / 8;             // 16-byte chunks per K/V row of one head
  static constexpr int KPL = 64 / CPK;          // keys covered by one wave-wide 16-byte load
  static constexpr int NW = 8 / NH;             // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static_assert(THREADS == 64 * (8 / NH), "launch bounds");
  static constexpr int WAVE_ROWS = 32 * NH;
  static constexpr int KPW = kStageKeys / NW;   // keys each wave copies per stage
  static constexpr int NL = KPW / KPL;          // wave-wide loads per wave, per tensor, per stage
  static constexpr int KS = D / 16;             // 16-channel steps of the QK contraction
  static constexpr int DT = D / 32;             // 32-channel output tiles
  static constexpr int RT = NW * WAVE_ROWS;
  static_assert(RT == tile_rows_of(2), "the plan and the kernel agree on the tile height");
  static constexpr int ROWB = 2 * D;            // bytes of one key row in LDS
  static constexpr int TILEB = kStageKeys * ROWB;
  static constexpr int STAGEB = 2 * TILEB;      // K tile + V tile
  static constexpr int NBUF = 4;                // ring_slot() orders exactly four slots
  static constexpr int RING = NBUF * STAGEB;
  // Merge slot of one wave, in floats: acc of its halves as [half][dt][j/4][lane][4], then (m, l) of
  // its rows.
  static constexpr int MACC = NH * DT * 16 * 64;
  static constexpr int MSLOT = MACC + NH * 32 * 2;
  static constexpr int MERGE_BYTES = NW * MSLOT * 4;
  static constexpr int SMEM = RING > MERGE_BYTES ? RING : MERGE_BYTES;
  static_assert(NL >= 1 && KPW % KPL == 0, "stage split");
  static_assert((STAGEB & (STAGEB - 1)) == 0, "a slot base is whole bits above every offset inside a slot");
};

// One work item (unit, kv head g) on 32-row waves.  Every thread of the workgroup calls it; `smem` is the
// workgroup's ring (at least WideGeo<D, NH>::SMEM bytes of LDS); thread 0 claims the next item into
// `next_item` once the item's last stage is consumed.
template <int D, int NH = 1>
__device__ __forceinline__ void wide_item(const AttnParams& p, const PlanWords& pw, unsigned char* smem,
                                          int unit, int g, int& next_item) {
  using T = WideGeo<D, NH>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Hq = p.num_q_heads;
  // Shared-prefix sequence (index num_seqs in the unit records; absent when it has no tokens).
  const int pre_keys = pw.pre_keys;
  const int pre_table = pw.pre_table;
  const int pre_P = pw.pre_P;
  const int bs_log2 = p.block_size_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int last_block = static_cast<int>(p.num_blocks - 1);
  const __bf16* const kc = static_cast<const __bf16*>(p.k_cache);
  const __bf16* const vc = static_cast<const __bf16*>(p.v_cache);
  const __bf16* const qg = static_cast<const __bf16*>(p.q);
  __bf16* const og = static_cast<__bf16*>(p.out);
  const float sl2 = p.scale_log2;
  const float inv_sl2 = 1.f / sl2;
  const unsigned lds_ring = static_cast<unsigned>(reinterpret_cast<size_t>((LDS_AS unsigned char*)smem));

  // Lane offsets of the fragment reads in the ring.  K (A operand of S^T): key l32, 16-byte chunk
  // 2ks + hf.  V (A operand of O^T, transpose reads): in each 16-lane group, lane i points at key
  // 4hf + i/4 (+8 for the second read of a step) and channels 32dt + 16(group % 2) + 4(i % 4).  Later key
  // groups (+16, +32) are constant offsets: the swizzle depends on the key modulo 16 only.  The offsets
  // include the current stage's slot: stage st sits in slot gray(st mod 4) (0, 1, 3, 2), so consecutive
  // stages' slots differ in one bit and one XOR per register moves every offset on to the next stage
  // (a slot base added per read would cost two instructions per register and chunk).
  int kof[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) kof[ks] = l32 * T::ROWB + (((2 * ks + hf) ^ wide_swizzle<D>(l32)) << 4);
  int vof[T::DT][2];
  {
    const int gi = lane & 15, gq = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
      for (int e8 = 0; e8 < 2; ++e8) {
        const int key = 4 * hf + (gi >> 2) + 8 * e8;
        vof[dt][e8] = T::TILEB + key * T::ROWB + (gi & 1) * 8 +
                      (((4 * dt + 2 * gq + ((gi & 3) >> 1)) ^ wide_swizzle<D>(key)) << 4);
      }
  }

  // Waves w and w + 4 share a SIMD.  Giving the lower one a higher issue priority lets its QK MFMAs run
  // first after each stage barrier, so that its softmax overlaps the partner's QK and its PV the partner's
  // softmax, instead of both waves reaching their vector phases together.  (Reset when the item ends.)
  if (T::NW == 8 && wave < 4) __builtin_amdgcn_s_setprio(1);

  {
    // Unit record through scalar loads: {sequence, tile, first key, first partial row} and the sequence's
    // {first query token, query tokens, context}.
    const CONST_AS int* const urec = (const CONST_AS int*)p.buf.units + 8 * unit;
    const int s = urec[0], tile = urec[1], kb = urec[2], pbase = urec[3];
    // The shared-prefix sequence: its query tokens are the member sequences' and every prefix key is
    // visible to each of them (its context is prefix length - 1 + token count); its rows' results are
    // partial rows of the members' tiles.
    const bool pre = s == p.num_seqs;
    const int q0 = urec[4];
    const int n = urec[5];
    const int L = urec[6];
    const int row0 = tile * T::RT;
    const int rows_here = min(T::RT, n * G - row0);
    const int kmax = L - n + (row0 + rows_here - 1) / G + 1;
    const int ke = pre ? min(min(kmax, kb + pre_P), pre_keys) : min(kmax, kb + (urec[7] >> 2));
    const int pre_part = pre ? kb / pre_P : 0;  // partition of the prefix sequence
    // Waves split the rows (WAVE_ROWS each) when there are enough, else the keys: WR row groups x WK key
    // groups.
    const int WR = rows_here <= T::WAVE_ROWS ? 1
                   : rows_here <= 2 * T::WAVE_ROWS ? 2
                   : (rows_here <= 4 * T::WAVE_ROWS || T::NW == 4) ? 4 : 8;
    const int WK = T::NW / WR;
    const int wr = wave / WK;
    const int wk = wave - wr * WK;
    const int my_row0 = row0 + wr * T::WAVE_ROWS;
    // 32-row halves of this wave that hold rows of the item (0 when its row group is empty).
    const int nh = min(NH, (row0 + rows_here - my_row0 + 31) >> 5);
    // Last visible key of the wave's first row (chunks ending by it need no mask) and of its last row
    // (later chunks are masked for the whole wave and skipped).
    const int lim0 = min(L - n + my_row0 / G, ke - 1);
    const int limw = min(L - n + (min(my_row0 + 32 * nh, row0 + rows_here) - 1) / G, ke - 1);
    const CONST_AS int* const tbl =
        (const CONST_AS int*)(p.block_tables + static_cast<int64_t>(pre ? pre_table : s) * p.max_blocks_per_seq);
    const int nst = (ke - kb + kStageKeys - 1) / kStageKeys;

    // Physical blocks of this wave's NL loads of stage st (scalar loads; keys past ke clamp to ke-1).
    auto fetch_table = [&](int st, int* phys) {
#pragma unroll
      for (int i = 0; i < T::NL; ++i) {
        const int kfirst = min(kb + st * kStageKeys + T::KPW * wave + T::KPL * i, ke - 1);
        phys[i] = tbl[kfirst >> bs_log2];
      }
    };
    // Wave w copies keys [KPW*w, KPW*(w+1)) of stage st into ring slot ring_slot(st); keys at or past ke are
    // clamped to row ke-1 of the same block and masked.  Row-split items (long chunks: the tiles of one
    // sequence re-read its K/V) copy with the default cache policy, key-split ones stream non-temporally.
    auto issue_p = [&](int st, const int* phys, auto keep_tag) __attribute__((always_inline)) {
      constexpr bool KEEP = decltype(keep_tag)::value;
      unsigned char* const kdst = smem + ring_slot(st) * T::STAGEB;
      const int key0 = kb + st * kStageKeys + T::KPW * wave;
#pragma unroll
      for (int i = 0; i < T::NL; ++i) {
        const int key_local = T::KPW * wave + T::KPL * i + lane / T::CPK;
        const int kk = min(key0 + T::KPL * i + lane / T::CPK, ke - 1);
        const int ph = min(max(phys[i], 0), last_block);
        const int c = (lane % T::CPK) ^ wide_swizzle<D>(key_local);
        const int64_t e = static_cast<int64_t>(ph) * p.block_stride +
                          (static_cast<int64_t>(kk & bs_mask) * Hkv + g) * D + c * 8;
        const unsigned dk =
            lds_ring + static_cast<unsigned>((kdst - smem) + (T::KPW * wave + T::KPL * i) * T::ROWB);
        if (KEEP) {
          dma16_keep(kc + e, dk);
          dma16_keep(vc + e, dk + T::TILEB);
        } else {
          dma16(kc + e, dk);
          dma16(vc + e, dk + T::TILEB);
        }
      }
    };
    auto issue = [&](int st, const int* phys) __attribute__((always_inline)) {
      if (WK == 1) issue_p(st, phys, std::true_type{});
      else issue_p(st, phys, std::false_type{});
    };

    int tb0[T::NL], tb1[T::NL], tb2[T::NL], tbn[T::NL];
    fetch_table(0, tb0);
    if (nst > 1) fetch_table(1, tb1);
    if (nst > 2) fetch_table(2, tb2);
    if (nst > 3) fetch_table(3, tbn);

    // Query fragments of both halves (B operand: Q[row][16ks + 8hf + 0..7]) and each lane row's last
    // visible key (-1 for padding rows).
    bf16x8 q[NH][T::KS];
    int lim[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int r = my_row0 + 32 * h + l32;
      if (r < row0 + rows_here) {
        const int ri = r / G;
        const int rh = r - ri * G;
        const __bf16* const qp = qg + ((static_cast<int64_t>(q0 + ri) * Hq + g * G + rh) * D + 8 * hf);
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) q[h][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + 16 * ks));
        lim[h] = min(L - n + ri, ke - 1);
      } else {
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) q[h][ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        lim[h] = -1;
      }
    }
    // The query must be in registers before the stage copies are issued: the compiler does not count the
    // copies, so any wait it placed for q inside the loop would drain them every stage.
    wait_vmem<0>();
    issue(0, tb0);
    if (nst > 1) issue(1, tb1);
    if (nst > 2) issue(2, tb2);

    f32x16 acc[NH][T::DT];
    float mw[NH], thw[NH], nmw[NH], lw[NH];  // reference max (log2), growth threshold (raw), -max, lane sum
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      mw[h] = -INFINITY;
      thw[h] = -INFINITY;
      nmw[h] = 0.f;
      lw[h] = 0.f;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[h][dt][j] = 0.f;
    }
    // Two bf16 ones: the row sums add the probabilities as rounded for the PV MFMAs, two per instruction.
    bf16x2 ones2;
    ones2[0] = static_cast<__bf16>(1.f);
    ones2[1] = static_cast<__bf16>(1.f);

    // One 32-key chunk (keys kc0 + [0, 32) at rows 32c .. 32c+31 of the stage tiles) for every half of
    // the wave (a half without rows computes on zero queries; its results are never written).
    auto chunk = [&](int c, int kc0) __attribute__((always_inline)) {
      f32x16 sc[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[h][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(smem + kof[ks] + 32 * c * T::ROWB));
#pragma unroll
        for (int h = 0; h < NH; ++h) sc[h] = mfma32(kf, q[h][ks], sc[h]);
      }
      // V^T operands of both 16-key steps, read before the softmax so their latency hides behind it.
      bf16x8 vf[T::DT][2];
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int ko = (32 * c + 16 * s2) * T::ROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(smem + vof[dt][0] + ko));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(smem + vof[dt][1] + ko));
          vf[dt][s2] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      float sv[NH][16];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) sv[h][j] = sc[h][j];
      if (kc0 + 31 > lim0) {  // the chunk reaches past some row's last visible key
        const int kl = kc0 + 4 * hf;
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int j = 0; j < 16; ++j) sv[h][j] = (kl + 8 * (j >> 2) + (j & 3) <= lim[h]) ? sv[h][j] : -INFINITY;
      }
      float x[NH];
      bool grow = false;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        x[h] = sv[h][0];
#pragma unroll
        for (int j = 1; j < 16; ++j) x[h] = fmaxf(x[h], sv[h][j]);
        grow |= x[h] > thw[h];
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const float mnew = fmaxf(mw[h], pair_max(x[h]) * sl2);  // lanes l, l^32 share the row
          if (mnew != -INFINITY) {
            const float alpha = __builtin_amdgcn_exp2f(mw[h] - mnew);
            lw[h] *= alpha;
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) acc[h][dt] *= alpha;
            mw[h] = mnew;
            nmw[h] = -mnew;
            thw[h] = (mnew + kLazyRescale) * inv_sl2;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        // P^T (B operand) of step s2: the lane's keys 16s2 + 8(t/4) + 4hf + t%4, t < 8.
        bf16x8 pf[2];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          pf[j >> 3][j & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv[h][j], sl2, nmw[h])));
#pragma unroll
        for (int j2 = 0; j2 < 8; ++j2) {
          bf16x2 pr;
          pr[0] = pf[j2 >> 2][2 * (j2 & 3)];
          pr[1] = pf[j2 >> 2][2 * (j2 & 3) + 1];
          lw[h] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, lw[h], false);
        }
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) acc[h][dt] = mfma32(vf[dt][s2], pf[s2], acc[h][dt]);
      }
    };

    for (int st = 0; st < nst; ++st) {
      // Stage st has landed once at most the later stages' loads are outstanding.
      const int later = min(2, nst - 1 - st);
      if (later == 2) wait_vmem<4 * T::NL>();
      else if (later == 1) wait_vmem<2 * T::NL>();
      else wait_vmem<0>();
      __syncthreads();  // all waves' loads of stage st landed; all waves done with stage st-1
      // Stage st + 3 refills the slot of stage st - 1, free since the barrier.  Its copies are issued between
      // the two chunks, so that each wave's first MFMAs follow the barrier directly.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kc0 = kb + st * kStageKeys + 32 * c;
        if (((st * 2 + c) % WK) == wk && kc0 <= limw && nh > 0) chunk(c, kc0);
        if (c == 0 && st + 3 < nst) issue(st + 3, tbn);
      }
      if (st + 4 < nst) fetch_table(st + 4, tbn);
      // On to the next stage's slot: gray(st) ^ gray(st + 1) is slot bit 0 for even st, bit 1 for odd.
      const int flip = (st & 1) ? 2 * T::STAGEB : T::STAGEB;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) kof[ks] ^= flip;
#pragma unroll
      for (int dt = 0; dt < T::DT; ++dt) {
        vof[dt][0] ^= flip;
        vof[dt][1] ^= flip;
      }
    }

    // (workgroup w's first item was item w: the queue hands out the items from gridDim.x on)
    if (tid == 0) next_item = static_cast<int>(gridDim.x) + atomicAdd(p.buf.hdr + kHdrQueue, 1);
    float lrow[NH];  // the rows' sums over both halves of the keys
#pragma unroll
    for (int h = 0; h < NH; ++h) lrow[h] = pair_sum(lw[h]);

    // Writes output tile dt of the lane's row in half h: the normalised bf16 output, or for a split tile
    // the partial (acc, and with_ml: m and l).
    auto emit = [&](int h, int dt, const f32x16& a, float mm, float ll, bool with_ml) __attribute__((always_inline)) {
      const int r = my_row0 + 32 * h + l32;
      if (r >= row0 + rows_here) return;
      const int ri = r / G;
      const int rh = r - ri * G;
      if (pbase < 0 && !pre) {
        const float inv = 1.f / ll;
        __bf16* const o = og + ((static_cast<int64_t>(q0 + ri) * Hq + g * G + rh) * D + 32 * dt + 4 * hf);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = static_cast<__bf16>(a[4 * i4 + t] * inv);
          *reinterpret_cast<bf16x4*>(o + 8 * i4) = v;
        }
      } else {
        int64_t prow;
        if (pre) {
          // token ri of the prefix sequence belongs to member info.x, whose tile keeps this partition's
          // partial rows from info.y on: partition pre_part, kv head g, the member's row
          const int4 info = p.buf.tok_info[ri];
          prow = static_cast<int64_t>(info.y) + (pre_part * Hkv + g) * info.z + (q0 + ri - info.w) * G + rh;
        } else {
          prow = static_cast<int64_t>(pbase) + g * rows_here + (r - row0);
        }
        float* const pa = p.buf.part_acc + prow * D + 32 * dt + 4 * hf;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          f32x4 v;
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = a[4 * i4 + t];
          *reinterpret_cast<f32x4*>(pa + 8 * i4) = v;
        }
        if (with_ml && hf == 0) p.buf.part_ml[prow] = make_float2(mm, ll);
      }
    };

    if (WK == 1) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) emit(h, dt, acc[h][dt], mw[h], lrow[h], dt == 0);
    } else {
      // The WK waves of a row group split the keys: each publishes its (acc, m, l) in LDS, then wave
      // (wr, wk) combines output tiles wk, wk + WK, ... of all WK states.
      __syncthreads();  // every wave is done with the ring
      float* const grp = reinterpret_cast<float*>(smem) + (wr * WK) * T::MSLOT;
      float* const mine = grp + wk * T::MSLOT;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if (h >= nh) break;
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            f32x4 v;
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = acc[h][dt][4 * j4 + t];
            *reinterpret_cast<f32x4*>(mine + ((h * T::DT + dt) * 4 + j4) * 256 + lane * 4) = v;
          }
        if (hf == 0) {
          mine[T::MACC + (h * 32 + l32) * 2] = mw[h];
          mine[T::MACC + (h * 32 + l32) * 2 + 1] = lrow[h];
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if (h >= nh) break;
        const float* const st0 = grp + T::MACC + (h * 32 + l32) * 2;  // (m, l) of partner 0
        float M = -INFINITY;
        for (int o = 0; o < WK; ++o) M = fmaxf(M, st0[o * T::MSLOT]);
        const float Mr = M == -INFINITY ? 0.f : M;
        float Lsum = 0.f;
        for (int o = 0; o < WK; ++o) Lsum += st0[o * T::MSLOT + 1] * __builtin_amdgcn_exp2f(st0[o * T::MSLOT] - Mr);
        for (int dt = wk; dt < T::DT; dt += WK) {
          f32x16 a;
#pragma unroll
          for (int j = 0; j < 16; ++j) a[j] = 0.f;
          for (int o = 0; o < WK; ++o) {
            const float w = __builtin_amdgcn_exp2f(st0[o * T::MSLOT] - Mr);
            const float* const src = grp + o * T::MSLOT + ((h * T::DT + dt) * 4) * 256 + lane * 4;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
              const f32x4 v = *reinterpret_cast<const f32x4*>(src + j4 * 256);
#pragma unroll
              for (int t = 0; t < 4; ++t) a[4 * j4 + t] += v[t] * w;
            }
          }
          emit(h, dt, a, M, Lsum, dt == 0);
        }
      }
    }
  }
  if (T::NW == 8 && wave < 4) __builtin_amdgcn_s_setprio(0);
}

}  // namespace
}  // namespace pkv
