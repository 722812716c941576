// Device helpers shared by the bf16 attention kernels (gfx950 only).  They live in an anonymous namespace,
// so every kernel source that includes them keeps its own copies.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))
#define CONST_AS __attribute__((address_space(4)))

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Slot of stage st in a four-slot LDS ring: the Gray code of st mod 4 (0, 1, 3, 2), so that the slots of
// consecutive stages differ in one bit.
__device__ __forceinline__ int ring_slot(int st) {
  const int r = st & 3;
  return r ^ (r >> 1);
}

// D[m][n] += sum_k A[m][k] B[k][n] over a 16x16x32 tile; lane l holds A[l%16][8(l/16) + 0..7],
// B[8(l/16) + 0..7][l%16] and D[4(l/16) + 0..3][l%16].
__device__ inline f32x4 mfma_qk(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same over a 32x32x16 tile (twice the sustained rate of the 16x16x32 form on MI355X); lane l holds
// A[l%32][8(l/32) + 0..7], B[8(l/32) + 0..7][l%32] and, in register j, D[8(j/4) + 4(l/32) + j%4][l%32].
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte HBM -> LDS copy per lane: lane l's 16 bytes from `src` land at LDS byte address
// lds_base + 16*l (lds_base uniform).  Issued as inline assembly so that the compiler's wait-count pass
// does not treat every later LDS read as dependent on it (it cannot tell ring slots apart and would drain
// all loads in flight); readiness of a slot is established explicitly with wait_vmem + a barrier.
// The copy is marked non-temporal: K/V are streamed once per (kv head, partition), and on MI355X the
// streaming policy raises the sustained HBM read rate of this access pattern by about 12%.
__device__ inline void dma16(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// The same copy with the default cache policy, for K/V that several row tiles read close together (long
// query chunks), so that L2 can serve the later reads.
__device__ inline void dma16_keep(const void* src, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}

// s_waitcnt on the vector-memory counter only: at most N vector memory operations still outstanding.
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Maximum over the four lanes l % 16 + 16 * {0, 1, 2, 3} (the lanes holding one row's scores): a swap of
// the wave halves, then of neighbouring 16-lane rows, each followed by a max of the two copies.
__device__ inline float row_max4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Maximum and sum of the values held by lanes l and l ^ 32.  The swap of the wave halves returns
// (v of lanes 0-31 in both halves, v of lanes 32-63 in both halves), so every lane sees both.
__device__ inline float pair_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ inline float pair_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// A row's reference maximum (log2 units) moves only when a chunk's maximum exceeds it by more than this,
// so probabilities stay below 2^kLazyRescale and the accumulator is rescaled rarely; acc, l and m stay
// mutually consistent, so the normalised result is unchanged.
constexpr float kLazyRescale = 8.f;

// 16-byte-chunk swizzle of LDS row `key`.
template <int D>
__device__ inline int k_swizzle(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

}  // namespace
}  // namespace pkv
