// device.h — gfx950 device primitives shared by the head's kernels.
//
// Element types: bf16 is carried as its 16-bit pattern (uint16_t) and fp32 as
// float. Every contraction accumulates in fp32 on the matrix cores:
//   bf16: v_mfma_f32_16x16x32_bf16 (16x16 output tile, 32-deep k step)
//   fp32: v_mfma_f32_16x16x4_f32   (16x16 output tile, 4-deep k step)
// In both, lane l supplies row (l & 15) of the left operand and row (l & 15)
// of the right operand (both are K-major, i.e. "NT"), for the k slots of
// group g = l >> 4; the 16x16 result holds, in lane l, column (l & 15) and
// rows 4*g .. 4*g+3. Because each group's k slots are summed, any fixed
// assignment of real k indices to (group, slot) gives the same dot product
// as long as both operands use it: here each lane reads 8 (bf16) or 4 (fp32)
// consecutive elements with one 16-byte load.
//
// Candidate order of the head ("EAGLE-4", section "Retrieve vocabulary
// candidates cheaply, then score them exactly", read as: the k best tokens,
// ties to the lower id): (s1, i1) precedes (s2, i2) when s1 > s2, or when
// s1 == s2 and i1 < i2. It is a total order on distinct ids, so every merge
// order yields the same list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrh {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kSentinelId = 0x7fffffff;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ T store_cast(float x);
template <> __device__ __forceinline__ uint16_t store_cast<uint16_t>(float x) { return f32_to_bf16(x); }
template <> __device__ __forceinline__ float store_cast<float>(float x) { return x; }

__device__ __forceinline__ bool precedes(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------- MFMA tile
// acc += A_rows . B_rows^T over [0, K) for one 16x16 tile. `a` and `b` point
// at the lane's own row (row l & 15 of each operand); a_ok / b_ok say whether
// that row exists (missing rows contribute zeros). K is a multiple of 8.
__device__ __forceinline__ f32x4 tile_dot(const uint16_t* __restrict__ a, bool a_ok,
                                          const uint16_t* __restrict__ b, bool b_ok,
                                          int K, f32x4 acc) {
  const int g = (threadIdx.x & 63) >> 4;
  for (int k0 = 0; k0 < K; k0 += 32) {
    const int kk = k0 + g * 8;
    u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (a_ok && kk < K) va = load16(a + kk);
    if (b_ok && kk < K) vb = load16(b + kk);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va),
                                                  __builtin_bit_cast(bf16x8, vb), acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ f32x4 tile_dot(const float* __restrict__ a, bool a_ok,
                                          const float* __restrict__ b, bool b_ok,
                                          int K, f32x4 acc) {
  const int g = (threadIdx.x & 63) >> 4;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int kk = k0 + g * 4;
    u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
    if (a_ok && kk < K) va = load16(a + kk);
    if (b_ok && kk < K) vb = load16(b + kk);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(va[j]), __uint_as_float(vb[j]),
                                                 acc, 0, 0, 0);
  }
  return acc;
}

// ------------------------------------------------------- wave-wide ordering
// One (score, id) pair per lane. After bitonic_sort_desc the 64 pairs are in
// candidate order across lanes 0..63 (best first).
__device__ __forceinline__ void cmpx(float& s, int& i, int stride, bool keep_better) {
  const float os = __shfl_xor(s, stride);
  const int oi = __shfl_xor(i, stride);
  const bool other_first = precedes(os, oi, s, i);
  if (other_first == keep_better) { s = os; i = oi; }
}

__device__ __forceinline__ void bitonic_sort_desc(float& s, int& i) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const bool lower = (lane & stride) == 0;
      const bool desc_block = (lane & size) == 0;
      cmpx(s, i, stride, lower == desc_block);
    }
  }
}

// Sorts a bitonic sequence of 64 pairs into candidate order.
__device__ __forceinline__ void bitonic_merge_desc(float& s, int& i) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int stride = kWave >> 1; stride > 0; stride >>= 1) cmpx(s, i, stride, (lane & stride) == 0);
}

// (s, i) is sorted (best first) across the wave and (ts, ti) holds another
// sorted list *reversed* (worst first). Leaves in (s, i) the best 64 of the
// union, sorted.
__device__ __forceinline__ void merge_reversed(float& s, int& i, float ts, int ti) {
  if (precedes(ts, ti, s, i)) { s = ts; i = ti; }
  bitonic_merge_desc(s, i);
}

}  // namespace lrh
