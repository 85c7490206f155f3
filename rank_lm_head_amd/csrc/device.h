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

// The wave's index in its block, as a wave-uniform (scalar) value, so that
// branches and loop bounds derived from it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
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

// A 16-byte load of data read once (a streamed weight matrix): non-temporal,
// so that it does not push code and reused data out of the caches.
__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
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
// Value of lane (l ^ S). Distances up to 8 stay inside a row of 16 lanes and
// use DPP, written only with direction-free patterns: quad permutes (1, 2),
// the half-row mirror followed by a quad reversal (4: lane i of a half row
// reads 7 - (3 - i) = i + 4, and the other way round), and a rotation of the
// row by 8. Distance 16 uses ds_swizzle (xor mask 16 within 32 lanes), 32 a
// ds_bpermute.
template <int S>
__device__ __forceinline__ int lane_xor(int x) {
  if constexpr (S == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, true);
  else if constexpr (S == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, true);
  else if constexpr (S == 4)
    return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, true), 0x1B, 0xf, 0xf, true);
  else if constexpr (S == 8) return __builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, true);
  else if constexpr (S == 16) return __builtin_amdgcn_ds_swizzle(x, 0x401F);
  else return __shfl_xor(x, 32);
}

template <int S>
__device__ __forceinline__ void cmpx(float& s, int& i, bool keep_better) {
  const float os = __int_as_float(lane_xor<S>(__float_as_int(s)));
  const int oi = lane_xor<S>(i);
  const bool other_first = precedes(os, oi, s, i);
  if (other_first == keep_better) {
    s = os;
    i = oi;
  }
}

// One merge step of a bitonic network: distance S inside blocks of SIZE.
template <int SIZE, int S>
__device__ __forceinline__ void bitonic_step(float& s, int& i, int lane) {
  const bool lower = (lane & S) == 0;
  const bool desc_block = SIZE >= kWave ? true : (lane & SIZE) == 0;
  cmpx<S>(s, i, lower == desc_block);
}

template <int SIZE>
__device__ __forceinline__ void bitonic_stage(float& s, int& i, int lane) {
  if constexpr (SIZE >= 64) bitonic_step<SIZE, 32>(s, i, lane);
  if constexpr (SIZE >= 32) bitonic_step<SIZE, 16>(s, i, lane);
  if constexpr (SIZE >= 16) bitonic_step<SIZE, 8>(s, i, lane);
  if constexpr (SIZE >= 8) bitonic_step<SIZE, 4>(s, i, lane);
  if constexpr (SIZE >= 4) bitonic_step<SIZE, 2>(s, i, lane);
  bitonic_step<SIZE, 1>(s, i, lane);
}

// Sorts the wave's 64 pairs into candidate order (best in lane 0).
__device__ __forceinline__ void bitonic_sort_desc(float& s, int& i) {
  const int lane = threadIdx.x & 63;
  bitonic_stage<2>(s, i, lane);
  bitonic_stage<4>(s, i, lane);
  bitonic_stage<8>(s, i, lane);
  bitonic_stage<16>(s, i, lane);
  bitonic_stage<32>(s, i, lane);
  bitonic_stage<64>(s, i, lane);
}

// Sorts a bitonic sequence of 64 pairs into candidate order.
__device__ __forceinline__ void bitonic_merge_desc(float& s, int& i) {
  bitonic_stage<64>(s, i, threadIdx.x & 63);
}

// (s, i) is sorted (best first) across the wave and (ts, ti) holds another
// sorted list *reversed* (worst first). Leaves in (s, i) the best 64 of the
// union, sorted.
__device__ __forceinline__ void merge_reversed(float& s, int& i, float ts, int ti) {
  if (precedes(ts, ti, s, i)) { s = ts; i = ti; }
  bitonic_merge_desc(s, i);
}

// ------------------------------------------------------------ lane groups
// Sum over aligned groups of N lanes (N a power of two <= 64); every lane of
// a group receives the group's sum. N <= 16 uses DPP within a row of 16
// lanes: quad permutes for distances 1 and 2, then the half-row and row
// mirrors (lane i with 7-i, and with 15-i), which pair lanes whose partial
// sums already cover disjoint halves.
template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), Ctrl, 0xf, 0xf, true));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
  if constexpr (N >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Dot product of 8 bf16 pairs (two 16-byte chunks) with fp32 accumulation.
// Each bf16 is widened exactly (it is the top half of an fp32 word) and the
// products are accumulated with fp32 FMAs in element order.
__device__ __forceinline__ float dot8_bf16(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__uint_as_float(a[q] << 16), __uint_as_float(b[q] << 16), acc);
    acc = fmaf(__uint_as_float(a[q] & 0xffff0000u), __uint_as_float(b[q] & 0xffff0000u), acc);
  }
  return acc;
}

// 8 bf16 widened to fp32, in element order.
struct f32x8 {
  float v[8];
};
__device__ __forceinline__ f32x8 widen8(u32x4 a) {
  f32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r.v[2 * q] = __uint_as_float(a[q] << 16);
    r.v[2 * q + 1] = __uint_as_float(a[q] & 0xffff0000u);
  }
  return r;
}

// Same sum as dot8_bf16 with the second operand already widened.
__device__ __forceinline__ float dot8_bf16(u32x4 a, const f32x8& b, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__uint_as_float(a[q] << 16), b.v[2 * q], acc);
    acc = fmaf(__uint_as_float(a[q] & 0xffff0000u), b.v[2 * q + 1], acc);
  }
  return acc;
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

}  // namespace lrh
