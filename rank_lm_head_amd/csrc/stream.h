// stream.h — the vocabulary score stream of the few-row paths.
//
// With a few draft rows, s[b][v] = P[v,:] . z_b is bound by reading P from
// HBM once ("EAGLE-4", section "Retrieve vocabulary candidates cheaply, then
// score them exactly": the low-rank head scores every vocabulary row). On
// the vector ALU (stream_scores) K/8 lanes hold one vocabulary row (16 bytes
// each), so one wave load is 1 KiB of consecutive rows; every wave keeps two
// groups of U loads in flight. On the matrix cores (stream_mfma_tiles) the
// rows go in 16-row tiles against up to four 16-row column tiles of z.
#pragma once

#include "device.h"

namespace lrh {

// Scores of rows [wlo, whi) of M (V x K, bf16) against the NB rows of X
// (B x K, bf16; rows past B score nothing) into sc[b * ldsc + (v - blo)].
// M is read once per call, with non-temporal loads.
// The z loads go first and are widened only after the first group of M
// loads is issued. Rows past the wave's range are loaded from its last row
// (a valid address, so no load is predicated) and never kept; a wave
// without rows loads row 0. The loop takes two groups per iteration with
// fixed buffers (no register copies, which would wait for the loads in
// flight); the last group prefetches nothing, so no load is outstanding
// when the function returns.
template <int K, int NB>
__device__ __forceinline__ void stream_scores(const uint16_t* __restrict__ M, const uint16_t* __restrict__ X,
                                              int B, int64_t blo, int64_t wlo, int64_t whi, float* sc,
                                              int ldsc) {
  constexpr int LPR = K / 8;
  constexpr int RPL = kWave / LPR;
  constexpr int U = 8;   // wave loads per group
  constexpr int STEP = U * RPL;
  static_assert(K % 8 == 0 && LPR <= kWave && (LPR & (LPR - 1)) == 0, "row length");
  const int lane = threadIdx.x & 63;
  const int c = lane % LPR, sub = lane / LPR;

  u32x4 zr[NB];
  f32x8 zc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) zr[b] = load16(X + (int64_t)(b < B ? b : 0) * K + 8 * c);

  const int64_t last = whi > 0 ? whi - 1 : 0;
  const int ng = wlo < whi ? (int)((whi - wlo + STEP - 1) / STEP) : 0;
  u32x4 buf0[U], buf1[U];
  auto issue = [&](u32x4 (&buf)[U], int64_t base) {
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int64_t row = base + t * RPL + sub;
      buf[t] = load16_stream(M + (row < last ? row : last) * K + 8 * c);
    }
  };
  auto consume = [&](const u32x4 (&buf)[U], int64_t base) {
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int64_t row = base + t * RPL + sub;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if (b >= B) break;
        const float s = group_sum<LPR>(dot8_bf16(buf[t], zc[b], 0.f));
        if (c == 0 && row < whi) sc[b * ldsc + (row - blo)] = s;
      }
    }
  };
  issue(buf0, wlo);   // unconditional: a branch here would make the first use wait for every load
  __builtin_amdgcn_sched_barrier(0);   // all of them before anything waits for z
#pragma unroll
  for (int b = 0; b < NB; ++b) zc[b] = widen8(b < B ? zr[b] : u32x4{0u, 0u, 0u, 0u});
  int g = 0;
  for (; g + 2 < ng; g += 2) {   // buf0 holds group g on entry
    const int64_t base = wlo + (int64_t)g * STEP;
    issue(buf1, base + STEP);
    consume(buf0, base);
    issue(buf0, base + 2 * STEP);
    consume(buf1, base + STEP);
  }
  if (g + 1 < ng) {
    const int64_t base = wlo + (int64_t)g * STEP;
    issue(buf1, base + STEP);
    consume(buf0, base);
    consume(buf1, base + STEP);
  } else if (g < ng) {
    consume(buf0, wlo + (int64_t)g * STEP);
  }
}

// The matrix-core tile stream over rows [wlo, whi) of M (V x K, bf16)
// against NT column tiles of X (16 rows each; rows past B are zeros). One
// v_mfma_f32_16x16x32_bf16 multiplies 16 rows of M by 16 rows of X over 32
// of K, so the vector ALU no longer widens and multiplies every element once
// per row. Lane l supplies row l & 15 of the 16-row tile and chunk l >> 4 (8
// elements) of each 32-deep step, the k steps accumulate in order from
// zero. For every 16-row tile the stream calls sink(base, acc) (base: the
// tile's first row, the same on all lanes): acc[c][q] is the score of M row
// base + 4 (l >> 4) + q against X row 16 c + (l & 15) (column tile c); rows
// at or past whi are the sink's to drop. X's fragments stay in registers for the whole pass.
// The tiles go in groups of TG, two groups of loads in flight
// (non-temporal); rows past the wave's range are loaded from its last row (a
// valid address, so no load is predicated), and the last group prefetches
// nothing, so no load is outstanding when the function returns.
//
// X's fragments come from xfrag(c, t) (the lane's 16 bytes of k step t of
// column tile c): stream_mfma_tiles keeps them in registers for the whole
// pass; stream_mfma_tiles_x takes any accessor (an LDS copy of X when its
// fragments would take too many registers: XMEM = true).
template <int K, int NT, int TG, bool XMEM = false, typename XFrag, typename Sink>
__device__ __forceinline__ void stream_mfma_tiles_x(const uint16_t* __restrict__ M, int64_t wlo, int64_t whi,
                                                    XFrag&& xfrag, Sink&& sink) {
  static_assert(K % 32 == 0 && NT >= 1 && NT <= 4, "k steps of 32, at most 64 rows of X");
  constexpr int KS = K / 32;   // k steps per tile
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  const int64_t last = whi > 0 ? whi - 1 : 0;
  const int ng = wlo < whi ? (int)((whi - wlo + 16 * TG - 1) / (16 * TG)) : 0;
  u32x4 buf0[TG][KS], buf1[TG][KS];
  auto issue = [&](u32x4 (&buf)[TG][KS], int64_t base) {
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      const int64_t row = base + u * 16 + col;
      const uint16_t* m = M + (row < last ? row : last) * K + g * 8;
#pragma unroll
      for (int t = 0; t < KS; ++t) buf[u][t] = load16_stream(m + t * 32);
    }
  };
  auto consume = [&](const u32x4 (&buf)[TG][KS], int64_t base) {
    // XMEM: xfrag reads memory that does not change; the empty asm keeps
    // those reads here, not hoisted out of the loop into registers
    if constexpr (XMEM) asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      f32x4 acc[NT];
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KS; ++t)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[u][t]),
                                                           __builtin_bit_cast(bf16x8, xfrag(c, t)), acc[c], 0, 0,
                                                           0);
      }
      sink(base + u * 16, acc);
    }
  };
  issue(buf0, wlo);
  int gi = 0;
  for (; gi + 2 < ng; gi += 2) {   // buf0 holds group gi on entry
    const int64_t base = wlo + (int64_t)gi * 16 * TG;
    issue(buf1, base + 16 * TG);
    consume(buf0, base);
    issue(buf0, base + 32 * TG);
    consume(buf1, base + 16 * TG);
  }
  if (gi + 1 < ng) {
    const int64_t base = wlo + (int64_t)gi * 16 * TG;
    issue(buf1, base + 16 * TG);
    consume(buf0, base);
    consume(buf1, base + 16 * TG);
  } else if (gi < ng) {
    consume(buf0, wlo + (int64_t)gi * 16 * TG);
  }
}

template <int K, int NT, int TG, typename Sink>
__device__ __forceinline__ void stream_mfma_tiles(const uint16_t* __restrict__ M, const uint16_t* __restrict__ X,
                                                  int B, int64_t wlo, int64_t whi, Sink&& sink) {
  constexpr int KS = K / 32;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  u32x4 xb[NT][KS];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      const int b = c * 16 + col;
      xb[c][t] = b < B ? load16(X + (int64_t)b * K + t * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  stream_mfma_tiles_x<K, NT, TG>(M, wlo, whi, [&](int c, int t) { return xb[c][t]; }, sink);
}

// The scores of stream_scores on the matrix cores, for 2 to 16 rows (K >=
// 32): one column tile of X, groups of about 8 wave loads, every score of a
// row of X below B to sc[b * ldsc + (v - blo)].
template <int K, int NB>
__device__ __forceinline__ void stream_scores_mfma(const uint16_t* __restrict__ M, const uint16_t* __restrict__ X,
                                                   int B, int64_t blo, int64_t wlo, int64_t whi, float* sc,
                                                   int ldsc) {
  static_assert(NB <= 16, "one column tile");
  constexpr int KS = K / 32;
  constexpr int TG = KS >= 8 ? 1 : 8 / KS;   // tiles per group
  const int col = threadIdx.x & 15, g = (threadIdx.x & 63) >> 4;
  const int BB = B < NB ? B : NB;
  stream_mfma_tiles<K, 1, TG>(M, X, BB, wlo, whi, [&](int64_t base, const f32x4 (&acc)[1]) {
    if (col < BB) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = base + 4 * g + q;
        if (row < whi) sc[col * ldsc + (row - blo)] = acc[0][q];
      }
    }
  });
}

}  // namespace lrh
