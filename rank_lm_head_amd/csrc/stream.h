// stream.h — the vocabulary score stream of the few-row (vector ALU) path.
//
// With one to eight draft rows, s[b][v] = P[v,:] . z_b is a matrix-vector
// product bound by reading P from HBM once ("EAGLE-4", section "Retrieve
// vocabulary candidates cheaply, then score them exactly": the low-rank
// head scores every vocabulary row). K/8 lanes hold one vocabulary row (16
// bytes each), so one wave load is 1 KiB of consecutive rows; every wave
// keeps two groups of U loads in flight.
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

// The same scores on the matrix cores, for 2 to 8 rows (K >= 32): one
// v_mfma_f32_16x16x32_bf16 multiplies 16 rows of M by the rows of X (padded
// to 16 with zeros) over 32 of K, so the vector ALU no longer widens and
// multiplies every element once per row. Lane l supplies row l & 15 of the
// 16-row tile and chunk l >> 4 (8 elements) of each 32-deep step; output q
// of lane l is the score of tile row 4 (l >> 4) + q for row l & 15 of X.
// X's fragments stay in registers for the whole pass. The wave's rows go in
// tiles of 16, two groups of about 8 wave loads in flight (non-temporal);
// rows past the wave's range are loaded from its last row and never kept.
template <int K, int NB>
__device__ __forceinline__ void stream_scores_mfma(const uint16_t* __restrict__ M, const uint16_t* __restrict__ X,
                                                   int B, int64_t blo, int64_t wlo, int64_t whi, float* sc,
                                                   int ldsc) {
  static_assert(K % 32 == 0 && NB <= 16, "k steps of 32, at most 16 rows of X");
  constexpr int KS = K / 32;                         // k steps per tile
  constexpr int TG = KS >= 8 ? 1 : 8 / KS;           // tiles per group
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  u32x4 xb[KS];
#pragma unroll
  for (int t = 0; t < KS; ++t)
    xb[t] = col < B && col < NB ? load16(X + (int64_t)col * K + t * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
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
#pragma unroll
    for (int u = 0; u < TG; ++u) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < KS; ++t)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, buf[u][t]),
                                                      __builtin_bit_cast(bf16x8, xb[t]), acc, 0, 0, 0);
      if (col < B && col < NB) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t row = base + u * 16 + 4 * g + q;
          if (row < whi) sc[col * ldsc + (row - blo)] = acc[q];
        }
      }
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

}  // namespace lrh
