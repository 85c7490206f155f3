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

}  // namespace lrh
