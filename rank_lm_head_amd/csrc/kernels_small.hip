// kernels_small.hip — the head for a few rows, bf16: draft calls with B <= 8,
// the full-head baseline with B <= 4.
//
// With one to eight rows both contractions are matrix-vector products and
// the time is HBM streaming ("EAGLE-4", section "Retrieve vocabulary
// candidates cheaply, then score them exactly": the low-rank head still
// scores every vocabulary row, so P is read once per call). The effort goes
// to the memory side (large loads, several in flight per wave). The
// arithmetic is still not free: widening every bf16 element and
// multiplying it once per row on the vector ALU made the 8-row score pass
// take 22 us against about 10 for its bytes. So with 2 to 8 rows and r >= 32
// the scores come from the matrix cores (stream_scores_mfma: half of each
// 16-column tile idle at 8 rows, which costs nothing here); one row, and
// the full-head rows, stay on the vector ALU. (The one-row pass on the
// matrix cores measured slower, 18.7 against 17.3 us per call at r = 128:
// its operand tiles turn each 1 KiB wave load into 16 pieces of 64 bytes,
// and with one row the pass is bound by the memory side alone.)
//
//   select_short_kernel s = P . z with the fused k-best of each block's
//                       slice, for r <= 512 (a power of two)
//   select_long_kernel  the same for rows longer than one wave load (the
//                       full-head baseline, W . h)
// z = Q . h comes from down_wide_kernel (kernels_b1.hip). The slice lists are
// merged, and the winners rescored, by merge_kernel; one-row calls take the
// fused pass of kernels_b1.hip instead.
#include "launch.h"
#include "stream.h"
#include "topk.h"

namespace lrh {

constexpr int kWavesSmall = 4;
constexpr int kSmallThreads = kWavesSmall * kWave;

// ------------------------------------------------- shared tail of the pass
// Each wave hands its per-row lists to LDS; wave b merges the four lists of
// row b and writes the block's sorted list: entry j to part_[b][j][block].
template <int NB>
struct SmallLds {
  float bs[kWavesSmall][NB][kBuf];
  int bi[kWavesSmall][NB][kBuf];
  float cs[kWavesSmall][NB][kWave];
  int ci[kWavesSmall][NB][kWave];
};

template <int NB>
__device__ __forceinline__ void finish_block(SmallLds<NB>& sm, WaveSel<NB>& st, int B, int k,
                                             float* __restrict__ part_s, int* __restrict__ part_i) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int nblk = gridDim.x;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= B) break;
    if (st.cnt[b] > 0) st.fold(b, sm.bs[wave][b], sm.bi[wave][b], k);
    sm.cs[wave][b][lane] = st.ls[b];
    sm.ci[wave][b][lane] = st.li[b];
  }
  __syncthreads();
  if (wave < B) {
    const int b = wave;
    float s = sm.cs[0][b][lane];
    int i = sm.ci[0][b][lane];
#pragma unroll
    for (int w = 1; w < kWavesSmall; ++w)
      merge_reversed(s, i, sm.cs[w][b][kWave - 1 - lane], sm.ci[w][b][kWave - 1 - lane]);
    if (lane < k) {
      const int64_t o = ((int64_t)b * k + lane) * nblk + blockIdx.x;
      part_s[o] = s;
      part_i[o] = i;
    }
  }
}

// ------------------------------------------- score pass, rows <= 512 long
// K/8 lanes hold one vocabulary row (16 bytes each), so one wave load is 1
// KiB of consecutive rows. Block x owns the contiguous slice
// [V*x/n, V*(x+1)/n) (at most kBlockRows rows) and each wave a quarter of
// it; the next U wave loads are issued before the current ones are used.
// The scores go to LDS. After the pass wave b writes the L best of the
// slice for row b, in order, entry j to part_[b][j][x] (depth-major, so that
// the leading entries of all lists are contiguous for the merge), while the
// other waves copy the scores to raw[b][v] (coalesced). L is small (min(4, k)): the
// merge needs more of a slice only when its L-th entry still reaches the
// merge's bound, and then reads the slice's raw scores.
constexpr int kBlockRows = 512;

template <int K, int NB, int E>
__global__ void __launch_bounds__(kSmallThreads) select_short_kernel(
    const uint16_t* __restrict__ M, const uint16_t* __restrict__ X, int64_t V, int B, int L,
    float* __restrict__ part_s, int* __restrict__ part_i, float* __restrict__ raw) {
  __shared__ float sc[NB][E * kWave];
  const int wave = wave_id(), lane = threadIdx.x & 63;

  // slice bounds V*x/n in 32 bits: this path keeps V*n below 2^27
  const int64_t nblk = gridDim.x;
  const uint32_t v32 = (uint32_t)V, n32 = gridDim.x;
  const int64_t blo = v32 * blockIdx.x / n32, bhi = v32 * (blockIdx.x + 1) / n32;
  const int64_t wlo = blo + (bhi - blo) * wave / kWavesSmall;
  const int64_t whi = blo + (bhi - blo) * (wave + 1) / kWavesSmall;
  if constexpr (NB >= 2 && K >= 32)
    stream_scores_mfma<K, NB>(M, X, B, blo, wlo, whi, &sc[0][0], E * kWave);
  else
    stream_scores<K, NB>(M, X, B, blo, wlo, whi, &sc[0][0], E * kWave);
  __syncthreads();
  const int nrows = (int)(bhi - blo);
  if (B < kWavesSmall) {
    // wave b selects for row b; the waves without a row copy every row's
    // raw scores
    if (wave < B) {
      const int64_t o = (int64_t)wave * L * nblk + blockIdx.x;
      wave_top_few<E>(sc[wave], nrows, (int)blo, L, part_s + o, part_i + o, nblk);
    } else {
      const int t0 = (wave - B) * kWave + lane, step = (kWavesSmall - B) * kWave;
      for (int b = 0; b < B; ++b)
        for (int j = t0; j < nrows; j += step) raw[(int64_t)b * V + blo + j] = sc[b][j];
    }
  } else {
    // wave w takes rows w, w + 4: the selection, then the raw copy
    for (int b = wave; b < B; b += kWavesSmall) {
      const int64_t o = (int64_t)b * L * nblk + blockIdx.x;
      wave_top_few<E>(sc[b], nrows, (int)blo, L, part_s + o, part_i + o, nblk);
      for (int j = lane; j < nrows; j += kWave) raw[(int64_t)b * V + blo + j] = sc[b][j];
    }
  }
}

// -------------------------------------------- score pass, long rows (W . h)
// One vocabulary row at a time per wave: NL wave loads of 1 KiB (K <= NL *
// 512), the next row's loads issued before the current row is reduced. The
// rows of H sit in LDS. Loads past K read a clamped address and are zeroed.
template <int NB, int NL>
__global__ void __launch_bounds__(kSmallThreads) select_long_kernel(
    const uint16_t* __restrict__ M, const uint16_t* __restrict__ X, int64_t V, int K, int B, int k,
    float* __restrict__ part_s, int* __restrict__ part_i) {
  __shared__ SmallLds<NB> sm;
  __shared__ u32x4 xs[NB][NL * kWave];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  for (int e = threadIdx.x; e < NB * NL * kWave; e += kSmallThreads) {
    const int b = e / (NL * kWave), rem = e - b * NL * kWave;
    const int col = rem * 8;
    xs[b][rem] = (b < B && col < K) ? load16(X + (int64_t)b * K + col) : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // slice bounds V*x/n in 32 bits: this path keeps V*n below 2^27
  const uint32_t v32 = (uint32_t)V, n32 = gridDim.x;
  const int64_t blo = v32 * blockIdx.x / n32, bhi = v32 * (blockIdx.x + 1) / n32;
  const int64_t wlo = blo + (bhi - blo) * wave / kWavesSmall;
  const int64_t whi = blo + (bhi - blo) * (wave + 1) / kWavesSmall;
  const int64_t last = whi - 1;

  WaveSel<NB> st;
  st.init();
  u32x4 cur[NL], nxt[NL];
  int cols[NL];
#pragma unroll
  for (int t = 0; t < NL; ++t) {
    const int col = (t * kWave + lane) * 8;
    cols[t] = col < K ? col : K - 8;
  }
  if (wlo < whi) {
#pragma unroll
    for (int t = 0; t < NL; ++t) cur[t] = load16(M + wlo * K + cols[t]);
  }
  for (int64_t row = wlo; row < whi; ++row) {
    const int64_t nr = row + 1 < last ? row + 1 : last;
#pragma unroll
    for (int t = 0; t < NL; ++t) nxt[t] = load16(M + nr * K + cols[t]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b >= B) break;
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < NL; ++t) acc = dot8_bf16(cur[t], xs[b][t * kWave + lane], acc);
      const float s = group_sum<kWave>(acc);
      const bool pass = lane == 0 && precedes(s, (int)row, st.ts[b], st.ti[b]);
      st.push(b, pass, s, (int)row, sm.bs[wave][b], sm.bi[wave][b]);
      if (st.cnt[b] >= kBuf) st.fold(b, sm.bs[wave][b], sm.bi[wave][b], k);
    }
#pragma unroll
    for (int t = 0; t < NL; ++t) cur[t] = nxt[t];
  }
  finish_block<NB>(sm, st, B, k, part_s, part_i);
}

// ================================================================ launchers

constexpr int kMaxSmallBlocks = 512;

int small_blocks(int64_t V) {
  int64_t n = (V + 255) / 256;   // >= 64 rows per wave
  if (n > kMaxSmallBlocks) n = kMaxSmallBlocks;
  return (int)(n < 1 ? 1 : n);
}

bool small_path(int dtype, int64_t B, int64_t K_lowrank, int64_t V) {
  // (rank-512 rows of five to eight rows once took the matrix-core path:
  // 77 against 107 us per call for eight rows while this pass multiplied on
  // the vector ALU; on the matrix cores it is the faster one)
  if (dtype != 0 || B > kSmallB) return false;
  if (V > (int64_t)kMaxSmallBlocks * kBlockRows) return false;   // rows per block
  return K_lowrank >= 8 && K_lowrank <= 512 && (K_lowrank & (K_lowrank - 1)) == 0;
}

constexpr int kMaxRowLoads = 16;   // rows up to 8192 elements

bool small_long_path(int dtype, int64_t B, int64_t K, int64_t V) {
  return dtype == 0 && B <= kLongB && K <= kMaxRowLoads * kWave * 8 &&
         V <= (int64_t)kMaxSmallBlocks * kBlockRows;
}

// Wave loads (of 512 elements) per row, rounded up to an instantiated count.
static int row_loads(int K) {
  const int nl = (K + kWave * 8 - 1) / (kWave * 8);
  static const int kCounts[] = {1, 2, 4, 6, 8, 10, 12, 16};
  for (int c : kCounts)
    if (nl <= c) return c;
  return -1;
}

#define LRH_NL_DISPATCH(nl, body)       \
  do {                                  \
    switch (nl) {                       \
      case 1: { constexpr int NL = 1; body; } break;   \
      case 2: { constexpr int NL = 2; body; } break;   \
      case 4: { constexpr int NL = 4; body; } break;   \
      case 6: { constexpr int NL = 6; body; } break;   \
      case 8: { constexpr int NL = 8; body; } break;   \
      case 10: { constexpr int NL = 10; body; } break; \
      case 12: { constexpr int NL = 12; body; } break; \
      case 16: { constexpr int NL = 16; body; } break; \
      default: return hipErrorInvalidValue;            \
    }                                   \
  } while (0)

// Rows per launch, rounded up to an instantiated count: 1, 2, 4 (and 8 for
// the kernels that take eight rows).
#define LRH_NB4_DISPATCH(B, ...) \
  do {                           \
    if ((B) <= 1) {              \
      constexpr int NB = 1;      \
      __VA_ARGS__;               \
    } else if ((B) == 2) {       \
      constexpr int NB = 2;      \
      __VA_ARGS__;               \
    } else {                     \
      constexpr int NB = 4;      \
      __VA_ARGS__;               \
    }                            \
  } while (0)

#define LRH_NB_DISPATCH(B, ...)          \
  do {                                   \
    if ((B) <= kLongB) {                 \
      LRH_NB4_DISPATCH(B, __VA_ARGS__);  \
    } else {                             \
      constexpr int NB = 8;              \
      __VA_ARGS__;                       \
    }                                    \
  } while (0)

int small_list_len(int k) { return k < kSliceList ? k : kSliceList; }

template <int K>
static hipError_t launch_short_k(const void* M, const void* X, int64_t V, int64_t B, int k, float* ps, int* pi,
                                 float* raw, hipStream_t stream, Timing t) {
  const int nblk = small_blocks(V);
  dim3 grid(nblk);
  const int64_t rows = (V + nblk - 1) / nblk;   // most rows of one block
  const int L = small_list_len(k);
  if (B < 1 || B > kSmallB || rows > 8 * kWave || V * nblk >= (int64_t)1 << 32) return hipErrorInvalidValue;
  if (rows <= 4 * kWave) {
    LRH_NB_DISPATCH(B, LRH_LAUNCH(t, (select_short_kernel<K, NB, 4>), grid, dim3(kSmallThreads), 0, stream,
                                  (const uint16_t*)M, (const uint16_t*)X, V, (int)B, L, ps, pi, raw));
  } else if (rows <= 5 * kWave) {
    LRH_NB_DISPATCH(B, LRH_LAUNCH(t, (select_short_kernel<K, NB, 5>), grid, dim3(kSmallThreads), 0, stream,
                                  (const uint16_t*)M, (const uint16_t*)X, V, (int)B, L, ps, pi, raw));
  } else {
    LRH_NB_DISPATCH(B, LRH_LAUNCH(t, (select_short_kernel<K, NB, 8>), grid, dim3(kSmallThreads), 0, stream,
                                  (const uint16_t*)M, (const uint16_t*)X, V, (int)B, L, ps, pi, raw));
  }
  return hipGetLastError();
}

hipError_t launch_select_small(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* ps,
                               int* pi, float* raw, hipStream_t stream, Timing t) {
  switch (K) {
    case 8: return launch_short_k<8>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 16: return launch_short_k<16>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 32: return launch_short_k<32>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 64: return launch_short_k<64>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 128: return launch_short_k<128>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 256: return launch_short_k<256>(M, X, V, B, k, ps, pi, raw, stream, t);
    case 512: return launch_short_k<512>(M, X, V, B, k, ps, pi, raw, stream, t);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_select_long(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* ps,
                              int* pi, hipStream_t stream, Timing t) {
  if (B > kLongB || V > (int64_t)kMaxSmallBlocks * kBlockRows) return hipErrorInvalidValue;
  dim3 grid(small_blocks(V));
  const int nl = row_loads(K);
  LRH_NB4_DISPATCH(B, LRH_NL_DISPATCH(nl, LRH_LAUNCH(t, (select_long_kernel<NB, NL>), grid, dim3(kSmallThreads), 0,
                                                    stream, (const uint16_t*)M, (const uint16_t*)X, V, K, (int)B, k,
                                                    ps, pi)));
  return hipGetLastError();
}

}  // namespace lrh
