// kernels.hip — gfx950 kernels of the low-rank draft LM head.
//
// Stages ("EAGLE-4", section "Retrieve vocabulary candidates cheaply, then
// score them exactly"):
//   down_kernel     z = Q . h, stored rounded in the weight dtype (MFMA)
//   select_kernel   s = P . z over a slice of the vocabulary, fused with the
//                   selection of the slice's k best ids (MFMA + wave-wide
//                   bitonic merges); s never goes to memory. With (W, h) in
//                   place of (P, z) it is the full-head baseline.
//   merge_kernel    per row, the k best of all slices' lists
//   rescore_kernel  exact logits W[id] . h of the selected ids (gather-GEMV)
//   dense_kernel    all V logits W . h (test aid)
#include "device.h"
#include "launch.h"

namespace lrh {

constexpr int kTile = 16;            // MFMA tile edge
constexpr int kWaves = 4;            // waves per block
constexpr int kBufCap = 64;          // candidate buffer per column
constexpr int kMergeAt = kBufCap - kTile;  // one tile adds <= 16 per column

// ------------------------------------------------------------ down-projection
// Block: 16 rows of Q x 16 rows of H; the 4 waves split d and add up in LDS.
template <typename T>
__global__ void __launch_bounds__(256) down_kernel(const T* __restrict__ Q, const T* __restrict__ H,
                                                   int r, int d, int64_t B, T* __restrict__ Z) {
  __shared__ f32x4 red[kWaves][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int j0 = blockIdx.x * kTile;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int qrow = j0 + col;
  const int64_t hrow = b0 + col;
  const bool q_ok = qrow < r, h_ok = hrow < B;
  // k range of this wave, a multiple of 32 elements
  const int per = ((d + kWaves - 1) / kWaves + 31) / 32 * 32;
  const int kb = min(d, wave * per), ke = min(d, kb + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = tile_dot(Q + (int64_t)(q_ok ? qrow : 0) * d + kb, q_ok, H + (h_ok ? hrow : 0) * (int64_t)d + kb,
                 h_ok, ke - kb, acc);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w][lane];
    // lane holds z for row b0 + col, components j0 + 4g .. j0 + 4g + 3
    if (h_ok) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 4 * g + q;
        if (j < r) Z[hrow * r + j] = store_cast<T>(sum[q]);
      }
    }
  }
}

// -------------------------------------------------- score pass + selection
struct WaveSel {
  float ls[kTile][kWave];   // best-so-far list per column, sorted
  int li[kTile][kWave];
  float bs[kTile][kBufCap]; // candidates that beat the column's k-th
  int bi[kTile][kBufCap];
  int cnt[kTile];
};

// Folds column n's buffer into its list and refreshes that column's k-th.
__device__ __forceinline__ void fold_column(WaveSel& st, int n, int k, float& thr_s, int& thr_i) {
  const int lane = threadIdx.x & 63;
  const int c = st.cnt[n];
  float s = neg_inf();
  int i = kSentinelId;
  if (lane < c) {
    s = st.bs[n][lane];
    i = st.bi[n][lane];
  }
  bitonic_sort_desc(s, i);
  merge_reversed(s, i, st.ls[n][kWave - 1 - lane], st.li[n][kWave - 1 - lane]);
  st.ls[n][lane] = s;
  st.li[n][lane] = i;
  if (lane == 0) st.cnt[n] = 0;
  const float ks = __shfl(s, k - 1);
  const int ki = __shfl(i, k - 1);
  if ((lane & 15) == n) {
    thr_s = ks;
    thr_i = ki;
  }
}

// Grid: (n_vsplit, ceil(B/16)). Block (split, bt) handles rows b0..b0+15 and
// the split's contiguous run of 16-row vocabulary tiles; wave w takes tiles
// w, w+4, ... Each wave keeps its own per-column list; the four are merged
// at the end and the k best go to part_[row][split].
template <typename T>
__global__ void __launch_bounds__(256) select_kernel(const T* __restrict__ M, const T* __restrict__ X,
                                                     int64_t V, int K, int64_t B, int k, int n_vsplit,
                                                     float* __restrict__ part_s, int* __restrict__ part_i) {
  __shared__ WaveSel sel[kWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  WaveSel& st = sel[wave];
  const int split = blockIdx.x;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int64_t ntiles = (V + kTile - 1) / kTile;
  const int64_t t_lo = ntiles * split / n_vsplit;
  const int64_t t_hi = ntiles * (split + 1) / n_vsplit;

#pragma unroll
  for (int n = 0; n < kTile; ++n) {
    st.ls[n][lane] = neg_inf();
    st.li[n][lane] = kSentinelId;
  }
  if (lane < kTile) st.cnt[lane] = 0;
  float thr_s = neg_inf();
  int thr_i = kSentinelId;

  const int col = lane & 15, g = lane >> 4;
  const int64_t xrow = b0 + col;
  const bool x_ok = xrow < B;
  const T* xp = X + (x_ok ? xrow : 0) * (int64_t)K;

  for (int64_t t = t_lo + wave; t < t_hi; t += kWaves) {
    const int64_t mrow = t * kTile + col;
    const bool m_ok = mrow < V;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = tile_dot(M + (m_ok ? mrow : 0) * (int64_t)K, m_ok, xp, x_ok, K, acc);
    // lane: row xrow, vocabulary ids t*16 + 4g + q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t v = t * kTile + 4 * g + q;
      if (x_ok && v < V && precedes(acc[q], (int)v, thr_s, thr_i)) {
        const int p = atomicAdd(&st.cnt[col], 1);
        st.bs[col][p] = acc[q];
        st.bi[col][p] = (int)v;
      }
    }
    const int c = lane < kTile ? st.cnt[lane] : 0;
    unsigned long long need = __ballot(c > kMergeAt);
    while (need) {
      const int n = __builtin_ctzll(need);
      need &= need - 1;
      fold_column(st, n, k, thr_s, thr_i);
    }
  }
  {
    const int c = lane < kTile ? st.cnt[lane] : 0;
    unsigned long long need = __ballot(c > 0);
    while (need) {
      const int n = __builtin_ctzll(need);
      need &= need - 1;
      fold_column(st, n, k, thr_s, thr_i);
    }
  }
  __syncthreads();
  // wave w combines columns 4w .. 4w+3 over the four waves' lists
#pragma unroll 1
  for (int q = 0; q < 4; ++q) {
    const int n = wave * 4 + q;
    if (b0 + n >= B) break;
    float s = sel[0].ls[n][lane];
    int i = sel[0].li[n][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
      merge_reversed(s, i, sel[w].ls[n][kWave - 1 - lane], sel[w].li[n][kWave - 1 - lane]);
    if (lane < k) {
      const int64_t o = ((b0 + n) * n_vsplit + split) * k + lane;
      part_s[o] = s;
      part_i[o] = i;
    }
  }
}

// ------------------------------------------------------------------ merge
// One block per row; each wave folds every 4th slice list into its own
// running list, then wave 0 folds the other three.
__global__ void __launch_bounds__(256) merge_kernel(const float* __restrict__ part_s,
                                                    const int* __restrict__ part_i, int n_parts, int k,
                                                    int32_t* __restrict__ idx, float* __restrict__ score) {
  __shared__ float cs[kWaves][kWave];
  __shared__ int ci[kWaves][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = blockIdx.x;
  float s = neg_inf();
  int i = kSentinelId;
  const int j = kWave - 1 - lane;  // reversed read: worst first
  for (int p = wave; p < n_parts; p += kWaves) {
    const int64_t o = (b * n_parts + p) * k;
    float os = neg_inf();
    int oi = kSentinelId;
    if (j < k) {
      os = part_s[o + j];
      oi = part_i[o + j];
    }
    merge_reversed(s, i, os, oi);
  }
  cs[wave][lane] = s;
  ci[wave][lane] = i;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kWaves; ++w) merge_reversed(s, i, cs[w][kWave - 1 - lane], ci[w][kWave - 1 - lane]);
    if (lane < k) {
      idx[b * k + lane] = i;
      if (score) score[b * k + lane] = s;
    }
  }
}

// ---------------------------------------------------------------- rescoring
// One wave per (row, candidate): the W row (d elements) is read with
// contiguous 16-byte loads, 1 KiB per wave instruction.
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 h, float acc, uint16_t) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__uint_as_float(w[q] << 16), __uint_as_float(h[q] << 16), acc);
    acc = fmaf(__uint_as_float(w[q] & 0xffff0000u), __uint_as_float(h[q] & 0xffff0000u), acc);
  }
  return acc;
}
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 h, float acc, float) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(w[q]), __uint_as_float(h[q]), acc);
  return acc;
}

template <typename T>
__global__ void __launch_bounds__(256) rescore_kernel(const T* __restrict__ W, const T* __restrict__ H,
                                                      const int32_t* __restrict__ idx, int64_t npairs,
                                                      int k, int64_t V, int d, float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * kWaves + wave;
  if (pair >= npairs) return;
  const int64_t b = pair / k;
  const int32_t v = idx[pair];
  if (v < 0 || v >= V) {
    if (lane == 0) logits[pair] = __builtin_nanf("");
    return;
  }
  constexpr int per = 16 / sizeof(T);  // elements per 16-byte load
  const T* w = W + (int64_t)v * d;
  const T* h = H + b * (int64_t)d;
  float acc = 0.f;
  for (int c = lane * per; c < d; c += kWave * per) acc = dot_chunk(load16(w + c), load16(h + c), acc, T());
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) logits[pair] = acc;
}

// ------------------------------------------------------------ dense logits
template <typename T>
__global__ void __launch_bounds__(256) dense_kernel(const T* __restrict__ W, const T* __restrict__ H,
                                                    int64_t V, int d, int64_t B, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int64_t ntiles = (V + kTile - 1) / kTile;
  if (t >= ntiles) return;
  const int64_t wrow = t * kTile + col, hrow = b0 + col;
  const bool w_ok = wrow < V, h_ok = hrow < B;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = tile_dot(W + (w_ok ? wrow : 0) * (int64_t)d, w_ok, H + (h_ok ? hrow : 0) * (int64_t)d, h_ok, d, acc);
  if (!h_ok) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t v = t * kTile + 4 * g + q;
    if (v < V) out[hrow * V + v] = acc[q];
  }
}

// ================================================================ launchers

int plan_vsplit(int64_t B, int64_t V) {
  const int64_t btiles = (B + kTile - 1) / kTile;
  const int64_t vtiles = (V + kTile - 1) / kTile;
  int64_t n = (512 + btiles - 1) / btiles;          // about 512 blocks in flight
  const int64_t cap = vtiles / kWaves > 0 ? vtiles / kWaves : 1;  // >= 1 tile per wave
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  return (int)n;
}

#define LRH_DISPATCH(dtype, body)         \
  do {                                    \
    if ((dtype) == 0) {                   \
      using T = uint16_t;                 \
      body;                               \
    } else {                              \
      using T = float;                    \
      body;                               \
    }                                     \
  } while (0)

hipError_t launch_down(int dtype, const void* Q, const void* H, int r, int d, int64_t B, void* Z,
                       hipStream_t stream) {
  dim3 grid((r + kTile - 1) / kTile, (unsigned)((B + kTile - 1) / kTile));
  LRH_DISPATCH(dtype, hipLaunchKernelGGL(down_kernel<T>, grid, dim3(256), 0, stream, (const T*)Q, (const T*)H,
                                         r, d, B, (T*)Z));
  return hipGetLastError();
}

hipError_t launch_select(int dtype, const void* M, const void* X, int64_t V, int K, int64_t B, int k,
                         int n_vsplit, float* part_s, int* part_i, hipStream_t stream) {
  dim3 grid(n_vsplit, (unsigned)((B + kTile - 1) / kTile));
  LRH_DISPATCH(dtype, hipLaunchKernelGGL(select_kernel<T>, grid, dim3(256), 0, stream, (const T*)M,
                                         (const T*)X, V, K, B, k, n_vsplit, part_s, part_i));
  return hipGetLastError();
}

hipError_t launch_merge(const float* part_s, const int* part_i, int n_parts, int64_t B, int k, int32_t* idx,
                        float* score, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)B), dim3(256), 0, stream, part_s, part_i, n_parts, k, idx,
                     score);
  return hipGetLastError();
}

hipError_t launch_rescore(int dtype, const void* W, const void* H, const int32_t* idx, int64_t B, int k,
                          int64_t V, int d, float* logits, hipStream_t stream) {
  const int64_t npairs = B * k;
  dim3 grid((unsigned)((npairs + kWaves - 1) / kWaves));
  LRH_DISPATCH(dtype, hipLaunchKernelGGL(rescore_kernel<T>, grid, dim3(256), 0, stream, (const T*)W,
                                         (const T*)H, idx, npairs, k, V, d, logits));
  return hipGetLastError();
}

hipError_t launch_dense(int dtype, const void* W, const void* H, int64_t V, int d, int64_t B, float* logits,
                        hipStream_t stream) {
  const int64_t ntiles = (V + kTile - 1) / kTile;
  dim3 grid((unsigned)((ntiles + kWaves - 1) / kWaves), (unsigned)((B + kTile - 1) / kTile));
  LRH_DISPATCH(dtype, hipLaunchKernelGGL(dense_kernel<T>, grid, dim3(256), 0, stream, (const T*)W, (const T*)H,
                                         V, d, B, logits));
  return hipGetLastError();
}

}  // namespace lrh
