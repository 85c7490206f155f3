// kernels_mfma.hip — the head on the matrix cores, for row batches (B > 4)
// and for fp32 weights.
//
// With many draft rows both contractions of "EAGLE-4" (section "Retrieve
// vocabulary candidates cheaply, then score them exactly") are matrix
// products: Z[B x r] = H . Q^T and S[B x V] = Z . P^T. They run as 16x16
// MFMA tiles (bf16 16x16x32 or fp32 16x16x4, fp32 accumulation), with the
// vocabulary as the tile's row dimension and the draft rows as its column
// dimension; S never goes to memory: each tile is filtered against its
// columns' running k-th best as soon as it leaves the matrix cores.
//
//   down_mfma_kernel    Z = H . Q^T, stored rounded in the weight dtype
//   select_mfma_kernel  per vocabulary slice, the k best of each draft row
//   dense_kernel        all V logits W . h (test aid)
// The slice lists are merged (and rescored) by merge_kernel.
#include "launch.h"
#include "topk.h"

namespace lrh {

constexpr int kTile = 16;
constexpr int kWaves = 4;
constexpr int kMergeAt = kBuf - kTile;   // one tile adds <= 16 per column
constexpr int kUnroll = 8;               // k steps whose loads are issued together

// Loads of operand rows for kUnroll k steps starting at k0. `p` is a valid
// row (callers clamp missing rows); columns past K read a clamped address
// and are zeroed, so no load is predicated and all of them are in flight
// together.
template <typename T>
__device__ __forceinline__ void load_steps(const T* __restrict__ p, bool ok, int K, int k0, u32x4* v) {
  constexpr int step = sizeof(T) == 2 ? 32 : 16;
  constexpr int per = 16 / sizeof(T);
  const int g = (threadIdx.x & 63) >> 4;
  u32x4 x[kUnroll];
#pragma unroll
  for (int t = 0; t < kUnroll; ++t) {
    const int kk = k0 + t * step + g * per;
    x[t] = load16(p + (kk < K ? kk : K - per));
  }
#pragma unroll
  for (int t = 0; t < kUnroll; ++t) {
    const int kk = k0 + t * step + g * per;
    v[t] = (ok && kk < K) ? x[t] : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ f32x4 mfma_step(u32x4 a, u32x4 b, f32x4 acc, uint16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(u32x4 a, u32x4 b, f32x4 acc, float) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc, 0, 0, 0);
  return acc;
}

// acc += A_rows . B_rows^T over [0, K): 16x16 tile, lane's own rows at a / b.
template <typename T>
__device__ __forceinline__ f32x4 tile_dot_unrolled(const T* __restrict__ a, bool a_ok, const T* __restrict__ b,
                                                   bool b_ok, int K, f32x4 acc) {
  constexpr int step = sizeof(T) == 2 ? 32 : 16;
  for (int k0 = 0; k0 < K; k0 += kUnroll * step) {
    u32x4 va[kUnroll], vb[kUnroll];
    load_steps<T>(a, a_ok, K, k0, va);
    load_steps<T>(b, b_ok, K, k0, vb);
#pragma unroll
    for (int t = 0; t < kUnroll; ++t) acc = mfma_step(va[t], vb[t], acc, T());
  }
  return acc;
}

// ------------------------------------------------------------ down-projection
// Block: 16 rows of Q x 16 rows of H; NW waves split d and add up in LDS
// (16 waves for long rows, so that each wave's loads are few round trips).
template <typename T, int NW>
__global__ void __launch_bounds__(NW * 64) down_mfma_kernel(const T* __restrict__ Q, const T* __restrict__ H, int r,
                                                            int d, int64_t B, T* __restrict__ Z) {
  __shared__ f32x4 red[NW][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int j0 = blockIdx.x * kTile;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int qrow = j0 + col;
  const int64_t hrow = b0 + col;
  const bool q_ok = qrow < r, h_ok = hrow < B;
  const int per = ((d + NW - 1) / NW + 31) / 32 * 32;
  const int kb = min(d, wave * per), ke = min(d, kb + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = tile_dot_unrolled<T>(Q + (int64_t)(q_ok ? qrow : 0) * d + kb, q_ok,
                             H + (h_ok ? hrow : 0) * (int64_t)d + kb, h_ok, ke - kb, acc);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) sum += red[w][lane];
    if (h_ok) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 4 * g + q;
        if (j < r) Z[hrow * r + j] = store_cast<T>(sum[q]);
      }
    }
  }
}

// ------------------------------------------- split-K down-projection
// For row batches the down-projection has few 16x16 output tiles (r/16 x
// B/16) and a long K = d, so it is split over K across blocks: wave w of
// block (x, y, kz) takes columns [(4 kz + w) * 128, +128) of its tile, the
// four waves add up in LDS, and wave 0 writes the fp32 partial tile to
// part[kz][b][j]. down_reduce_kernel then adds the partials of every z
// component in kz order (a fixed order, so repeated calls agree bit for
// bit) and rounds the sum to bf16.
constexpr int kDownChunk = 128;   // K columns per wave

__global__ void __launch_bounds__(256) down_split_kernel(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ H, int r, int d, int64_t B,
                                                         float* __restrict__ part) {
  __shared__ f32x4 red[4][kWave];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int j0 = blockIdx.x * kTile;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int kz = blockIdx.z;
  const int qrow = j0 + col;
  const int64_t hrow = b0 + col;
  const bool q_ok = qrow < r, h_ok = hrow < B;
  const int kb = min(d, (kz * 4 + wave) * kDownChunk), ke = min(d, kb + kDownChunk);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (ke > kb)
    acc = tile_dot_unrolled<uint16_t>(Q + (int64_t)(q_ok ? qrow : 0) * d + kb, q_ok,
                                      H + (h_ok ? hrow : 0) * (int64_t)d + kb, h_ok, ke - kb, acc);
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && h_ok) {
    const f32x4 sum = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = j0 + 4 * g + q;
      if (j < r) part[((int64_t)kz * B + hrow) * r + j] = sum[q];
    }
  }
}

// Z[i] = bf16(sum over kz of part[kz][i]) for the n = B * r components.
__global__ void __launch_bounds__(256) down_reduce_kernel(const float* __restrict__ part, int S, int64_t n,
                                                          uint16_t* __restrict__ Z) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // up to 16 parts per round, all loads in flight (clamped addresses), added
  // in kz order
  float s = 0.f;
  for (int kz = 0; kz < S; kz += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = part[(int64_t)min(kz + u, S - 1) * n + i];
#pragma unroll
    for (int u = 0; u < 16; ++u) s = kz + u < S ? s + v[u] : s;
  }
  Z[i] = f32_to_bf16(s);
}

// -------------------------------------------------- score pass + selection
// Per wave and per column (draft row) of its tile: a sorted list of the best
// 64 seen so far and a buffer of candidates that beat the column's k-th.
struct TileSel {
  float ls[kTile][kWave];
  int li[kTile][kWave];
  float bs[kTile][kBuf];
  int bi[kTile][kBuf];
  int cnt[kTile];
};

__device__ __forceinline__ void fold_column(TileSel& st, int n, int k, float& thr_s, int& thr_i) {
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
// w, w+4, ... Each wave keeps its own per-column lists; the four are merged
// at the end and the k best go to part_[row][entry][split].
template <typename T>
__global__ void __launch_bounds__(256) select_mfma_kernel(const T* __restrict__ M, const T* __restrict__ X,
                                                          int64_t V, int K, int64_t B, int k, int n_vsplit,
                                                          float* __restrict__ part_s, int* __restrict__ part_i) {
  __shared__ TileSel sel[kWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  TileSel& st = sel[wave];
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
    acc = tile_dot_unrolled<T>(M + (m_ok ? mrow : 0) * (int64_t)K, m_ok, xp, x_ok, K, acc);
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
      const int64_t o = ((b0 + n) * k + lane) * n_vsplit + split;
      part_s[o] = s;
      part_i[o] = i;
    }
  }
}

// ------------------------------------------------------------ dense logits
template <typename T>
__global__ void __launch_bounds__(256) dense_kernel(const T* __restrict__ W, const T* __restrict__ H, int64_t V,
                                                    int d, int64_t B, float* __restrict__ out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, g = lane >> 4;
  const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t b0 = (int64_t)blockIdx.y * kTile;
  const int64_t ntiles = (V + kTile - 1) / kTile;
  if (t >= ntiles) return;
  const int64_t wrow = t * kTile + col, hrow = b0 + col;
  const bool w_ok = wrow < V, h_ok = hrow < B;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = tile_dot_unrolled<T>(W + (w_ok ? wrow : 0) * (int64_t)d, w_ok, H + (h_ok ? hrow : 0) * (int64_t)d, h_ok,
                             d, acc);
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
  int64_t n = (512 + btiles - 1) / btiles;
  const int64_t cap = vtiles / kWaves > 0 ? vtiles / kWaves : 1;
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  return (int)n;
}

#define LRH_DISPATCH(dtype, body) \
  do {                            \
    if ((dtype) == 0) {           \
      using T = uint16_t;         \
      body;                       \
    } else {                      \
      using T = float;            \
      body;                       \
    }                             \
  } while (0)

hipError_t launch_down(int dtype, const void* Q, const void* H, int r, int d, int64_t B, void* Z,
                       hipStream_t stream) {
  dim3 grid((r + kTile - 1) / kTile, (unsigned)((B + kTile - 1) / kTile));
  if (d >= 2048)
    LRH_DISPATCH(dtype, hipLaunchKernelGGL((down_mfma_kernel<T, 16>), grid, dim3(16 * 64), 0, stream, (const T*)Q,
                                           (const T*)H, r, d, B, (T*)Z));
  else
    LRH_DISPATCH(dtype, hipLaunchKernelGGL((down_mfma_kernel<T, 4>), grid, dim3(4 * 64), 0, stream, (const T*)Q,
                                           (const T*)H, r, d, B, (T*)Z));
  return hipGetLastError();
}

int down_split_parts(int d) { return ((d + kDownChunk - 1) / kDownChunk + 3) / 4; }

hipError_t launch_down_split(const void* Q, const void* H, int r, int d, int64_t B, void* Z, float* part,
                             hipStream_t stream) {
  const int S = down_split_parts(d);
  const dim3 grid((r + kTile - 1) / kTile, (unsigned)((B + kTile - 1) / kTile), (unsigned)S);
  hipLaunchKernelGGL(down_split_kernel, grid, dim3(256), 0, stream, (const uint16_t*)Q, (const uint16_t*)H, r, d, B,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = B * r;
  hipLaunchKernelGGL(down_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part, S, n,
                     (uint16_t*)Z);
  return hipGetLastError();
}

hipError_t launch_down_reduce(const float* part, int S, int64_t n, void* Z, hipStream_t stream) {
  hipLaunchKernelGGL(down_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part, S, n,
                     (uint16_t*)Z);
  return hipGetLastError();
}

hipError_t launch_select(int dtype, const void* M, const void* X, int64_t V, int K, int64_t B, int k,
                         int n_vsplit, float* part_s, int* part_i, hipStream_t stream, Timing t) {
  dim3 grid(n_vsplit, (unsigned)((B + kTile - 1) / kTile));
  LRH_DISPATCH(dtype, LRH_LAUNCH(t, select_mfma_kernel<T>, grid, dim3(256), 0, stream, (const T*)M, (const T*)X, V,
                                 K, B, k, n_vsplit, part_s, part_i));
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
