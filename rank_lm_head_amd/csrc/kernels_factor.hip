// kernels_factor.hip — building the low-rank head (P, Q) from W.
//
// The pages say token prediction is factored into smaller matrices ("EAGLE-4
// Triples Qwen3 Inference Speed by Adapting to Serving Load", section
// "Runtime-sized speculation") but not how the factors are made. This builds
// them from W by a randomized range finder with subspace iteration (Halko,
// Martinsson and Tropp's randomized low-rank approximation):
//
//   Y = orth(W . Omega);  q times: Z = orth(W^T . Y), Y = orth(W . Z);
//   P = Y (V x r, orthonormal columns),  Q = Y^T . W (r x d)
//
// so that P . Q is the projection of W onto the captured column space.
// orth() is CholeskyQR2: G = X^T X (accumulated in fp64), its Cholesky
// factor G = L L^T, X <- X L^-T, twice.
//
// The four W-sized products (W . Omega, W^T . Y, W . Z, W^T . Y) run on the
// bf16 matrix cores when V and d are multiples of 8 (the fp32 panel split
// into two bf16 halves, below); otherwise, and for the panel-sized products
// of the orthonormalisation, which need fp32 or fp64 operands, on the vector
// ALU:
//   fgemm_kernel    C = op(A) . B for 64 x 64 tiles of C, K in chunks of 16
//                   staged through LDS, 4 x 4 outputs per thread; A is W
//                   (bf16) or an fp32 panel, read as is (M x K) or transposed
//                   (stored K x M); long K runs as split-K partials
//   reduce_kernel   sums the split-K partials
//   chol_panel_kernel / chol_update_kernel
//                   blocked right-looking Cholesky of the n x n Gram matrix
//                   in fp64: per 32-column panel, its diagonal block
//                   factored in LDS, the rows below it solved one per thread,
//                   then the trailing lower triangle updated in 64 x 64 tiles
//   trinv_kernel    the rows of L^-T (= columns of L^-1), one wave per
//                   column, forward substitution, written as fp32
//   cast kernels    P and Q in bf16 (Q transposed from W^T . Y)
#include "launch.h"

namespace lrh {

namespace {

template <typename T>
__device__ __forceinline__ float ld_f32(const T* p);
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p) {
  return *p;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {   // round to nearest even (finite inputs)
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

constexpr int kTile = 64;
constexpr int kTk = 16;
constexpr int kGemmThreads = 256;

// Partial z of C (M x N, row-major) = op(A)[:, Kz] . B[Kz, :] with
// Kz = [z * kchunk, min(K, (z + 1) * kchunk)). op(A) is M x K: A itself
// (AT = false, A[m * lda + k]) or A transposed (AT = true, A[k * lda + m]).
// B is K x N row-major (B[k * ldb + n]). Out-of-range elements load as 0.
template <typename TA, bool AT, typename ACC>
__global__ void __launch_bounds__(kGemmThreads) fgemm_kernel(const TA* __restrict__ A, int64_t lda,
                                                             const float* __restrict__ Bm, int64_t ldb,
                                                             ACC* __restrict__ C, int M, int N, int64_t K,
                                                             int64_t kchunk) {
  __shared__ ACC As[kTk][kTile + 1];
  __shared__ ACC Bs[kTk][kTile + 1];
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int m0 = blockIdx.x * kTile, n0 = blockIdx.y * kTile;
  const int64_t kb = (int64_t)blockIdx.z * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  ACC acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += kTk) {
#pragma unroll
    for (int q = 0; q < kTile * kTk / kGemmThreads; ++q) {
      const int e = q * kGemmThreads + threadIdx.x;
      int kk, mm;
      if (AT) {
        kk = e / kTile;
        mm = e % kTile;
      } else {
        mm = e / kTk;
        kk = e % kTk;
      }
      const int64_t gk = k0 + kk;
      const int gm = m0 + mm;
      float v = 0.f;
      if (gk < ke && gm < M) v = ld_f32<TA>(AT ? A + gk * lda + gm : A + (int64_t)gm * lda + gk);
      As[kk][mm] = (ACC)v;
      const int kb2 = e / kTile, nn = e % kTile;
      const int64_t gk2 = k0 + kb2;
      const int gn = n0 + nn;
      Bs[kb2][nn] = (ACC)((gk2 < ke && gn < N) ? Bm[gk2 * ldb + gn] : 0.f);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTk; ++kk) {
      ACC a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  ACC* Cz = C + (int64_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) Cz[(int64_t)m * N + n] = acc[i][j];
    }
  }
}

// The same product for N >= 128 on 128 x 128 tiles of C: 8 x 8 outputs per
// thread (16 LDS reads per 64 multiply-adds instead of 8 per 16), and the
// operand tiles loaded 16 bytes at a time (8 bf16 or 4 fp32 elements of a
// contiguous run): op(A)'s run is along K (AT = false) or along M (AT =
// true), B's along N. Requires lda and ldb to be multiples of 8 (bf16) or 4
// (fp32) and 16-byte aligned rows; runs past the matrix are zero-filled.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBig = 128;
constexpr int kBigK = 16;
template <typename TA, bool AT, typename ACC>
__global__ void __launch_bounds__(kGemmThreads) fgemm_big_kernel(const TA* __restrict__ A, int64_t lda,
                                                                 const float* __restrict__ Bm, int64_t ldb,
                                                                 ACC* __restrict__ C, int M, int N, int64_t K,
                                                                 int64_t kchunk) {
  constexpr int PA = 16 / sizeof(TA);   // elements of A per 16-byte load
  __shared__ ACC As[kBigK][kBig + 4];
  __shared__ ACC Bs[kBigK][kBig + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;   // outputs rows ty * 8 + i, columns tx * 8 + j
  const int m0 = blockIdx.x * kBig, n0 = blockIdx.y * kBig;
  const int64_t kb = (int64_t)blockIdx.z * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  ACC acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0;
  for (int64_t k0 = kb; k0 < ke; k0 += kBigK) {
    // A tile: kBigK x kBig values of op(A)
    constexpr int NA = kBigK * kBig / PA / kGemmThreads;   // 16-byte loads per thread
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      const int e = q * kGemmThreads + tid;
      float v[PA];
      if (!AT) {   // run along K: row mm, columns kk .. kk + PA
        const int mm = e / (kBigK / PA), kk = (e % (kBigK / PA)) * PA;
        const int gm = m0 + mm;
        const int64_t gk = k0 + kk;
        if (gm < M && gk + PA <= ke) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(A + (int64_t)gm * lda + gk);
#pragma unroll
          for (int u = 0; u < PA; ++u) v[u] = sizeof(TA) == 2 ? __uint_as_float(u % 2 ? w[u / 2] & 0xFFFF0000u : w[u / 2] << 16)
                                                              : __uint_as_float(w[u]);
        } else {
#pragma unroll
          for (int u = 0; u < PA; ++u) v[u] = gm < M && gk + u < ke ? ld_f32<TA>(A + (int64_t)gm * lda + gk + u) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < PA; ++u) As[kk + u][mm] = (ACC)v[u];
      } else {     // run along M: row kk of the stored matrix, columns mm .. mm + PA
        const int kk = e / (kBig / PA), mm = (e % (kBig / PA)) * PA;
        const int64_t gk = k0 + kk;
        const int gm = m0 + mm;
        if (gk < ke && gm + PA <= M) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(A + gk * lda + gm);
#pragma unroll
          for (int u = 0; u < PA; ++u) v[u] = sizeof(TA) == 2 ? __uint_as_float(u % 2 ? w[u / 2] & 0xFFFF0000u : w[u / 2] << 16)
                                                              : __uint_as_float(w[u]);
        } else {
#pragma unroll
          for (int u = 0; u < PA; ++u) v[u] = gk < ke && gm + u < M ? ld_f32<TA>(A + gk * lda + gm + u) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < PA; ++u) As[kk][mm + u] = (ACC)v[u];
      }
    }
    // B tile: kBigK x kBig fp32, runs of 4 along N
    constexpr int NB = kBigK * kBig / 4 / kGemmThreads;
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int e = q * kGemmThreads + tid;
      const int kk = e / (kBig / 4), nn = (e % (kBig / 4)) * 4;
      const int64_t gk = k0 + kk;
      const int gn = n0 + nn;
      float v[4];
      if (gk < ke && gn + 4 <= N) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(Bm + gk * ldb + gn);
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __uint_as_float(w[u]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = gk < ke && gn + u < N ? Bm[gk * ldb + gn + u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) Bs[kk][nn + u] = (ACC)v[u];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBigK; ++kk) {
      ACC a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = As[kk][ty * 8 + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = Bs[kk][tx * 8 + j];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  ACC* Cz = C + (int64_t)blockIdx.z * M * N;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + ty * 8 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + tx * 8 + j;
      if (n < N) Cz[(int64_t)m * N + n] = acc[i][j];
    }
  }
}

// out[i] = sum over z < S of part[z * count + i]
template <typename ACC>
__global__ void __launch_bounds__(256) reduce_kernel(const ACC* __restrict__ part, int S, int64_t count,
                                                     ACC* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    ACC s = 0;
    for (int z = 0; z < S; ++z) s += part[(int64_t)z * count + i];
    out[i] = s;
  }
}

// In place, the lower triangle of G (n x n, row-major, symmetric) becomes L
// with G = L L^T, 32 columns at a time (right-looking, blocked):
//  chol_panel_kernel  every block copies the diagonal block G[k0.., k0..]
//                     (32 x 32) to LDS and factors it there, one column per
//                     step (pivot, scale the column, update the trailing
//                     triangle); block 0 writes it back. Then each thread
//                     takes one row i below the block and solves
//                     x . L11^T = G[i, k0..] by forward substitution, with
//                     the row in registers;
//  chol_update_kernel G[i, c] -= sum_l L[i, k0 + l] L[c, k0 + l] for the
//                     trailing rows and columns c <= i, one 64 x 64 tile of
//                     the lower triangle per block, 4 x 4 outputs per thread.
// A pivot that is not positive (a rank-deficient panel) is replaced by a tiny
// one and counted in *status.
constexpr int kCholMax = 512;
constexpr int kCholNb = 32;
constexpr int kCholRows = 256;   // rows below the diagonal block per panel block
constexpr int kCholTile = 64;

__global__ void __launch_bounds__(kCholRows) chol_panel_kernel(double* __restrict__ G, int n, int k0,
                                                               uint32_t* __restrict__ status) {
  __shared__ double a[kCholNb][kCholNb + 1];
  const int tid = threadIdx.x;
  const int nb = min(kCholNb, n - k0);
  for (int t = tid; t < nb * nb; t += kCholRows) {
    const int i = t / nb, c = t % nb;
    a[i][c] = c <= i ? G[(int64_t)(k0 + i) * n + k0 + c] : 0.0;
  }
  __syncthreads();
  for (int j = 0; j < nb; ++j) {
    double d = a[j][j];
    if (!(d > 0.0)) {
      if (blockIdx.x == 0 && tid == 0) atomicAdd(status, 1u);
      d = 1e-300;
    }
    const double piv = sqrt(d);
    __syncthreads();   // every thread has read the old diagonal
    if (tid == 0) a[j][j] = piv;
    if (tid > j && tid < nb) a[tid][j] /= piv;
    __syncthreads();
    const int m = nb - j - 1;
    for (int t = tid; t < m * m; t += kCholRows) {
      const int i = j + 1 + t / m, c = j + 1 + t % m;
      if (c <= i) a[i][c] -= a[i][j] * a[c][j];
    }
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int t = tid; t < nb * nb; t += kCholRows) {
      const int i = t / nb, c = t % nb;
      if (c <= i) G[(int64_t)(k0 + i) * n + k0 + c] = a[i][c];
    }
  const int i = k0 + nb + blockIdx.x * kCholRows + tid;
  if (i >= n) return;
  double x[kCholNb];
  double* row = G + (int64_t)i * n + k0;
#pragma unroll
  for (int j = 0; j < kCholNb; ++j) x[j] = j < nb ? row[j] : 0.0;
#pragma unroll
  for (int j = 0; j < kCholNb; ++j) {
    if (j < nb) {
      double s = x[j];
#pragma unroll
      for (int l = 0; l < j; ++l) s -= x[l] * a[j][l];
      x[j] = s / a[j][j];
    }
  }
#pragma unroll
  for (int j = 0; j < kCholNb; ++j)
    if (j < nb) row[j] = x[j];
}

__global__ void __launch_bounds__(256) chol_update_kernel(double* __restrict__ G, int n, int k0) {
  __shared__ double li[kCholTile][kCholNb + 1], lc[kCholTile][kCholNb + 1];
  const int r0 = k0 + kCholNb;   // first trailing row and column
  // block -> tile (ti, tc) of the lower triangle, tc <= ti
  int ti = 0, rem = blockIdx.x;
  while (rem > ti) {
    rem -= ti + 1;
    ++ti;
  }
  const int tc = rem;
  const int i0 = r0 + ti * kCholTile, c0 = r0 + tc * kCholTile;
  const int tid = threadIdx.x;
  for (int t = tid; t < kCholTile * kCholNb; t += 256) {
    const int rr = t / kCholNb, l = t % kCholNb;
    li[rr][l] = i0 + rr < n ? G[(int64_t)(i0 + rr) * n + k0 + l] : 0.0;
    lc[rr][l] = c0 + rr < n ? G[(int64_t)(c0 + rr) * n + k0 + l] : 0.0;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;   // rows ty + 16 u, columns tx + 16 v
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
#pragma unroll 8
  for (int l = 0; l < kCholNb; ++l) {
    double xa[4], xb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) xa[u] = li[ty + 16 * u][l];
#pragma unroll
    for (int v = 0; v < 4; ++v) xb[v] = lc[tx + 16 * v][l];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] += xa[u] * xb[v];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + ty + 16 * u, c = c0 + tx + 16 * v;
      if (i < n && c <= i) G[(int64_t)i * n + c] -= acc[u][v];
    }
}

hipError_t cholesky(double* G, int n, uint32_t* status, hipStream_t s) {
  for (int k0 = 0; k0 < n; k0 += kCholNb) {
    const int below = n - k0 - kCholNb;
    const int blocks = below > 0 ? (below + kCholRows - 1) / kCholRows : 1;
    hipLaunchKernelGGL(chol_panel_kernel, dim3((unsigned)blocks), dim3(kCholRows), 0, s, G, n, k0, status);
    if (below > 0) {
      const int T = (below + kCholTile - 1) / kCholTile;
      hipLaunchKernelGGL(chol_update_kernel, dim3((unsigned)(T * (T + 1) / 2)), dim3(256), 0, s, G, n, k0);
    }
  }
  return hipGetLastError();
}

// Rinv = L^-T (fp32), n x n row-major. Wave c solves L x = e_c by forward
// substitution (x is column c of L^-1, i.e. row c of L^-T): x_c = 1 / L_cc,
// then for each i > c the dot product of row i of L with x so far, taken by
// the whole wave (lanes stride over j) and reduced by DPP and two shuffles;
// x is kept in fp64 in LDS.
constexpr int kInvWaves = 4;
constexpr int kInvMax = 512;
__global__ void __launch_bounds__(kInvWaves * 64) trinv_kernel(const double* __restrict__ L, int n,
                                                               float* __restrict__ Rinv) {
  __shared__ double xs[kInvWaves][kInvMax];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kInvWaves + wave;
  if (c >= n) return;   // whole waves
  double* x = xs[wave];
  float* row = Rinv + (int64_t)c * n;
  for (int i = lane; i < c; i += 64) row[i] = 0.f;
  const double xc = 1.0 / L[(int64_t)c * n + c];
  if (lane == 0) x[c] = xc;
  if (lane == 0) row[c] = (float)xc;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int i = c + 1; i < n; ++i) {
    const double* Li = L + (int64_t)i * n;
    double s = 0.0;
    for (int j = c + lane; j < i; j += 64) s += Li[j] * x[j];
    // wave sum in fp64 by butterfly shuffles
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const double xi = -s / Li[i];
    if (lane == 0) {
      x[i] = xi;
      row[i] = (float)xi;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

__global__ void zero_kernel(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

// P = bf16(Y) (V x r); Q[i][j] = bf16(Z[j][i]) (Z: d x r, Q: r x d)
__global__ void __launch_bounds__(256) cast_p_kernel(const float* __restrict__ Y, int64_t n, uint16_t* __restrict__ P) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    P[i] = to_bf16(Y[i]);
}
__global__ void __launch_bounds__(256) cast_q_kernel(const float* __restrict__ Z, int d, int r,
                                                     uint16_t* __restrict__ Q) {
  const int64_t n = (int64_t)d * r;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n; t += (int64_t)gridDim.x * 256) {
    const int i = (int)(t / d), j = (int)(t % d);   // Q[i][j], coalesced writes
    Q[t] = to_bf16(Z[(int64_t)j * r + i]);
  }
}

// ------------------------------------------------ matrix-core W products
// With V and d multiples of 8 the four W-sized products run on the bf16
// matrix cores (launch_gemm_f32): the fp32 panel B (K x r) is split into two
// bf16 halves, hi = bf16(B) and lo = bf16(B - hi) (together within 2^-17 of
// B), and W . B = W . hi + W . lo is one product with 2r rows, accumulated
// in fp32. The GEMM wants both operands K-contiguous, so the panel goes in
// transposed (2r x K) and W^T . Y takes W transposed (d x V, once per build).

// At (cols x rows) = A^T for A (rows x cols, bf16; rows and cols multiples
// of 8): 64 x 64 tiles through LDS, 16-byte loads and stores.
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const uint16_t* __restrict__ A, int64_t rows,
                                                             int64_t cols, uint16_t* __restrict__ At) {
  __shared__ uint16_t t[64][64 + 2];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // 512 chunks of 8 per tile
    const int e = h * 256 + tid, i = e >> 3, j = (e & 7) * 8;
    const int64_t row = r0 + i, c = c0 + j;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows && c < cols) v = *reinterpret_cast<const u32x4*>(A + row * cols + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      t[i][j + 2 * q] = (uint16_t)(v[q] & 0xFFFFu);
      t[i][j + 2 * q + 1] = (uint16_t)(v[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = h * 256 + tid, a = e >> 3, b = (e & 7) * 8;   // At row c0 + a, columns r0 + b ..
    const int64_t orow = c0 + a, ocol = r0 + b;
    if (orow < cols && ocol < rows) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (uint32_t)t[b + 2 * q][a] | ((uint32_t)t[b + 2 * q + 1][a] << 16);
      *reinterpret_cast<u32x4*>(At + orow * rows + ocol) = v;
    }
  }
}

// out (2r x rows, bf16): out[n][k] = hi(X[k][n]), out[r + n][k] = lo(X[k][n])
// for the fp32 panel X (rows x r); 64 x 64 tiles through LDS.
__global__ void __launch_bounds__(256) split_t_kernel(const float* __restrict__ X, int64_t rows, int r,
                                                      uint16_t* __restrict__ out) {
  __shared__ float t[64][65];
  const int64_t k0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    const int e = h * 256 + tid, kl = e >> 6, nl = e & 63;
    const int64_t k = k0 + kl;
    const int n = n0 + nl;
    t[kl][nl] = k < rows && n < r ? X[k * r + n] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    const int e = h * 256 + tid, nl = e >> 6, kl = e & 63;
    const int64_t k = k0 + kl;
    const int n = n0 + nl;
    if (k < rows && n < r) {
      const float x = t[kl][nl];
      const uint16_t hi = to_bf16(x);
      const uint16_t lo = to_bf16(x - __uint_as_float((uint32_t)hi << 16));
      out[(int64_t)n * rows + k] = hi;
      out[(int64_t)(r + n) * rows + k] = lo;
    }
  }
}

// out (M x r, fp32): out[m][n] = sum over the parts p, in order, of
// S[p][n][m] + S[p][r + n][m] (S: parts x 2r x M, the GEMM's partial
// products of the two halves); 64 x 64 tiles through LDS.
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ S, int parts, int r, int64_t M,
                                                      float* __restrict__ out) {
  __shared__ float t[64][65];
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int64_t plane = 2 * (int64_t)r * M;
#pragma unroll 4
  for (int h = 0; h < 16; ++h) {
    const int e = h * 256 + tid, nl = e >> 6, ml = e & 63;
    const int64_t m = m0 + ml;
    const int n = n0 + nl;
    float acc = 0.f;
    if (m < M && n < r) {
      for (int p = 0; p < parts; ++p) {
        const float* sp = S + p * plane;
        acc += sp[(int64_t)n * M + m] + sp[(int64_t)(r + n) * M + m];
      }
    }
    t[nl][ml] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    const int e = h * 256 + tid, ml = e >> 6, nl = e & 63;
    const int64_t m = m0 + ml;
    const int n = n0 + nl;
    if (m < M && n < r) out[m * r + n] = t[nl][ml];
  }
}

// K splits of the W^T . Y product (M = d rows of W^T, K = V): about 512
// blocks of the GEMM, at least 4 stages of 64 each.
int wt_splits(int64_t V, int64_t d, int r) {
  const int64_t bn = 2 * r > 128 ? 256 : 2 * r > 64 ? 128 : 64;
  const int64_t nt = (2 * r + bn - 1) / bn;
  int64_t nvb = (d + 255) / 256;
  if (nvb >= 8) nvb = (nvb + 7) / 8 * 8;
  const int64_t tiles = nvb * nt;
  int64_t s = (512 + tiles - 1) / tiles;
  const int64_t smax = std::max<int64_t>(1, (V + 63) / 64 / 4);
  return (int)std::min<int64_t>(std::min<int64_t>(s, smax), 64);
}

bool factor_on_mfma(int64_t V, int64_t d) { return V % 8 == 0 && d % 8 == 0; }

struct FactorWs {
  float* Y[2];      // V x r
  float* Z[2];      // d x r
  float* part;      // split-K partials (fp32), kSplitMax x max(V, d) x r ... sized below
  double* partd;    // split-K partials of Gram matrices (fp64)
  double* G;        // r x r
  float* Rinv;      // r x r
  uint32_t* status;
  // matrix-core products only
  uint16_t* Wt;     // d x V
  uint16_t* Xh;     // 2r x max(V, d): the panel's halves, transposed
  float* S;         // the GEMM's fp32 products: max(2r x V, splits x 2r x d)
};

constexpr int kSplitZ = 16;     // splits of K = V for W^T . Y

// Splits of a Gram matrix X^T X (r x r, K = rows): about 2048 blocks in all.
int gram_splits(int r) {
  const int tiles = ((r + kTile - 1) / kTile) * ((r + kTile - 1) / kTile);
  int s = 2048 / tiles;
  return s < 8 ? 8 : (s > 256 ? 256 : s);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t ws_layout(int64_t V, int64_t d, int r, FactorWs* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  FactorWs t;
  t.Y[0] = (float*)take((size_t)V * r * 4);
  t.Y[1] = (float*)take((size_t)V * r * 4);
  t.Z[0] = (float*)take((size_t)d * r * 4);
  t.Z[1] = (float*)take((size_t)d * r * 4);
  t.part = (float*)take((size_t)kSplitZ * d * r * 4);
  t.partd = (double*)take((size_t)gram_splits(r) * r * r * 8);
  t.G = (double*)take((size_t)r * r * 8);
  t.Rinv = (float*)take((size_t)r * r * 4);
  t.status = (uint32_t*)take(256);
  t.Wt = nullptr;
  t.Xh = nullptr;
  t.S = nullptr;
  if (factor_on_mfma(V, d)) {
    const int64_t mx = V > d ? V : d;
    t.Wt = (uint16_t*)take((size_t)d * V * 2);
    t.Xh = (uint16_t*)take((size_t)2 * r * mx * 2);
    const size_t s1 = (size_t)2 * r * V, s2 = (size_t)wt_splits(V, d, r) * 2 * r * d;
    t.S = (float*)take((s1 > s2 ? s1 : s2) * 4);
  }
  if (w) *w = t;
  return off;
}

template <typename TA, bool AT, typename ACC>
hipError_t gemm(const TA* A, int64_t lda, const float* B, int64_t ldb, ACC* C, int M, int N, int64_t K, int S,
                hipStream_t s) {
  const int64_t kchunk = ((K + S - 1) / S + kTk - 1) / kTk * kTk;
  const int Sz = (int)((K + kchunk - 1) / kchunk);
  constexpr int PA = 16 / sizeof(TA);
  const bool aligned = lda % PA == 0 && ldb % 4 == 0 && (reinterpret_cast<uintptr_t>(A) & 15u) == 0 &&
                       (reinterpret_cast<uintptr_t>(B) & 15u) == 0;
  if (N >= kBig && aligned) {
    dim3 grid((unsigned)((M + kBig - 1) / kBig), (unsigned)((N + kBig - 1) / kBig), (unsigned)Sz);
    hipLaunchKernelGGL((fgemm_big_kernel<TA, AT, ACC>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, C, M, N, K,
                       kchunk);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((M + kTile - 1) / kTile), (unsigned)((N + kTile - 1) / kTile), (unsigned)Sz);
  hipLaunchKernelGGL((fgemm_kernel<TA, AT, ACC>), grid, dim3(kGemmThreads), 0, s, A, lda, B, ldb, C, M, N, K, kchunk);
  return hipGetLastError();
}

int splits_for(int64_t K, int S) {
  const int64_t kchunk = ((K + S - 1) / S + kTk - 1) / kTk * kTk;
  return (int)((K + kchunk - 1) / kchunk);
}

#define LRH_F(x)                          \
  do {                                    \
    const hipError_t e_ = (x);            \
    if (e_ != hipSuccess) return e_;      \
  } while (0)

// X (rows x r, fp32) <- orth(X) by CholeskyQR2; X and T are the two buffers
// of the panel, the result ends in X.
hipError_t orth(float*& X, float*& T, int64_t rows, int r, const FactorWs& w, hipStream_t s) {
  for (int pass = 0; pass < 2; ++pass) {
    int S = (int)((rows + 255) / 256);
    if (S > gram_splits(r)) S = gram_splits(r);
    const int Sz = splits_for(rows, S);
    LRH_F((gemm<float, true, double>(X, r, X, r, w.partd, r, r, rows, S, s)));
    hipLaunchKernelGGL(reduce_kernel<double>, dim3((unsigned)(((int64_t)r * r + 255) / 256)), dim3(256), 0, s,
                       w.partd, Sz, (int64_t)r * r, w.G);
    LRH_F(hipGetLastError());
    LRH_F(cholesky(w.G, r, w.status, s));
    hipLaunchKernelGGL(trinv_kernel, dim3((unsigned)((r + kInvWaves - 1) / kInvWaves)), dim3(kInvWaves * 64), 0, s,
                       w.G, r, w.Rinv);
    LRH_F(hipGetLastError());
    // T = X . L^-T: (rows x r) . (r x r)
    LRH_F((gemm<float, false, float>(X, r, w.Rinv, r, T, (int)rows, r, r, 1, s)));
    float* t = X;
    X = T;
    T = t;
  }
  return hipSuccess;
}

// out (rows_out x r) = A . B on the matrix cores, A given as the bf16 matrix
// Am (rows_out x K, K-contiguous: W, or W^T for W^T . Y), B the fp32 panel
// (K x r): the panel's halves transposed, one GEMM over 2r rows (K split in
// `splits` parts), the parts and halves added in a fixed order.
hipError_t mfma_times(const uint16_t* Am, int64_t rows_out, int64_t K, int r, const float* B, float* out, int splits,
                      const FactorWs& w, hipStream_t s) {
  hipLaunchKernelGGL(split_t_kernel, dim3((unsigned)((K + 63) / 64), (unsigned)((r + 63) / 64)), dim3(256), 0, s, B,
                     K, r, w.Xh);
  LRH_F(hipGetLastError());
  LRH_F(launch_gemm_f32(Am, rows_out, (int)K, w.Xh, 2 * r, w.S, splits, s));
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows_out + 63) / 64), (unsigned)((r + 63) / 64)), dim3(256), 0,
                     s, w.S, splits, r, rows_out, out);
  return hipGetLastError();
}

// Y = W . B (V x r) for the panel B (d x r)
hipError_t w_times(const uint16_t* W, int64_t V, int64_t d, int r, const float* B, float* Y, const FactorWs& w,
                   hipStream_t s) {
  if (w.Wt) return mfma_times(W, V, d, r, B, Y, 1, w, s);
  return gemm<uint16_t, false, float>(W, d, B, r, Y, (int)V, r, d, 1, s);
}

// Z = W^T . Y (d x r), reduced into Zout
hipError_t wt_times(const uint16_t* W, int64_t V, int64_t d, int r, const float* Y, float* Zout, const FactorWs& w,
                    hipStream_t s) {
  if (w.Wt) return mfma_times(w.Wt, d, V, r, Y, Zout, wt_splits(V, d, r), w, s);
  const int Sz = splits_for(V, kSplitZ);
  LRH_F((gemm<uint16_t, true, float>(W, d, Y, r, w.part, (int)d, r, V, kSplitZ, s)));
  hipLaunchKernelGGL(reduce_kernel<float>, dim3((unsigned)((d * r + 255) / 256)), dim3(256), 0, s, w.part, Sz,
                     (int64_t)d * r, Zout);
  return hipGetLastError();
}

}  // namespace

size_t factor_workspace_bytes(int64_t V, int64_t d, int r) { return ws_layout(V, d, r, nullptr, nullptr); }

hipError_t launch_factor(const void* Wv, int64_t V, int64_t d, int r, int q, const float* omega, void* Pv, void* Qv,
                         void* workspace, hipStream_t s) {
  const uint16_t* W = static_cast<const uint16_t*>(Wv);
  if (r > kCholMax || r > kInvMax) return hipErrorInvalidValue;
  FactorWs w;
  ws_layout(V, d, r, &w, static_cast<char*>(workspace));
  hipLaunchKernelGGL(zero_kernel, dim3(1), dim3(64), 0, s, w.status, 1);
  LRH_F(hipGetLastError());
  float *Y = w.Y[0], *Yt = w.Y[1], *Z = w.Z[0], *Zt = w.Z[1];
  if (w.Wt) {   // W^T for the matrix-core W^T . Y
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)((d + 63) / 64), (unsigned)((V + 63) / 64)), dim3(256),
                       0, s, W, V, d, w.Wt);
    LRH_F(hipGetLastError());
  }
  // Y = orth(W . Omega)
  LRH_F(w_times(W, V, d, r, omega, Y, w, s));
  LRH_F(orth(Y, Yt, V, r, w, s));
  for (int it = 0; it < q; ++it) {
    LRH_F(wt_times(W, V, d, r, Y, Z, w, s));
    LRH_F(orth(Z, Zt, d, r, w, s));
    LRH_F(w_times(W, V, d, r, Z, Y, w, s));
    LRH_F(orth(Y, Yt, V, r, w, s));
  }
  // P = Y, Q = (W^T . Y)^T
  LRH_F(wt_times(W, V, d, r, Y, Z, w, s));
  hipLaunchKernelGGL(cast_p_kernel, dim3(2048), dim3(256), 0, s, Y, V * r, static_cast<uint16_t*>(Pv));
  LRH_F(hipGetLastError());
  hipLaunchKernelGGL(cast_q_kernel, dim3(2048), dim3(256), 0, s, Z, (int)d, r, static_cast<uint16_t*>(Qv));
  return hipGetLastError();
}

}  // namespace lrh
