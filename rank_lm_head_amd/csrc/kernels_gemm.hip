// kernels_gemm.hip — the vocabulary pass on the matrix cores for row
// batches (bf16, B > 4): S = X . M^T with M = P (low-rank scores, K = r) or
// M = W (full-head logits, K = d), followed by an exact per-row top-k
// ("EAGLE-4", section "Retrieve vocabulary candidates cheaply, then score
// them exactly": the k best candidates of every draft row over the whole
// vocabulary).
//
// S is B x V and never stored whole. The selection uses a per-row bound:
//
//   1. Sample pass. The same GEMM over every `stride`-th block of vocabulary
//      rows keeps, per draft row, the maximum of each 32-row tile. The k-th
//      largest of those maxima, theta_b, is reached by at least k distinct
//      scores of row b (one per tile), so it is a lower bound of the row's
//      k-th best score.
//   2. Main pass. The GEMM over all vocabulary rows writes only the scores
//      that reach theta_b (a few hundred per row), each at its own column of
//      a sparse B x V score array, with a bit mask per 32 of them.
//   3. Collect. One block per row gathers the flagged scores and ranks the k
//      best (windowed bisection and counting ranks, topk.h); a row with more
//      than a buffer's worth of flagged scores (heavy ties) is taken in
//      rounds, so the result is exact in every case.
//
// Both passes compute every 16x16 tile with the same MFMA sequence (same
// operands, same k order), so the bound of the sample pass holds bit for bit
// in the main pass.
//
// GEMM layout: a block computes a BM x BN tile of S^T (BM vocabulary rows x
// BN draft rows) with 4 waves in a WM x WN grid; K advances in stages of 64
// bf16 copied from global memory straight into LDS (three stage buffers: two
// stages in flight while the third feeds the matrix cores). In LDS each row
// of a stage is 8 chunks of 16 bytes, chunk c of row r stored at position
// c ^ (r & 7), so the 16-byte fragment reads of eight consecutive rows hit
// distinct banks.
// Blocks are numbered so that the BN-tiles of one vocabulary block run on the
// same XCD (consecutive workgroup ids go to consecutive XCDs), which keeps
// the shared M tile in that XCD's L2.
#include "launch.h"
#include "topk.h"

namespace lrh {

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;                  // K elements per LDS stage
constexpr int kRowChunks = kBK / 8;      // 16-byte chunks per row per stage
constexpr int kXcds = 8;
constexpr int kMaxSampleTiles = 2048;    // tile maxima per row kept by the sample pass

template <int BM_, int BN_, int WM_, int WN_, int ST_ = 3>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int ST = ST_;                     // LDS stage buffers (ST - 1 stages in flight)
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave tile
  static constexpr int FM = TM / 16, FN = TN / 16;   // 16x16 tiles per wave
  static constexpr int A_LD = BM * kRowChunks / kGemmThreads;
  static constexpr int B_LD = BN * kRowChunks / kGemmThreads;
  static_assert(WM * WN == 4, "four waves");
  static_assert(FM * 4 <= 32, "a wave's rows of one column fit a 32-bit mask per lane group");
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for the loaders");
};

enum { kModeMax = 0, kModeFilter = 1, kModeStore = 2, kModePartial = 3 };

__device__ __forceinline__ int swz(int row, int c) { return row * kRowChunks + (c ^ (row & 7)); }

// Operand rows [row0, row0 + rows) of a row-major bf16 matrix with K
// columns, copied stage by stage (64 columns) from global memory straight
// into LDS (buffer loads with the LDS as destination, 16 bytes per lane).
// One such load of a wave fills 1 KiB of LDS, lane l the l-th 16 bytes,
// i.e. 8 rows of the stage; lane l therefore fetches chunk
// (l % 8) ^ (row & 7) of its row so that the swizzled layout comes out.
// Rows past the matrix and columns past K get an offset beyond the
// resource's size and read as zeros. Flags: raw (untyped) dword access.
constexpr int kRawBufferFlags = 0x00020000;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The wave's index in the block, as a value the compiler knows to be
// uniform (it feeds the LDS destination register of the copies).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

template <int LD>
struct StageDma {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[LD];   // byte offset of the lane's chunk in stage 0
  int col[LD];        // first column of the lane's chunk in stage 0
  uint32_t oob;       // an offset past the resource

  // The resource covers the block's own tile_rows rows from row0 (fewer at
  // the matrix's end): at most 256 rows of at most 65536 columns, 32 MiB,
  // so its 32-bit size cannot wrap however large the matrix is.
  __device__ __forceinline__ void init(const uint16_t* __restrict__ base, int64_t row0, int64_t nrows, int K,
                                       int tile_rows) {
    const int64_t valid = min(nrows - row0, (int64_t)tile_rows);   // >= 1
    const uint32_t bytes = uniform_u32((uint32_t)(valid * K * 2));
    const uint64_t addr = reinterpret_cast<uint64_t>(base + row0 * (int64_t)K);
    const uint64_t ua = ((uint64_t)uniform_u32((uint32_t)(addr >> 32)) << 32) | uniform_u32((uint32_t)addr);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ua), (short)0, (int)bytes, kRawBufferFlags);
    oob = bytes;
    const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int row = (i * 4 + wave) * 8 + lane / 8;
      const int c = (lane % 8) ^ (row & 7);
      col[i] = c * 8;
      off[i] = row < valid ? (uint32_t)(row * K + c * 8) * 2u : oob;
    }
  }

  // Wave w's loads of stage kc into `stage` (LDS, BM or BN rows x 128 B).
  __device__ __forceinline__ void issue(u32x4* stage, int kc, int K, bool tail) const {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const uint32_t o = (tail && kc * kBK + col[i] >= K) ? oob : off[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(stage + (i * 4 + wave) * kWave), 16, (int)o,
                                               kc * kBK * 2, 0, 0);
    }
  }
};

// A block barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the stage copies still in flight (the explicit
// wait_vmcnt before it decides which of those must have landed).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS reads are done
  asm volatile("s_barrier" ::: "memory");
}

// Waits until at most N of this wave's vector memory operations are
// outstanding (s_waitcnt vmcnt(N), the other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ float fmax_lanes(float m) {
  m = fmaxf(m, __int_as_float(lane_xor<16>(__float_as_int(m))));
  m = fmaxf(m, __int_as_float(lane_xor<32>(__float_as_int(m))));
  return m;
}

// Grid: 1-D, round_up(nvb, 8) * ceil(B / BN) blocks (see the XCD mapping
// above); nvb vocabulary blocks of BM rows, the s-th being block s * stride.
//  kModeMax:    aux_f = tile maxima, row n at aux_f + n * ns_tiles, tile
//               index s * (BM/32) + (32-row tile within the block).
//  kModeFilter: theta = per-row bound; S = sparse scores (row n at
//               S + n * ldS); mask = per row NW words, word
//               ((vb * WM + wm) * 4 + g) holds bit (i * 4 + q) for vocabulary
//               row (vb * WM + wm) * TM + i * 16 + 4 * g + q.
template <class C, int MODE>
__global__ void __launch_bounds__(kGemmThreads) gemm_sel_kernel(
    const uint16_t* __restrict__ M, const uint16_t* __restrict__ X, int64_t V, int K, int64_t B, int nvb,
    int stride, float* __restrict__ aux_f, int ns_tiles, const float* __restrict__ theta, float* __restrict__ S,
    int64_t ldS, uint32_t* __restrict__ mask, int NW) {
  extern __shared__ u32x4 lds[];
  constexpr int SA = C::BM * kRowChunks, SB = C::BN * kRowChunks;   // 16-byte chunks per stage
  // K stages [kb, kb + nk) of the nk_all: all of them, or with kModePartial
  // the blockIdx.y-th of gridDim.y equal shares
  const int nk_all = (K + kBK - 1) / kBK;
  const int kb = MODE == kModePartial ? (int)((int64_t)nk_all * blockIdx.y / gridDim.y) : 0;
  const int nk = MODE == kModePartial ? (int)((int64_t)nk_all * (blockIdx.y + 1) / gridDim.y) - kb : nk_all;
  const int nbuf = max(1, min(C::ST, nk));   // stage buffers (fewer for short K)
  u32x4* As = lds;                  // [nbuf][SA]
  u32x4* Bs = lds + nbuf * SA;      // [nbuf][SB]

  const int NT = (int)((B + C::BN - 1) / C::BN);
  const int L = blockIdx.x;
  int vb_local, nt;
  if (nvb >= kXcds) {
    const int xcd = L % kXcds, j = L / kXcds;
    vb_local = (j / NT) * kXcds + xcd;
    nt = j % NT;
  } else {   // too few vocabulary blocks to spread over the XCDs
    vb_local = L / NT;
    nt = L % NT;
  }
  if (vb_local >= nvb) return;
  const int vb = vb_local * stride;
  const int64_t m0 = (int64_t)vb * C::BM;
  const int64_t n0 = (int64_t)nt * C::BN;

  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int g = lane >> 4, col = lane & 15;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool ktail = (K % kBK) != 0;   // the last of all stages is partial
  StageDma<C::A_LD> la;
  StageDma<C::B_LD> lb;
  la.init(M, m0, V, K, C::BM);
  lb.init(X, n0, B, K, C::BN);
  // Stage kc lives in buffer kc % nbuf; ST - 1 stages are in flight while
  // one is used.
  static_assert(C::ST == 2 || C::ST == 3, "two or three stage buffers");
#pragma unroll
  for (int st = 0; st < C::ST - 1; ++st) {
    if (st < nk) {
      la.issue(As + st * SA, kb + st, K, ktail && kb + st == nk_all - 1);
      lb.issue(Bs + st * SB, kb + st, K, ktail && kb + st == nk_all - 1);
    }
  }
  for (int kc = 0; kc < nk; ++kc) {
    // this wave's copies of stage kc are done once only the later stages'
    // (ST - 2 of them, fewer at the end) remain
    if (C::ST == 3 && kc + 1 < nk)
      wait_vmcnt<(C::ST == 3 ? C::A_LD + C::B_LD : 0)>();
    else
      wait_vmcnt<0>();
    lds_barrier();     // every wave's copies of stage kc landed; stage kc-1 is no longer read
    if (kc + C::ST - 1 < nk) {
      const int nx = kc + C::ST - 1;
      const int nb = nx % nbuf;
      la.issue(As + nb * SA, kb + nx, K, ktail && kb + nx == nk_all - 1);
      lb.issue(Bs + nb * SB, kb + nx, K, ktail && kb + nx == nk_all - 1);
    }
    const u32x4* as = As + (kc % nbuf) * SA;
    const u32x4* bs = Bs + (kc % nbuf) * SB;
    // both k-steps' fragments are read first, so the second step's LDS
    // latency hides under the first step's matrix work
    constexpr int KS = kBK / 32;
    u32x4 fa[KS][C::FM], fb[KS][C::FN];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int c = s * 4 + g;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[s][i] = as[swz(wm * C::TM + i * 16 + col, c)];
#pragma unroll
      for (int jn = 0; jn < C::FN; ++jn) fb[s][jn] = bs[swz(wn * C::TN + jn * 16 + col, c)];
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jn = 0; jn < C::FN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[s][i]),
                                                               __builtin_bit_cast(bf16x8, fb[s][jn]), acc[i][jn], 0,
                                                               0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, KS * (C::FM + C::FN), 0);   // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, KS * C::FM * C::FN, 0);     // then the MFMAs
  }

  // --------------------------------------------------------------- epilogue
  const int64_t vrow = m0 + wm * C::TM + 4 * g;   // + i * 16 + q
  if constexpr (MODE == kModeMax) {
    // the maximum of each 32-row tile (two 16-row tiles of the wave)
    static_assert(C::FM % 2 == 0, "whole 32-row tiles per wave");
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      const int64_t n = n0 + wn * C::TN + jn * 16 + col;
#pragma unroll
      for (int i2 = 0; i2 < C::FM / 2; ++i2) {
        float m = neg_inf();
#pragma unroll
        for (int i = 2 * i2; i < 2 * i2 + 2; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (vrow + i * 16 + q < V) m = fmaxf(m, acc[i][jn][q]);
        m = fmax_lanes(m);
        if (g == 0 && n < B) aux_f[n * ns_tiles + vb_local * (C::BM / 32) + wm * (C::FM / 2) + i2] = m;
      }
    }
  } else if constexpr (MODE == kModePartial) {
    // fp32 partial products of this block's K stages: row n of part
    // blockIdx.y at S + (blockIdx.y * B + n) * ldS
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      const int64_t n = n0 + wn * C::TN + jn * 16 + col;
      if (n >= B) continue;
      float* prow = S + ((int64_t)blockIdx.y * B + n) * ldS;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int64_t m = vrow + i * 16;
        if (m + 4 <= V) {
          *reinterpret_cast<f32x4*>(prow + m) = acc[i][jn];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (m + q < V) prow[m + q] = acc[i][jn][q];
        }
      }
    }
  } else if constexpr (MODE == kModeStore) {
    // the product itself, rounded to bf16: Z row n at S + n * ldS (bf16)
    uint16_t* Z = reinterpret_cast<uint16_t*>(S);
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      const int64_t n = n0 + wn * C::TN + jn * 16 + col;
      if (n >= B) continue;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int64_t m = vrow + i * 16;
        uint16_t* z = Z + n * ldS + m;
        if (m + 4 <= V) {
          const uint32_t lo = (uint32_t)f32_to_bf16(acc[i][jn][0]) | ((uint32_t)f32_to_bf16(acc[i][jn][1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(acc[i][jn][2]) | ((uint32_t)f32_to_bf16(acc[i][jn][3]) << 16);
          *reinterpret_cast<uint2*>(z) = uint2{lo, hi};
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (m + q < V) z[q] = f32_to_bf16(acc[i][jn][q]);
        }
      }
    }
  } else {
    // Flags first, without branches (theta is waited for once, before any
    // store), then the rare stores of flagged scores.
    const bool full = m0 + C::BM <= V;
    float th[C::FN];
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      const int64_t n = n0 + wn * C::TN + jn * 16 + col;
      th[jn] = theta[n < B ? n : B - 1];
    }
    uint32_t bits[C::FN];
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      uint32_t b = 0;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) b |= (acc[i][jn][q] >= th[jn] ? 1u : 0u) << (i * 4 + q);
      bits[jn] = b;
    }
    if (!full) {
      uint32_t valid = 0;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) valid |= (vrow + i * 16 + q < V ? 1u : 0u) << (i * 4 + q);
#pragma unroll
      for (int jn = 0; jn < C::FN; ++jn) bits[jn] &= valid;
    }
#pragma unroll
    for (int jn = 0; jn < C::FN; ++jn) {
      const int64_t n = n0 + wn * C::TN + jn * 16 + col;
      if (n >= B) continue;
      mask[n * NW + ((int64_t)vb * C::WM + wm) * 4 + g] = bits[jn];
      if (bits[jn] == 0) continue;
      // the lane's 4 consecutive rows of a tile go out as one 16-byte store
      // when any of them is flagged (only flagged ones are read back)
      float* srow = S + n * ldS + vrow;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        if ((bits[jn] >> (i * 4)) & 15u) *reinterpret_cast<f32x4*>(srow + i * 16) = acc[i][jn];
    }
  }
}

// --------------------------------------------------------- per-row bound
// theta[b] = a value that between k and `cap` tile maxima of row b reach
// (at most the k-th largest maximum); -inf when fewer than k tiles exist.
// One wave per row, kThetaE maxima per lane.
template <int kThetaE>
__global__ void __launch_bounds__(256) theta_kernel(const float* __restrict__ tmax, int ns_tiles, int64_t B, int k,
                                                     int cap, float* __restrict__ theta) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= B) return;
  const float* t = tmax + row * ns_tiles;
  // all loads first (clamped, branch-free), then the keys
  float mv[kThetaE];
#pragma unroll
  for (int e = 0; e < kThetaE; ++e) mv[e] = t[min(e * kWave + lane, ns_tiles - 1)];
  uint64_t key[kThetaE];
  float vmin = __builtin_inff();
#pragma unroll
  for (int e = 0; e < kThetaE; ++e) {
    const int j = e * kWave + lane;
    const bool ok = j < ns_tiles && mv[e] > neg_inf();
    key[e] = ok ? cand_key(mv[e], j) : 0ull;
    vmin = ok ? fminf(vmin, mv[e]) : vmin;
  }
  int valid = 0;
#pragma unroll
  for (int e = 0; e < kThetaE; ++e) valid += wave_count(key[e] != 0);
  float th = neg_inf();
  if (valid >= k) {
    const uint64_t T = wave_window_threshold<kThetaE>(key, k, cap);
    if (T == 1) {
      th = __uint_as_float(order_key_inv(wave_min_u32(order_key(vmin))));
    } else {
      th = key_score(T);
    }
  }
  if (lane == 0) theta[row] = th;
}

// ----------------------------------------------------------------- collect
// One block per row. The four waves split the row's mask words (16-byte
// loads, a round's words in flight together); the flagged ids go to an LDS
// buffer (a slot from a prefix over the wave's lanes, the wave's base from
// an LDS counter: the order is free, the keys are ranked), then the wave
// fetches their scores in batches and stores their keys. Wave 0 then ranks
// the buffer.
// A row with more than kColCap flags (ties) is taken by wave 0 alone in
// rounds of kColCap slots (collect_rounds), each round's best k merged into
// a running list.
constexpr int kColCap = 1024;
constexpr int kColE = kColCap / kWave;

struct CollectWave {
  uint64_t key[kColCap];
  int vid[kColCap];
  uint64_t tmp[kWave];
  float ls[2][kWave];   // 0: this round's best, 1: running best
  int li[2][kWave];
};

// The vocabulary row of bit b of a row's 32-bit mask word w. A slice word
// s covers lane group g = s & 3 of the TM-row block s >> 2: its bit i * 4 + q
// stands for row (s >> 2) * TM + i * 16 + 4 g + q. Without HALF word w is
// slice word w; with HALF it holds the 16-bit slice words 2 w (low half)
// and 2 w + 1 (high half).
template <int TM, bool HALF>
__device__ __forceinline__ int mask_row(int w, int b) {
  const int s = HALF ? 2 * w + (b >> 4) : w;
  const int bb = HALF ? b & 15 : b;
  return (s >> 2) * TM + (bb >> 2) * 16 + 4 * (s & 3) + (bb & 3);
}

template <int TM, bool HALF>
__device__ __forceinline__ void collect_rounds(CollectWave& m, const uint32_t* __restrict__ mask, int NW,
                                               const float* __restrict__ S, int64_t ldS, int64_t row, int k,
                                               int32_t* __restrict__ idx, float* __restrict__ score) {
  const int lane = threadIdx.x & 63;
  const uint32_t* mw = mask + row * NW;
  const float* sr = S + row * ldS;

  // the lane's words, chunk c: w = 4 * (lane + 64 * (c * T4 + t)) + 0..3
  constexpr int T4 = 8;
  const int nq = (NW + 3) / 4;
  const int nchunk = (nq + kWave * T4 - 1) / (kWave * T4);
  auto load_chunk = [&](int c, u32x4 (&wd)[T4]) {
#pragma unroll
    for (int t = 0; t < T4; ++t) {
      const int q = lane + kWave * (c * T4 + t);
      wd[t] = *reinterpret_cast<const u32x4*>(mw + 4 * min(q, nq - 1));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q >= nq || 4 * q + e >= NW) wd[t][e] = 0u;
    }
  };
  int cnt = 0;
  for (int c = 0; c < nchunk; ++c) {
    u32x4 wd[T4];
    load_chunk(c, wd);
#pragma unroll
    for (int t = 0; t < T4; ++t) cnt += __popc(wd[t][0]) + __popc(wd[t][1]) + __popc(wd[t][2]) + __popc(wd[t][3]);
  }
  int before = 0, C = 0;
#pragma unroll
  for (int bit = 0; bit < 20; ++bit) {   // counts below 2^20
    const unsigned long long plane = __ballot((cnt >> bit) & 1);
    before += lanes_below(plane) << bit;
    C += __popcll(plane) << bit;
  }
  if (lane < kWave) {
    m.ls[1][lane] = neg_inf();
    m.li[1][lane] = kSentinelId;
  }
  for (int base = 0; base < max(C, 1); base += kColCap) {
    const int n = min(kColCap, C - base);
    // ids of the slots [base, base + n)
    int pos = before;
    for (int c = 0; c < nchunk; ++c) {
      u32x4 wd[T4];
      load_chunk(c, wd);
#pragma unroll
      for (int t = 0; t < T4; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t bits = wd[t][e];
          const int w = 4 * (lane + kWave * (c * T4 + t)) + e;
          while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1;
            if (pos >= base && pos < base + kColCap) m.vid[pos - base] = mask_row<TM, HALF>(w, b);
            ++pos;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // their scores: all ids from LDS, then all loads, then the keys
    int vv[kColE];
#pragma unroll
    for (int e = 0; e < kColE; ++e) {
      const int j = e * kWave + lane;
      vv[e] = j < n ? m.vid[j] : 0;
    }
    float xs[kColE];
#pragma unroll
    for (int e = 0; e < kColE; ++e) xs[e] = sr[vv[e]];
    uint64_t key[kColE];
#pragma unroll
    for (int e = 0; e < kColE; ++e) key[e] = e * kWave + lane < n ? cand_key(xs[e], vv[e]) : 0ull;
    if (C <= kColCap) {
      // one round: straight to the output
      wave_topk_emit<kColE>(key, k, m.tmp, m.ls[1], m.li[1]);
    } else {
      wave_topk_emit<kColE>(key, k, m.tmp, m.ls[0], m.li[0]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      uint64_t k2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int id = lane < k ? m.li[e][lane] : kSentinelId;
        k2[e] = id != kSentinelId ? cand_key(m.ls[e][lane], id) : 0ull;
      }
      wave_topk_emit<2>(k2, k, m.tmp, m.ls[1], m.li[1]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  if (lane < k) {
    idx[row * k + lane] = m.li[1][lane];
    if (score) score[row * k + lane] = m.ls[1][lane];
  }
}


template <int TM, int T4, bool HALF>
__global__ void __launch_bounds__(kGemmThreads) collect_kernel(const uint32_t* __restrict__ mask, int NW,
                                                                const float* __restrict__ S, int64_t ldS, int64_t B,
                                                                int k, int32_t* __restrict__ idx,
                                                                float* __restrict__ score) {
  __shared__ CollectWave m;
  __shared__ int n_flag;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x;
  const uint32_t* mw = mask + row * NW;
  const float* sr = S + row * ldS;
  if (threadIdx.x == 0) n_flag = 0;
  __syncthreads();
  // wave w takes the 16-byte word groups q = w * per + [0, per), in rounds of
  // T4 per lane (T4 = 12: one round for a 151936-token row, its loads all in
  // flight; T4 = 4 for large batches, where more blocks per CU pay off)
  const int nq = (NW + 3) / 4;
  const int per = (nq + 3) / 4;
  const int q0 = wave * per, q1 = min(nq, q0 + per);
  for (int qb = q0; qb < q1; qb += kWave * T4) {
    u32x4 wd[T4];
#pragma unroll
    for (int t = 0; t < T4; ++t) {
      const int q = qb + t * kWave + lane;
      wd[t] = *reinterpret_cast<const u32x4*>(mw + 4 * min(q, nq - 1));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (q >= q1 || 4 * q + e >= NW) wd[t][e] = 0u;
    }
    int cnt = 0;
#pragma unroll
    for (int t = 0; t < T4; ++t) cnt += __popc(wd[t][0]) + __popc(wd[t][1]) + __popc(wd[t][2]) + __popc(wd[t][3]);
    int before = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {   // counts from 256 on take the rounds below
      const unsigned long long plane = __ballot((cnt >> bit) & 1);
      before += lanes_below(plane) << bit;
      total += __popcll(plane) << bit;
    }
    const unsigned long long hi = __ballot(cnt >> 8);
    if (hi) total += kColCap + 1;   // cannot happen with distinct scores; forces the rounds
    int base = 0;
    if (lane == 0 && total) base = atomicAdd(&n_flag, total);
    base = __builtin_amdgcn_readfirstlane(base);
    int pos = base + before;
#pragma unroll
    for (int t = 0; t < T4; ++t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t bits = wd[t][e];
        const int w = 4 * (qb + t * kWave + lane) + e;
        while (bits) {
          const int b = __builtin_ctz(bits);
          bits &= bits - 1;
          if (pos < kColCap) m.vid[pos] = mask_row<TM, HALF>(w, b);
          ++pos;
        }
      }
    }
    // the scores of this round's slots [base, base + total), loads in batches
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int send = min(base + total, kColCap);
    for (int s0 = base; s0 < send; s0 += 8 * kWave) {
      int vv[8];
      float xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sl = s0 + u * kWave + lane;
        vv[u] = sl < send ? m.vid[sl] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) xs[u] = sr[vv[u]];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sl = s0 + u * kWave + lane;
        if (sl < send) m.key[sl] = cand_key(xs[u], vv[u]);
      }
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const int C = n_flag;
  if (C > kColCap) {
    collect_rounds<TM, HALF>(m, mask, NW, S, ldS, row, k, idx, score);
    return;
  }
  uint64_t key[kColE];
#pragma unroll
  for (int e = 0; e < kColE; ++e) {
    const int j = e * kWave + lane;
    key[e] = j < C ? m.key[j] : 0ull;
  }
  wave_topk_emit<kColE>(key, k, m.tmp, m.ls[1], m.li[1]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    idx[row * k + lane] = m.li[1][lane];
    if (score) score[row * k + lane] = m.ls[1][lane];
  }
}

// ------------------------------------------------ short-K vocabulary pass
// For the low-rank scores K = r <= 256 is short: a block keeps its BN draft
// rows of X (= z, BN x K) in LDS for its whole life and streams strips of
// 256 vocabulary rows of M past them:
//  - wave w owns rows [64 w, 64 w + 64) of a strip (four 16-row tiles), and
//    reads their K columns straight from global memory into the A operands
//    of the matrix cores;
//  - the A operands of four k steps are held in registers: once a k step's
//    MFMAs are issued, its registers are refilled with the k step four
//    ahead (in this strip or the block's next one), so the loads run about
//    half a strip ahead of their use (no LDS stage for M);
//  - the B operands (X) come from LDS, chunk c of row n at c ^ (n & 15).
// Blocks are persistent: block (grp, nt) takes strips grp, grp + G, ... for
// batch tile nt. When several batch tiles exist, the NT blocks of one strip
// group sit on one XCD (consecutive workgroup ids go to consecutive XCDs),
// so a strip comes from HBM once and from that XCD's L2 after.
// K past the row (K % 32 != 0) meets zero X chunks, so every product there
// is an exact zero. M rows past V read as zeros and are never flagged.
// Both passes of a selection (sample and main) run on this kernel, so each
// 16x16 tile of scores comes out of the same MFMA sequence in both, and the
// bound of the sample pass holds bit for bit in the main pass.
// Strip s covers vocabulary rows [s * stride * 256, s * stride * 256 + 256).
//  kModeMax:    tile maxima, row n at aux_f + n * ns_tiles, index s * 8 +
//               w * 2 + i2 for the 32-row tile i2 of wave w;
//  kModeFilter: per-row bound theta; flagged scores into S (row n at
//               S + n * ldS) and one 16-bit mask word per (row, 64-row
//               slice, lane group): 16-bit word (vb * 4 + w) * 4 + g of row
//               n (rows 2 NW such words apart) holds bit i * 4 + q for
//               vocabulary row (vb * 4 + w) * 64 + i * 16 + 4 * g + q.
constexpr int kStripRows = 256;

template <int BN, int KT, int MODE>
__global__ void __launch_bounds__(kGemmThreads) strip_sel_kernel(
    const uint16_t* __restrict__ M, const uint16_t* __restrict__ X, int64_t V, int K, int64_t B, int nstrips,
    int stride, int G, float* __restrict__ aux_f, int ns_tiles, const float* __restrict__ theta,
    float* __restrict__ S, int64_t ldS, uint32_t* __restrict__ mask, int NW) {
  constexpr int NF = BN / 16;                   // 16-column tiles of draft rows
  constexpr int CH = KT * 4;                    // 16-byte chunks per X row in LDS
  constexpr int SW = (CH < 16 ? CH : 16) - 1;   // swizzle mask
  extern __shared__ u32x4 xs[];                 // [BN][CH]

  const int NT = (int)((B + BN - 1) / BN);
  const int Lb = blockIdx.x;
  int grp, nt;
  if (NT > 1 && G % kXcds == 0) {
    const int xcd = Lb % kXcds, j = Lb / kXcds;
    grp = (j / NT) * kXcds + xcd;
    nt = j % NT;
  } else {
    grp = Lb / NT;
    nt = Lb % NT;
  }
  const int64_t n0 = (int64_t)nt * BN;

  // X tile to LDS, eight loads in flight per thread (clamped addresses,
  // zeros selected after the loads, so none of them waits on another)
  {
    constexpr int NL = BN * CH / kGemmThreads, NB = NL < 8 ? NL : 8;
    static_assert(NL * kGemmThreads == BN * CH && NL % NB == 0, "whole chunks per thread");
#pragma unroll
    for (int e0 = 0; e0 < NL; e0 += NB) {
      u32x4 v[NB];
      bool ok[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = (e0 + u) * kGemmThreads + threadIdx.x;
        const int n = e / CH, c = e % CH;
        ok[u] = n0 + n < B && c * 8 < K;
        v[u] = load16(X + (ok[u] ? (n0 + n) * K + c * 8 : 0));
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = (e0 + u) * kGemmThreads + threadIdx.x;
        const int n = e / CH, c = e % CH;
        xs[n * CH + (c ^ (n & SW))] = ok[u] ? v[u] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // the bound of each of the block's draft rows (main pass), read per
  // column tile in the epilogue
  __shared__ float th_s[MODE == kModeFilter ? BN : 1];
  if constexpr (MODE == kModeFilter) {
    for (int n = threadIdx.x; n < BN; n += kGemmThreads) th_s[n] = theta[n0 + n < B ? n0 + n : B - 1];
  }
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  __syncthreads();
  if (grp >= nstrips) return;

  // M rows of a strip through a buffer resource whose base and size are
  // the strip's (scalar registers): the lane's offsets do not change
  // between strips, and rows past V lie outside the resource and read as
  // zeros. Columns past K read the next row's first columns (finite) or
  // zeros; they meet zero X chunks either way.
  const uint32_t lane_off = (uint32_t)(((wave * 64 + col) * K + g * 8) * 2);
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = lane_off + (uint32_t)(i * 16 * K * 2);
  auto strip_rsrc = [&](int s) {
    const int64_t row0 = (int64_t)s * stride * kStripRows;
    const int64_t rows = V - row0 < kStripRows ? V - row0 : kStripRows;
    const uint64_t addr = reinterpret_cast<uint64_t>(M + row0 * K);
    const uint64_t ua = ((uint64_t)uniform_u32((uint32_t)(addr >> 32)) << 32) | uniform_u32((uint32_t)addr);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(ua), (short)0,
                                             (int)uniform_u32((uint32_t)(rows * K * 2)), kRawBufferFlags);
  };

  // A operands of the next KW k steps in a ring: slot t % KW holds k step
  // t; once its MFMAs are issued it is refilled with k step t + KW, of this
  // strip or of the block's next one.
  constexpr int KW = KT < 4 ? KT : 4;
  u32x4 a[KW][4];
  {
    const __amdgpu_buffer_rsrc_t rs = strip_rsrc(grp);
#pragma unroll
    for (int t = 0; t < KW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[t][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i] + t * 64, 0, 0);
  }

  for (int s = grp; s < nstrips; s += G) {
    const int sn = s + G < nstrips ? s + G : s;   // the last strip reloads itself (in bounds, unused)
    const __amdgpu_buffer_rsrc_t rc = strip_rsrc(s), rn = strip_rsrc(sn);

    f32x4 acc[4][NF];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < NF; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The X fragments do not change between strips. When they fit in 64
    // registers the compiler keeps them there for the block's life; above
    // that they are read from LDS two fragments ahead of their MFMAs (the
    // empty asm keeps the reads from being hoisted out of the strip loop).
    if constexpr (KT * NF > 16) asm volatile("" ::: "memory");
    constexpr int NU = KT * NF;
    auto xfrag = [&](int u) {
      const int t = u / NF, jn = u % NF;
      return xs[(jn * 16 + col) * CH + ((t * 4 + g) ^ (col & SW))];
    };
    u32x4 b0 = xfrag(0), b1 = NU > 1 ? xfrag(1) : b0;
    __builtin_amdgcn_sched_group_barrier(0x100, NU > 1 ? 2 : 1, 0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int t = u / NF, jn = u % NF;
      u32x4 b2 = b1;
      if (u + 2 < NU) {
        b2 = xfrag(u + 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the read two fragments ahead
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[t % KW][i]),
                                                             __builtin_bit_cast(bf16x8, b0), acc[i][jn], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (jn == NF - 1) {
        // k step t is done with its slot: k step t + KW takes its place
        const int tn = t + KW;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[t % KW][i] = tn < KT ? __builtin_amdgcn_raw_buffer_load_b128(rc, voff[i] + tn * 64, 0, 0)
                                 : __builtin_amdgcn_raw_buffer_load_b128(rn, voff[i] + (tn - KT) * 64, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 4, 0);
      }
      b0 = b1;
      b1 = b2;
    }

    // ------------------------------------------------------------ epilogue
    const int64_t vb = (int64_t)s * stride;
    const int64_t vrow = vb * kStripRows + wave * 64 + 4 * g;   // + i * 16 + q
    if constexpr (MODE == kModeMax) {
#pragma unroll
      for (int jn = 0; jn < NF; ++jn) {
        const int64_t n = n0 + jn * 16 + col;
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {   // the maximum of each 32-row tile
          float m = neg_inf();
#pragma unroll
          for (int i = 2 * i2; i < 2 * i2 + 2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if (vrow + i * 16 + q < V) m = fmaxf(m, acc[i][jn][q]);
          m = fmax_lanes(m);
          if (g == 0 && n < B) aux_f[n * ns_tiles + s * 8 + wave * 2 + i2] = m;
        }
      }
    } else {
      uint32_t valid = 0xFFFFu;
      if (vb * kStripRows + kStripRows > V) {
        valid = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) valid |= (vrow + i * 16 + q < V ? 1u : 0u) << (i * 4 + q);
      }
#pragma unroll
      for (int jn = 0; jn < NF; ++jn) {
        const int64_t n = n0 + jn * 16 + col;
        const float th = th_s[jn * 16 + col];
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) bits |= (acc[i][jn][q] >= th ? 1u : 0u) << (i * 4 + q);
        bits &= valid;
        if (n >= B) continue;
        reinterpret_cast<uint16_t*>(mask)[n * 2 * NW + (vb * 4 + wave) * 4 + g] = (uint16_t)bits;
        if (bits == 0) continue;
        float* srow = S + n * ldS + vrow;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((bits >> (i * 4)) & 15u) *reinterpret_cast<f32x4*>(srow + i * 16) = acc[i][jn];
      }
    }
  }
}

// ================================================================ launchers

namespace {

using CfgBig = GemmCfg<256, 256, 2, 2, 2>;  // B > 128: 128x128 per wave, two stage buffers (LDS)
using CfgWide = GemmCfg<256, 128, 2, 2>;    // 64 < B <= 128
using CfgNarrow = GemmCfg<256, 64, 4, 1>;   // B <= 64
using CfgDown = GemmCfg<64, 64, 2, 2>;      // z = Q . h for many rows (r is small)

constexpr int kGemmBM = 256;

int64_t vblocks(int64_t V) { return (V + kGemmBM - 1) / kGemmBM; }

// The sample pass reads every s-th vocabulary block: about 4 k sampled
// 16-row tiles, at most every 7th block (at 2048 rows, r = 256, k = 64:
// 523.3 -> 519.5 us per call against every 8th, the denser sample cutting
// the flagged scores by more than its own cost; every 6th was no better).
int sample_stride(int64_t V, int k) {
  const int64_t nvb = vblocks(V);
  int64_t s = nvb * (kGemmBM / 16) / (4 * (int64_t)k);
  if (s > 7) s = 7;
  if (s < 1) s = 1;
  const int64_t lo = (nvb + kMaxSampleTiles / (kGemmBM / 16) - 1) / (kMaxSampleTiles / (kGemmBM / 16));
  if (s < lo) s = lo;
  return (int)s;
}

template <class C>
size_t gemm_lds_bytes(int K = 1 << 30) {
  const int nk = (K + kBK - 1) / kBK;
  return size_t(nk < C::ST ? nk : C::ST) * (C::BM + C::BN) * kRowChunks * sizeof(u32x4);
}

template <class C>
hipError_t allow_lds() {
  for (const void* f : {(const void*)gemm_sel_kernel<C, kModeMax>, (const void*)gemm_sel_kernel<C, kModeFilter>,
                        (const void*)gemm_sel_kernel<C, kModeStore>, (const void*)gemm_sel_kernel<C, kModePartial>}) {
    const hipError_t e =
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds_bytes<C>());
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class C>
hipError_t run_gemm(int mode, const uint16_t* M, const uint16_t* X, int64_t V, int K, int64_t B, int nvb,
                    int stride, float* tmax, int ns_tiles, const float* theta, float* S, int64_t ldS,
                    uint32_t* mask, int NW, hipStream_t stream, Timing t = {}, int ksplit = 1) {
  const int64_t NT = (B + C::BN - 1) / C::BN;
  const int64_t nvb_pad = nvb >= kXcds ? (nvb + kXcds - 1) / kXcds * kXcds : nvb;
  const dim3 grid((unsigned)(nvb_pad * NT), (unsigned)(mode == kModePartial ? ksplit : 1));
  const size_t lds = gemm_lds_bytes<C>(K);
  if (mode == kModePartial)
    hipLaunchKernelGGL((gemm_sel_kernel<C, kModePartial>), grid, dim3(kGemmThreads), lds, stream, M, X, V, K, B,
                       nvb, stride, tmax, ns_tiles, theta, S, ldS, mask, NW);
  else if (mode == kModeMax)
    hipLaunchKernelGGL((gemm_sel_kernel<C, kModeMax>), grid, dim3(kGemmThreads), lds, stream, M, X, V, K, B, nvb,
                       stride, tmax, ns_tiles, theta, S, ldS, mask, NW);
  else if (mode == kModeStore)
    hipLaunchKernelGGL((gemm_sel_kernel<C, kModeStore>), grid, dim3(kGemmThreads), lds, stream, M, X, V, K, B, nvb,
                       stride, tmax, ns_tiles, theta, S, ldS, mask, NW);
  else
    LRH_LAUNCH(t, (gemm_sel_kernel<C, kModeFilter>), grid, dim3(kGemmThreads), lds, stream, M, X, V, K, B, nvb,
               stride, tmax, ns_tiles, theta, S, ldS, mask, NW);
  return hipGetLastError();
}

// One block per row; the width of the mask rounds by batch size. NW counts
// 32-bit words per row; HALF: each holds two 16-bit slice words.
template <int TM, bool HALF = false>
hipError_t launch_collect(const uint32_t* mask, int NW, const float* S, int64_t ldS, int64_t B, int k, int32_t* idx,
                          float* score, hipStream_t stream) {
  if (B <= 1024)
    hipLaunchKernelGGL((collect_kernel<TM, 12, HALF>), dim3((unsigned)B), dim3(kGemmThreads), 0, stream, mask, NW, S,
                       ldS, B, k, idx, score);
  else
    hipLaunchKernelGGL((collect_kernel<TM, 4, HALF>), dim3((unsigned)B), dim3(kGemmThreads), 0, stream, mask, NW, S,
                       ldS, B, k, idx, score);
  return hipGetLastError();
}

// theta of every row from the sample pass's tile maxima. The bound need not
// be the exact k-th maximum: any value that between k and cap maxima reach
// is valid (a looser one flags more scores). A window of 4 over k: per call
// at 2048 rows, 507.3 -> 504.9 us at r = 256, k = 64 (a window of k / 4) and
// 222.8 -> 221.2 at r = 128, k = 8; the exact k-th took 4.7 us more in theta
// than it saved.
hipError_t launch_theta(const BatchPlan& p, int64_t B, int k, const BatchScratch& w, hipStream_t stream) {
  const int cap = k + 4;
  const dim3 tg((unsigned)((B + 3) / 4)), tb(256);
  const int te = (p.ns_tiles + kWave - 1) / kWave;
  if (te <= 8)
    hipLaunchKernelGGL(theta_kernel<8>, tg, tb, 0, stream, w.tmax, p.ns_tiles, B, k, cap, w.theta);
  else if (te <= 16)
    hipLaunchKernelGGL(theta_kernel<16>, tg, tb, 0, stream, w.tmax, p.ns_tiles, B, k, cap, w.theta);
  else if (te <= 24)
    hipLaunchKernelGGL(theta_kernel<24>, tg, tb, 0, stream, w.tmax, p.ns_tiles, B, k, cap, w.theta);
  else
    hipLaunchKernelGGL(theta_kernel<32>, tg, tb, 0, stream, w.tmax, p.ns_tiles, B, k, cap, w.theta);
  return hipGetLastError();
}

// ----------------------------------------------------- short-K strip pass
constexpr int kStripMaxK = 256;
constexpr int64_t kStripMinB = 128;
constexpr int kStripBN = 256;   // draft rows per block (batch tile)

int num_cus() {
  static const int n = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    return cus;
  }();
  return n;
}

template <int BN, int KT>
size_t strip_lds_bytes() {
  return size_t(BN) * KT * 4 * sizeof(u32x4);
}

// Blocks of this kernel resident on the whole GPU at once.
template <int BN, int KT, int MODE>
int strip_slots() {
  static const int slots = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, strip_sel_kernel<BN, KT, MODE>, kGemmThreads,
                                                     strip_lds_bytes<BN, KT>()) != hipSuccess ||
        nb < 1)
      nb = 1;
    return nb * num_cus();
  }();
  return slots;
}

// Strip groups G: the grid is G x NT persistent blocks. With several batch
// tiles G is a multiple of 8 (the XCD mapping); with one, the strips are
// spread evenly over at most `slots` blocks.
int strip_groups(int nstrips, int NT, int slots) {
  int G = slots / NT;
  if (NT > 1) {
    G = G / kXcds * kXcds;
    if (G < kXcds) G = kXcds;
    return G < nstrips ? G : nstrips;
  }
  if (G < 1) G = 1;
  if (G > nstrips) G = nstrips;
  const int per = (nstrips + G - 1) / G;
  return (nstrips + per - 1) / per;
}

template <int BN, int KT>
hipError_t allow_strip_lds() {
  for (const void* f : {(const void*)strip_sel_kernel<BN, KT, kModeMax>,
                        (const void*)strip_sel_kernel<BN, KT, kModeFilter>}) {
    const hipError_t e =
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)strip_lds_bytes<BN, KT>());
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BN, int KT>
hipError_t strip_pass(const BatchPlan& p, const uint16_t* M, const uint16_t* X, int64_t V, int K, int64_t B, int k,
                      const BatchScratch& w, int32_t* idx, float* score, hipStream_t stream, Timing t) {
  const int NT = (int)((B + BN - 1) / BN);
  const size_t lds = strip_lds_bytes<BN, KT>();
  const int NW = (int)(p.nvb * (kGemmBM / 64) * 4 / 2);   // 64-row mask slices, two 16-bit words in 32 bits
  const int Gs = strip_groups(p.ns, NT, strip_slots<BN, KT, kModeMax>());
  hipLaunchKernelGGL((strip_sel_kernel<BN, KT, kModeMax>), dim3((unsigned)(Gs * NT)), dim3(kGemmThreads), lds,
                     stream, M, X, V, K, B, p.ns, p.stride, Gs, w.tmax, p.ns_tiles, nullptr, nullptr, 0, nullptr, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_theta(p, B, k, w, stream)) != hipSuccess) return e;
  const int nvb = (int)p.nvb;
  const int Gm = strip_groups(nvb, NT, strip_slots<BN, KT, kModeFilter>());
  LRH_LAUNCH(t, (strip_sel_kernel<BN, KT, kModeFilter>), dim3((unsigned)(Gm * NT)), dim3(kGemmThreads), lds, stream,
             M, X, V, K, B, nvb, 1, Gm, nullptr, 0, w.theta, w.S, p.ldS, w.mask, NW);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_collect<64, true>(w.mask, NW, w.S, p.ldS, B, k, idx, score, stream);
}

template <int KT>
hipError_t allow_strip_lds_k() {
  return allow_strip_lds<kStripBN, KT>();
}

template <class C>
hipError_t run_pass(const BatchPlan& p, const uint16_t* M, const uint16_t* X, int64_t V, int K, int64_t B, int k,
                    const BatchScratch& w, int32_t* idx, float* score, hipStream_t stream, Timing t) {
  hipError_t e = run_gemm<C>(kModeMax, M, X, V, K, B, p.ns, p.stride, w.tmax, p.ns_tiles, nullptr, nullptr, 0,
                             nullptr, 0, stream);
  if (e != hipSuccess) return e;
  if ((e = launch_theta(p, B, k, w, stream)) != hipSuccess) return e;
  e = run_gemm<C>(kModeFilter, M, X, V, K, B, (int)p.nvb, 1, nullptr, 0, w.theta, w.S, p.ldS, w.mask, p.NW,
                  stream, t);
  if (e != hipSuccess) return e;
  return launch_collect<C::TM>(w.mask, p.NW, w.S, p.ldS, B, k, idx, score, stream);
}

}  // namespace

bool batch_path(int dtype, int64_t B) { return dtype == 0 && B > kLongB; }

hipError_t batch_init() {
  hipError_t e = allow_lds<CfgWide>();
  if (e == hipSuccess) e = allow_lds<CfgBig>();
  if (e == hipSuccess) e = allow_lds<CfgNarrow>();
  if (e == hipSuccess) e = allow_lds<CfgDown>();
  if (e == hipSuccess) e = allow_strip_lds_k<2>();
  if (e == hipSuccess) e = allow_strip_lds_k<4>();
  if (e == hipSuccess) e = allow_strip_lds_k<8>();
  return e;
}

hipError_t launch_down_gemm(const void* Q, const void* H, int r, int d, int64_t B, void* Z, float* part,
                            size_t part_bytes, hipStream_t stream) {
  const int nvb = (r + CfgDown::BM - 1) / CfgDown::BM;
  const auto* q = static_cast<const uint16_t*>(Q);
  const auto* h = static_cast<const uint16_t*>(H);
  // K split over blocks until the grid has about 512 of them (at least 4
  // K stages each); the parts are added in a fixed order by down_reduce.
  // At 2048 rows, r = 256, d = 5120 (128 tiles): one block per tile took
  // 34.6 us; 2, 4, 8 and 16 parts 25.9, 23.8, 25.4 and 30.7 us with the
  // reduction (the tiles re-read H from L2, which more parts do not change).
  const int64_t tiles = (nvb >= kXcds ? (nvb + kXcds - 1) / kXcds * kXcds : nvb) *
                        ((B + CfgDown::BN - 1) / CfgDown::BN);
  const int nk = (d + kBK - 1) / kBK;
  int split = (int)std::min<int64_t>((512 + tiles - 1) / tiles, nk / 4);
  while (split > 1 && size_t(split) * size_t(B) * size_t(r) * 4 > part_bytes) --split;
  if (split <= 1)
    return run_gemm<CfgDown>(kModeStore, q, h, r, d, B, nvb, 1, nullptr, 0, nullptr, static_cast<float*>(Z), r,
                             nullptr, 0, stream);
  hipError_t e = run_gemm<CfgDown>(kModePartial, q, h, r, d, B, nvb, 1, nullptr, 0, nullptr, part, r, nullptr, 0,
                                   stream, {}, split);
  if (e != hipSuccess) return e;
  return launch_down_reduce(part, split, B * r, Z, stream);
}

hipError_t launch_gemm_f32(const uint16_t* M, int64_t Mrows, int K, const uint16_t* X, int64_t Xrows, float* S,
                           int ksplit, hipStream_t stream) {
  if (Mrows < 1 || Xrows < 1 || K < 8 || K % 8 || ksplit < 1) return hipErrorInvalidValue;
  auto go = [&](auto cfg) {
    using C = decltype(cfg);
    const int nvb = (int)((Mrows + C::BM - 1) / C::BM);
    return run_gemm<C>(kModePartial, M, X, Mrows, K, Xrows, nvb, 1, nullptr, 0, nullptr, S, Mrows, nullptr, 0,
                       stream, {}, ksplit);
  };
  if (Xrows > 128) return go(CfgBig{});
  if (Xrows > 64) return go(CfgWide{});
  return go(CfgNarrow{});
}

BatchPlan plan_batch(int64_t V, int64_t B, int k) {
  BatchPlan p;
  p.nvb = vblocks(V);
  p.stride = sample_stride(V, k);
  p.ns = (int)((p.nvb + p.stride - 1) / p.stride);
  p.ns_tiles = p.ns * (kGemmBM / 32);
  p.ldS = p.nvb * kGemmBM;
  const int tm = B <= 64 ? CfgNarrow::TM : CfgWide::TM;
  p.NW = (int)(p.nvb * (kGemmBM / tm) * 4);
  return p;
}

size_t batch_scratch_bytes(int64_t V, int64_t B_max) {
  // sized for the largest of every plan any k and B <= B_max can choose
  const int64_t nvb = vblocks(V);
  const size_t tmax = size_t(B_max) * kMaxSampleTiles * 4;
  const size_t theta = size_t(B_max) * 4;
  const size_t mask = size_t(B_max) * size_t(nvb) * (kGemmBM / CfgNarrow::TM) * 4 * 4;
  const size_t S = size_t(B_max) * size_t(nvb) * kGemmBM * 4;
  auto a = [](size_t x) { return (x + 255) & ~size_t(255); };
  return a(tmax) + a(theta) + a(mask) + a(S);
}

BatchScratch batch_scratch(void* base, int64_t V, int64_t B_max) {
  const int64_t nvb = vblocks(V);
  auto a = [](size_t x) { return (x + 255) & ~size_t(255); };
  char* p = static_cast<char*>(base);
  BatchScratch w;
  w.tmax = reinterpret_cast<float*>(p);
  p += a(size_t(B_max) * kMaxSampleTiles * 4);
  w.theta = reinterpret_cast<float*>(p);
  p += a(size_t(B_max) * 4);
  w.mask = reinterpret_cast<uint32_t*>(p);
  p += a(size_t(B_max) * size_t(nvb) * (kGemmBM / CfgNarrow::TM) * 4 * 4);
  w.S = reinterpret_cast<float*>(p);
  w.S_bytes = size_t(B_max) * size_t(nvb) * kGemmBM * 4;
  return w;
}

hipError_t launch_batch_select(const void* M, const void* X, int64_t V, int K, int64_t B, int k,
                               const BatchScratch& w, int32_t* idx, float* score, hipStream_t stream, Timing t) {
  const BatchPlan p = plan_batch(V, B, k);
  const uint16_t* m = static_cast<const uint16_t*>(M);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  // Above 128 rows the strip kernel beats the staged one with 256-row tiles
  // (r = 128, k = 32: 80.4 against 90.6 us per call at 160 rows, 94.0
  // against 100.6 at 256); up to 128 rows the staged kernel's 128-row tiles
  // are faster (71.7 against 75.3 us at 128 rows).
  if (K <= kStripMaxK && B > kStripMinB) {
    if (K <= 64) return strip_pass<kStripBN, 2>(p, m, x, V, K, B, k, w, idx, score, stream, t);
    if (K <= 128) return strip_pass<kStripBN, 4>(p, m, x, V, K, B, k, w, idx, score, stream, t);
    return strip_pass<kStripBN, 8>(p, m, x, V, K, B, k, w, idx, score, stream, t);
  }
  if (B <= 64) return run_pass<CfgNarrow>(p, m, x, V, K, B, k, w, idx, score, stream, t);
  if (B <= 128) return run_pass<CfgWide>(p, m, x, V, K, B, k, w, idx, score, stream, t);
  static_assert(CfgBig::TM == CfgWide::TM, "one mask layout above 64 rows");
  return run_pass<CfgBig>(p, m, x, V, K, B, k, w, idx, score, stream, t);
}

}  // namespace lrh
