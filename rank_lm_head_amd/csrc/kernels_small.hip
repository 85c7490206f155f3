// kernels_small.hip — the head for a few rows, bf16: draft calls with B <= 64,
// the full-head baseline with B <= 4.
//
// With a few rows both contractions are close to matrix-vector products and
// the time is HBM streaming ("EAGLE-4", section "Retrieve vocabulary
// candidates cheaply, then score them exactly": the low-rank head still
// scores every vocabulary row, so P is read once per call). The effort goes
// to the memory side (large loads, several in flight per wave). The
// arithmetic is still not free: widening every bf16 element and
// multiplying it once per row on the vector ALU made the 8-row score pass
// take 22 us against about 10 for its bytes. So with 2 to 64 rows and r >=
// 32 the scores come from the matrix cores (stream_mfma_tiles: 16-row column
// tiles of z, idle columns cost nothing here); one row, and the full-head
// rows, stay on the vector ALU. (The one-row pass on the
// matrix cores measured slower, 18.7 against 17.3 us per call at r = 128:
// its operand tiles turn each 1 KiB wave load into 16 pieces of 64 bytes,
// and with one row the pass is bound by the memory side alone.)
//
//   select_short_kernel s = P . z with the fused k-best of each block's
//                       slice, scores staged in LDS (2-4 rows; 5-8 at r < 32)
//   select_rows_kernel  the same for 5-64 rows, the slice lists kept in
//                       registers
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

// ------------------------------------------- score pass, 5 to 64 rows
// The matrix-core stream (stream_mfma_tiles) with NB/16 column tiles of z
// (z's fragments in registers, or in LDS from 64 VGPRs of them), and no
// score leaves the registers: each lane keeps, for each of its rows
// of z (16 c + (l & 15) in column tile c), the 4 best of the vocabulary rows
// it is handed (rows 4 (l >> 4) .. +3 of every 16-row tile of its wave's
// quarter of the slice), in candidate order. At the end the block merges its
// 16 lists per row of z (4 waves x 4 lane groups) through LDS and writes the
// slice's L best, entry j to part_[b][x][j] (row-major: a block's entries of
// one row are one 16-byte write, and the merge still reads a row's lists
// coalesced; depth-major, as in select_short_kernel, made every entry a
// separate 32-byte write, 8.4 MB for 1 MB of lists at 64 rows, and
// block-major made the merge's reads 1 KiB apart: 2 us slower per call).
// No raw scores are kept: a slice that the merge needs more of is
// recomputed there in the same arithmetic.

// Inserts (x, id) into a list in candidate order whose empty slots hold NaN
// (at the end). The ids a list is handed increase, so an entry with an equal
// score precedes x: x goes below every entry it does not beat, or into the
// first empty slot (!(s >= x) holds for both). c[e] (x goes at e or above)
// implies c[e + 1], so every slot takes one of three values. Branch-free.
__device__ __forceinline__ void list_insert4(float (&ts)[kSliceList], int (&ti)[kSliceList], float x, int id) {
  static_assert(kSliceList == 4, "four entries");
  bool c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = !(ts[e] >= x);
#pragma unroll
  for (int e = 3; e > 0; --e) {
    const float s1 = c[e] ? x : ts[e];
    const int i1 = c[e] ? id : ti[e];
    ts[e] = c[e - 1] ? ts[e - 1] : s1;
    ti[e] = c[e - 1] ? ti[e - 1] : i1;
  }
  ts[0] = c[0] ? x : ts[0];
  ti[0] = c[0] ? id : ti[0];
}

// a := the 4 best of lists a and b (each in candidate order, empty entries
// (-inf, kSentinelId) last), in order: the better of a[i] and b[3 - i] for
// each i are the 4 best, as a bitonic sequence, which two rounds of
// compare-exchanges put in order.
__device__ __forceinline__ void merge_list4(float (&as)[4], int (&ai)[4], const float (&bs)[4], const int (&bi)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool keep = precedes(as[i], ai[i], bs[3 - i], bi[3 - i]);
    as[i] = keep ? as[i] : bs[3 - i];
    ai[i] = keep ? ai[i] : bi[3 - i];
  }
  auto cx = [&](int x, int y) {
    const bool keep = precedes(as[x], ai[x], as[y], ai[y]);
    const float sx = as[x], sy = as[y];
    const int ix = ai[x], iy = ai[y];
    as[x] = keep ? sx : sy;
    ai[x] = keep ? ix : iy;
    as[y] = keep ? sy : sx;
    ai[y] = keep ? iy : ix;
  };
  cx(0, 2);
  cx(1, 3);
  cx(0, 1);
  cx(2, 3);
}

// The lists of a block in LDS, the row of z innermost: the 16 lanes of a
// lane group write (and the threads of the merge read) consecutive words,
// and the rows of one lane group are padded by 4 words, so that the four
// lane groups of a wave fall on different banks.
template <int NB>
struct RowsLds {
  static constexpr int kRow = NB + 4;
  float ls[kWavesSmall][4][kSliceList][kRow];         // wave, lane group, entry, row of z
  int li[kWavesSmall][4][kSliceList][kRow];
};

// z's fragments for NT column tiles take NT * K / 8 VGPRs; from 64 of them
// (more rows of z at a larger rank) the block keeps z in LDS instead (chunk
// j of row b at b * K/8 + (j ^ (b & 15)), so that the 16 rows a fragment
// read touches sit on different banks) and reads each fragment just before
// its matrix-core step: every wave loading z from L2 on its own cost more
// at 64 VGPRs (1 us a launch at 16 x 512, 32 x 256 and 64 x 128). The copy
// shares its LDS with the lists at the end.
template <int K, int NB>
constexpr bool rows_z_in_lds() {
  return NB * K >= 16 * 512;
}

template <int K, int NB>
__global__ void __launch_bounds__(kSmallThreads) select_rows_kernel(
    const uint16_t* __restrict__ M, const uint16_t* __restrict__ X, int64_t V, int B, int L,
    float* __restrict__ part_s, int* __restrict__ part_i) {
  static_assert(NB == 16 || NB == 32 || NB == 64, "column tiles of 16 rows");
  constexpr int NT = NB / 16;
  constexpr int KS = K / 32;
  constexpr int TG = KS >= 4 ? 1 : 4 / KS;   // about 4 wave loads per group (more measured slower)
  constexpr bool ZL = rows_z_in_lds<K, NB>();
  constexpr int CH = K / 8;                  // 16-byte chunks of a row of z
  constexpr size_t kZBytes = ZL ? size_t(NB) * CH * 16 : 0;
  constexpr size_t kLds = sizeof(RowsLds<NB>) > kZBytes ? sizeof(RowsLds<NB>) : kZBytes;
  __shared__ __align__(16) unsigned char lds_raw[kLds];
  RowsLds<NB>& sm = *reinterpret_cast<RowsLds<NB>*>(lds_raw);
  u32x4* zs = reinterpret_cast<u32x4*>(lds_raw);
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  if constexpr (ZL) {
    static_assert(CH >= 16, "the swizzle stays inside the row");
    for (int e = threadIdx.x; e < NB * CH; e += kSmallThreads) {
      const int b = e / CH, j = e % CH;
      zs[b * CH + (j ^ (b & 15))] = b < B ? load16(X + (int64_t)b * K + j * 8) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }

  // slice bounds V*x/n in 32 bits: this path keeps V*n below 2^32
  const uint32_t v32 = (uint32_t)V, n32 = gridDim.x;
  const int64_t blo = v32 * blockIdx.x / n32, bhi = v32 * (blockIdx.x + 1) / n32;
  const int64_t wlo = blo + (bhi - blo) * wave / kWavesSmall;
  const int64_t whi = blo + (bhi - blo) * (wave + 1) / kWavesSmall;

  float ts[NT][kSliceList];
  int ti[NT][kSliceList];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int e = 0; e < kSliceList; ++e) {
      ts[c][e] = __builtin_nanf("");
      ti[c][e] = kSentinelId;
    }
  // ids in 32 bits (V < 2^31); a tile past the wave's range (its last one)
  // keeps only its rows below whi
  const int whi32 = (int)whi;
  // (the column tiles' lists are independent: interleaved for the scheduler)
  auto sink = [&](int64_t base, const f32x4 (&acc)[NT]) {
    const int row0 = (int)base + 4 * g;
    if ((int)base + 16 <= whi32) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < NT; ++c) list_insert4(ts[c], ti[c], acc[c][q], row0 + q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (row0 + q < whi32) {
#pragma unroll
          for (int c = 0; c < NT; ++c) list_insert4(ts[c], ti[c], acc[c][q], row0 + q);
        }
    }
  };
  if constexpr (ZL) {
    stream_mfma_tiles_x<K, NT, TG, true>(
        M, wlo, whi, [&](int c, int t) { return zs[(c * 16 + col) * CH + ((t * 4 + g) ^ col)]; }, sink);
    __syncthreads();   // the lists below reuse z's LDS
  } else {
    stream_mfma_tiles<K, NT, TG>(M, X, B, wlo, whi, sink);
  }

  // the 16 lists of each row of z (4 waves x 4 lane groups) to LDS; then T
  // consecutive lanes per row of z (T = 256 / NB: 4, 8 or 16, inside one
  // wave) each merge 16 / T of them, and a butterfly over the T lanes (DPP
  // exchanges; both partners compute the same merge, as the order is total)
  // leaves the row's 4 best on all of them
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int e = 0; e < kSliceList; ++e) {
      const bool empty = ti[c][e] == kSentinelId;
      sm.ls[wave][g][e][c * 16 + col] = empty ? neg_inf() : ts[c][e];
      sm.li[wave][g][e][c * 16 + col] = ti[c][e];
    }
  __syncthreads();
  constexpr int T = kSmallThreads / NB, PER = kWavesSmall * 4 / T;
  const int b = threadIdx.x / T, p = threadIdx.x % T;
  float as[4], bs[4];
  int ai[4], bi[4];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int list = p * PER + j, w = list >> 2, gg = list & 3;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bs[e] = sm.ls[w][gg][e][b];
      bi[e] = sm.li[w][gg][e][b];
    }
    if (j == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        as[e] = bs[e];
        ai[e] = bi[e];
      }
    } else {
      merge_list4(as, ai, bs, bi);
    }
  }
  auto exchange = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bs[e] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(as[e]), C, 0xf, 0xf, true));
      bi[e] = __builtin_amdgcn_mov_dpp(ai[e], C, 0xf, 0xf, true);
    }
    merge_list4(as, ai, bs, bi);
  };
  exchange(std::integral_constant<int, 0xB1>{});                           // lane ^ 1
  exchange(std::integral_constant<int, 0x4E>{});                           // lane ^ 2
  if constexpr (T >= 8) exchange(std::integral_constant<int, 0x141>{});    // 7 - lane in 8
  if constexpr (T >= 16) exchange(std::integral_constant<int, 0x128>{});   // lane + 8 in 16
  if (p == 0 && b < B) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < L) {
        const int64_t o = ((int64_t)b * gridDim.x + blockIdx.x) * L + e;
        part_s[o] = as[e];
        part_i[o] = ai[e];
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

// 5 to 64 rows: column tiles of 16, 32 or 64 rows of z, their fragments in
// registers below 64 VGPRs, else in LDS.
bool rows_path(int dtype, int64_t B, int64_t K_lowrank, int64_t V) {
  if (dtype != 0 || B < kRowsMinB || B > kRowsMaxB) return false;
  if (V > (int64_t)kMaxSmallBlocks * kBlockRows) return false;
  return K_lowrank >= 32 && K_lowrank <= 512 && (K_lowrank & (K_lowrank - 1)) == 0;
}

template <int K>
static hipError_t launch_rows_k(const void* M, const void* X, int64_t V, int64_t B, int k, float* ps, int* pi,
                                hipStream_t stream, Timing t) {
  const int nblk = small_blocks(V);
  const int L = small_list_len(k);
  if (!rows_path(0, B, K, V) || V * nblk >= (int64_t)1 << 32) return hipErrorInvalidValue;
  const dim3 grid(nblk), block(kSmallThreads);
#define LRH_RW(NB)                                                                                        \
  LRH_LAUNCH(t, (select_rows_kernel<K, NB>), grid, block, 0, stream, (const uint16_t*)M, (const uint16_t*)X, V, \
             (int)B, L, ps, pi)
  if (B <= 16)
    LRH_RW(16);
  else if (B <= 32)
    LRH_RW(32);
  else
    LRH_RW(64);
#undef LRH_RW
  return hipGetLastError();
}

hipError_t launch_select_rows(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* ps,
                              int* pi, hipStream_t stream, Timing t) {
  switch (K) {
    case 32: return launch_rows_k<32>(M, X, V, B, k, ps, pi, stream, t);
    case 64: return launch_rows_k<64>(M, X, V, B, k, ps, pi, stream, t);
    case 128: return launch_rows_k<128>(M, X, V, B, k, ps, pi, stream, t);
    case 256: return launch_rows_k<256>(M, X, V, B, k, ps, pi, stream, t);
    case 512: return launch_rows_k<512>(M, X, V, B, k, ps, pi, stream, t);
    default: return hipErrorInvalidValue;
  }
}

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
