// kernels_merge.hip — the k best of the slice lists, and exact rescoring.
//
// After the score pass every draft row has n sorted lists (one per
// vocabulary slice) of its slice's k best ids. merge_kernel finds the row's
// k best overall and, in the draft-head call, gives them their exact logits
// with the full-rank head ("EAGLE-4", section "Retrieve vocabulary
// candidates cheaply, then score them exactly": the retrieved candidates are
// scored exactly by the original full-rank head).
//
// Merge. Take any bound T that at least k list entries reach. Then an entry
// below T is preceded by k others and cannot win, and a list whose head is
// below T holds no winner. The kernel reads the leading entries of all lists
// of a row in one coalesced pass, finds such a T among them (a histogram of
// score images), gathers the entries that reach it (a few more than k) and
// ranks the k best of those.
//
// Rescoring: logit = W[id, :] . h with fp32 accumulation, one wave per
// candidate, every load of the W row and of h issued before the products.
#include "launch.h"
#include "merge.h"

namespace lrh {

// ------------------------------------------------------------ rescoring
// One wave per (row, candidate) pair; ids outside [0, V) give NaN.
template <typename T>
__global__ void __launch_bounds__(256) rescore_kernel(const T* __restrict__ W, const T* __restrict__ H,
                                                      const int32_t* __restrict__ idx, int64_t npairs, int k,
                                                      int64_t V, int d, float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= npairs) return;
  const int64_t b = pair / k;
  const int32_t v = idx[pair];
  if (v < 0 || v >= V) {
    if (lane == 0) logits[pair] = __builtin_nanf("");
    return;
  }
  const float acc = wave_row_dot<T>(W + (int64_t)v * d, H + b * (int64_t)d, d);
  if (lane == 0) logits[pair] = acc;
}

// ---------------------------------------------------------------- merge
// Grid (G, B), 512 threads: block (g, b) merges row b's n lists (sorted;
// depth-major: entry j of list p at part + (b * L + j) * n + p, or with
// `rowmajor`: at part + (b * n + p) * L + j) and, with
// RESCORE, gives the winners their exact logits. All G blocks of a row
// compute the same winners; block 0 writes idx and score.
//  1. The first 4 entries of every list are read in one coalesced pass (one
//     list per thread).
//  2. A bound T that at least k of these front entries reach comes from a
//     histogram of their score images (below); every thread sends its front
//     entries that reach T to the candidate buffer. Only a list whose 4th
//     entry still reaches T can hold more candidates; those (rare) lists are
//     read further, one per wave.
//  3. Wave 0 ranks the candidates. Meanwhile, with `speculate` and few
//     enough candidates, waves 1..7 of the G blocks already compute the
//     logits of all of them, so the W rows are in flight during the
//     selection: a candidate with token id v belongs to block v % G (the
//     blocks' buffers hold the same candidates in different orders, the ids
//     agree), and the block's waves take its candidates in turn. Afterwards
//     each block writes the logits of the winners that belong to it.
//     Otherwise block g's waves rescore winners g*per .. (g+1)*per - 1 after
//     the ranking, one per wave at a time. Speculation reads W rows of a few
//     more candidates than k: worth it when the call is latency-bound (few
//     rows), not when many rows already keep the chip busy.
template <typename T, bool RESCORE>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(
    const float* __restrict__ part_s, const int* __restrict__ part_i, int n, int L, int rowmajor, int speculate,
    const float* __restrict__ raw, const uint16_t* __restrict__ P, const uint16_t* __restrict__ Z, int K, int64_t V,
    int k,
    const T* __restrict__ W, const T* __restrict__ H, int d, int32_t* __restrict__ idx, float* __restrict__ score,
    float* __restrict__ logits) {
  __shared__ MergeSmem m;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y;
  const int G = gridDim.x, g = blockIdx.x;

  // 1-2. the leading entries of every list, the bound, the candidates
  const int64_t R = b * (int64_t)L * n;   // row base
  const ListLayout lay = rowmajor ? ListLayout{1, L} : ListLayout{n, 1};
  const RowScores src{raw ? raw + b * V : nullptr, raw ? nullptr : P, raw || !P ? nullptr : Z + b * K, K};
  const int nc = merge_collect(m, part_s + R, part_i + R, n, L, lay, src, V, k);

  // 3. selection, with the rescoring in flight when it can be
  const bool fits = nc <= kCandSlots;
  const bool spec = RESCORE && speculate && fits && nc <= G * (kMergeWaves - 1);
  if (wave == 0) {
    if (fits) {
      select_candidates(m, nc, k);
    } else if (L == k) {
      float s;
      int i;
      merge_lists_seq(part_s + R, part_i + R, n, k, lay, s, i);
      m.top_s[lane] = s;
      m.top_i[lane] = i;
    } else {
      // ties flag too many candidates: the k best of all the row's scores
      select_raw_row(m, src, V, k);
    }
  } else if (spec) {
    // this block's candidates in slot order; the t-th goes to wave 1 + t % 7
    int seen = 0;
    for (int base = 0; base < nc; base += kWave) {
      const int j = base + lane;
      const bool own = j < nc && key_id(m.cand[j]) % G == g;
      const unsigned long long mk = __ballot(own);
      const bool take = own && (seen + lanes_below(mk)) % (kMergeWaves - 1) == wave - 1;
      unsigned long long mt = __ballot(take);
      while (mt) {
        const int jj = base + __builtin_ctzll(mt);
        mt &= mt - 1;
        const int v = key_id(m.cand[jj]);
        const float x = (v >= 0 && v < V) ? wave_row_dot<T>(W + (int64_t)v * d, H + b * (int64_t)d, d)
                                          : __builtin_nanf("");
        if (lane == 0) m.spec[jj] = x;
      }
      seen += __popcll(mk);
    }
  }
  __syncthreads();
  if (g == 0 && wave == 0 && lane < k) {
    idx[b * k + lane] = m.top_i[lane];
    if (score) score[b * k + lane] = m.top_s[lane];
  }
  if constexpr (RESCORE) {
    if (spec) {
      if (threadIdx.x < k) {
        const int r = threadIdx.x, v = m.top_i[r];
        if (v == kSentinelId) {
          if (g == 0) logits[b * k + r] = __builtin_nanf("");   // fewer than k candidates
        } else if (v % G == g) {
          logits[b * k + r] = m.spec[m.slot_of[r]];
        }
      }
    } else {
      const int per = (k + G - 1) / G;
      const int j1 = min(k, (g + 1) * per);
      for (int j = g * per + wave; j < j1; j += kMergeWaves) {
        const int v = m.top_i[j];
        float acc = __builtin_nanf("");
        if (v >= 0 && v < V) acc = wave_row_dot<T>(W + (int64_t)v * d, H + b * (int64_t)d, d);
        if (lane == 0) logits[b * k + j] = acc;
      }
    }
  }
}

// ================================================================ launchers

hipError_t launch_rescore(int dtype, const void* W, const void* H, const int32_t* idx, int64_t B, int k,
                          int64_t V, int d, float* logits, hipStream_t stream) {
  const int64_t npairs = B * k;
  dim3 grid((unsigned)((npairs + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(rescore_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)W,
                       (const uint16_t*)H, idx, npairs, k, V, d, logits);
  else
    hipLaunchKernelGGL(rescore_kernel<float>, grid, dim3(256), 0, stream, (const float*)W, (const float*)H, idx,
                       npairs, k, V, d, logits);
  return hipGetLastError();
}

constexpr int kMergeRowBlocks = 4;
constexpr int64_t kMergeGridBlocks = 256;

hipError_t launch_merge(int dtype, const float* part_s, const int* part_i, int n, int L, bool rowmajor,
                        const float* raw, const void* P, const void* Z, int K, int64_t V, int64_t B, int k,
                        const void* W, const void* H, int d, int32_t* idx, float* score, float* logits,
                        bool speculate, hipStream_t stream) {
  if (n < 1 || n > kMaxLists || L < 1 || L > k) return hipErrorInvalidValue;
  if (L < k && !raw && !(P && Z && K >= 32 && K % 32 == 0)) return hipErrorInvalidValue;
  const uint16_t* Pm = static_cast<const uint16_t*>(P);
  const uint16_t* Zm = static_cast<const uint16_t*>(Z);
  const int bl = rowmajor ? 1 : 0, sp = speculate ? 1 : 0;
  const dim3 block(kMergeThreads);
  if (!logits) {
    const dim3 grid(1, (unsigned)B);
    hipLaunchKernelGGL((merge_kernel<uint16_t, false>), grid, block, 0, stream, part_s, part_i, n, L, bl, sp, raw, Pm,
                       Zm, K, V, k, (const uint16_t*)nullptr, (const uint16_t*)nullptr, d, idx, score, logits);
    return hipGetLastError();
  }
  // speculative: enough blocks that waves 1..7 of all of them can hold 2k
  // candidates, and up to twice that while the grid stays within 256
  // blocks (the candidates' logits spread over more waves: 6.5 -> 5.95 us
  // at 4 rows, 7.2 -> 6.5 at 8, 7.4 -> 6.9 at 16, r = 128, k = 32; beyond
  // 256 blocks 10.9 us at 16 rows). Otherwise one winner per wave, in up
  // to eight blocks per row while the grid stays within 256 blocks, else
  // up to four (each block ranks the row's lists; at r = 128, k = 64: 18.6
  // against 23.9 us with six blocks at 48 rows, 19.5 against 25.3 with
  // eight at 64 rows, but 9.8 against 11.2 with eight rather than four at
  // 16 rows)
  const int spec_min = (2 * k + kMergeWaves - 2) / (kMergeWaves - 1);
  const int spec_max = (4 * k + kMergeWaves - 2) / (kMergeWaves - 1);
  const int cap = B * 2 * kMergeRowBlocks <= kMergeGridBlocks ? 2 * kMergeRowBlocks : kMergeRowBlocks;
  const int G = speculate ? min(spec_max, max(spec_min, (int)(kMergeGridBlocks / B)))
                          : min(cap, (k + kMergeWaves - 1) / kMergeWaves);
  const dim3 grid((unsigned)G, (unsigned)B);
  if (dtype == 0)
    hipLaunchKernelGGL((merge_kernel<uint16_t, true>), grid, block, 0, stream, part_s, part_i, n, L, bl, sp, raw, Pm, Zm,
                       K, V, k, (const uint16_t*)W, (const uint16_t*)H, d, idx, score, logits);
  else
    hipLaunchKernelGGL((merge_kernel<float, true>), grid, block, 0, stream, part_s, part_i, n, L, bl, sp, raw, Pm, Zm, K,
                       V, k, (const float*)W, (const float*)H, d, idx, score, logits);
  return hipGetLastError();
}

}  // namespace lrh
