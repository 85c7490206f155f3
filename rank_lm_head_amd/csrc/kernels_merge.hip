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
#include "topk.h"

namespace lrh {

constexpr int kMergeWaves = 8;
constexpr int kMergeThreads = kMergeWaves * kWave;
constexpr int kMaxLists = kMergeWaves * kWave;   // lists of a row (one per thread)

// ------------------------------------------------------------- row dot
template <typename T>
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 h, float acc);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(u32x4 w, u32x4 h, float acc) {
  return dot8_bf16(w, h, acc);
}
template <>
__device__ __forceinline__ float dot_chunk<float>(u32x4 w, u32x4 h, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(w[q]), __uint_as_float(h[q]), acc);
  return acc;
}

// w . h over d elements by one wave; every lane returns the sum. A row of
// up to U wave loads has all of them in flight (U is the row's load count
// rounded up to 4, 8, 10, 12 or 16, so that no load is wasted on a short
// row); longer rows go in chunks of 16. Loads past d read a clamped, valid
// address and are zeroed, so none is predicated. For every U the lane's
// sum runs over its chunks in the same order.
template <typename T, int U>
__device__ __forceinline__ float wave_row_dot_u(const T* __restrict__ w, const T* __restrict__ h, int d) {
  constexpr int per = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int c0 = 0; c0 < d; c0 += U * kWave * per) {
    u32x4 wv[U], hv[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = c0 + (t * kWave + lane) * per;
      const int cc = c < d ? c : d - per;
      wv[t] = load16(w + cc);
      hv[t] = load16(h + cc);
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const bool ok = c0 + (t * kWave + lane) * per < d;
      acc = dot_chunk<T>(ok ? wv[t] : u32x4{0u, 0u, 0u, 0u}, hv[t], acc);
    }
  }
  return group_sum<kWave>(acc);
}

template <typename T>
__device__ __forceinline__ float wave_row_dot(const T* __restrict__ w, const T* __restrict__ h, int d) {
  constexpr int per = 16 / sizeof(T);
  const int nl = (d + kWave * per - 1) / (kWave * per);   // wave loads per row
  if (nl <= 4) return wave_row_dot_u<T, 4>(w, h, d);
  if (nl <= 8) return wave_row_dot_u<T, 8>(w, h, d);
  if (nl <= 10) return wave_row_dot_u<T, 10>(w, h, d);
  if (nl <= 12) return wave_row_dot_u<T, 12>(w, h, d);
  return wave_row_dot_u<T, 16>(w, h, d);
}

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
constexpr int kCandE = 8;                   // candidates per lane of wave 0
constexpr int kCandSlots = kCandE * kWave;
constexpr int kFront = 4;                   // leading entries of each list read up front
constexpr int kRawPerLane = 8;              // a slice's raw scores per lane (slices <= 512 rows)

constexpr int kHistBins = 256;
constexpr int kRankSlots = 2 * kWave;     // candidates ranked directly

struct MergeSmem {
  uint32_t hist[kHistBins];   // front entries per bin of score images
  uint32_t wmin[kMergeWaves], wmax[kMergeWaves];
  int wcnt[kMergeWaves];
  uint64_t cand[kCandSlots];
  float spec[kCandSlots];   // exact logit of candidate slot j (this block's share)
  int slot_of[kWave];       // candidate slot of each winner
  uint64_t tmp[kRankSlots];
  int tslot[kRankSlots];
  float top_s[kWave];
  int top_i[kWave];
  int deep[kMaxLists];       // lists whose front entries all reach the bound
  uint64_t deep_key[kMaxLists];   // and the key of their last front entry
  int n_cand;
  int n_deep;
};

// The k best of the n_cand candidate keys in m.cand, in candidate order, to
// m.top_s / m.top_i (wave 0), and m.slot_of[rank] = the winner's slot. Up to
// 128 candidates are ranked directly (two per lane); beyond that a bound
// that between k and 128 of them reach is found first.
__device__ __forceinline__ void select_candidates(MergeSmem& m, int nc, int k) {
  const int lane = threadIdx.x & 63;
  uint64_t key[kCandE];
#pragma unroll
  for (int e = 0; e < kCandE; ++e) {
    const int j = e * kWave + lane;
    key[e] = j < nc ? m.cand[j] : 0ull;
  }
  const uint64_t T = wave_window_threshold<kCandE>(key, k, kRankSlots);
  int n = 0;
#pragma unroll
  for (int e = 0; e < kCandE; ++e) {
    const bool sel = key[e] != 0 && key[e] >= T;
    const unsigned long long mk = __ballot(sel);
    if (sel) {
      const int p = n + lanes_below(mk);
      if (p < kRankSlots) {
        m.tmp[p] = key[e];
        m.tslot[p] = e * kWave + lane;
      }
    }
    n += __popcll(mk);
  }
  n = min(n, kRankSlots);
#pragma unroll
  for (int h = 0; h < 2; ++h) {   // zeros up to round_up(n, 8)
    const int q = lane + h * kWave;
    if (q >= n && q < ((n + 7) & ~7)) m.tmp[q] = 0ull;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int slot[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) slot[h] = lane + h * kWave < n ? m.tslot[lane + h * kWave] : 0;
  int r[2];
  wave_rank_emit2(m.tmp, n, k, m.top_s, m.top_i, r);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (r[h] < k) m.slot_of[r[h]] = slot[h];
}

// Grid (G, B), 512 threads: block (g, b) merges row b's n lists (sorted,
// depth-major: entry j of list p at part + (b * k + j) * n + p) and, with
// RESCORE, gives the winners their exact logits. All G blocks of a row
// compute the same winners; block 0 writes idx and score.
//  1. The first 4 entries of every list are read in one coalesced pass (one
//     list per thread).
//  2. A bound T that at least k of these front entries reach comes from a
//     histogram of their score images (below); every thread sends its front
//     entries that reach T to the candidate buffer. Only a list whose 4th
//     entry still reaches T can hold more candidates; those (rare) lists are
//     read further, one per wave.
//  3. Wave 0 ranks the candidates. Meanwhile, when there are few enough
//     candidates, waves 1..7 of the G blocks already compute the logits of
//     all of them, so the W rows are in flight during the selection: a
//     candidate with token id v belongs to block v % G (the blocks' buffers
//     hold the same candidates in different orders, the ids agree), and the
//     block's waves take its candidates in turn. Afterwards each block
//     writes the logits of the winners that belong to it. With more
//     candidates, wave w of block g rescores winner g*per + w instead.
template <typename T, bool RESCORE>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(
    const float* __restrict__ part_s, const int* __restrict__ part_i, int n, int L, const float* __restrict__ raw,
    int64_t V, int k, const T* __restrict__ W, const T* __restrict__ H, int d, int32_t* __restrict__ idx,
    float* __restrict__ score, float* __restrict__ logits) {
  __shared__ MergeSmem m;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y;
  const int G = gridDim.x, g = blockIdx.x;

  // 1. the first kFront entries of every list (contiguous across lists in
  //    the depth-major layout), one list per thread
  const int64_t R = b * (int64_t)L * n;   // row base
  const int F = min(kFront, L);           // front entries held
  const int p = threadIdx.x;
  const int pc = min(p, n - 1);
  float fs[kFront];
  int fi[kFront];
#pragma unroll
  for (int j = 0; j < kFront; ++j) {
    const int jc = min(j, L - 1);
    fs[j] = part_s[R + (int64_t)jc * n + pc];
    fi[j] = part_i[R + (int64_t)jc * n + pc];
    if (p >= n || j >= L) fi[j] = kSentinelId;
  }
  // score images (order-preserving, -0 as +0); 0 marks an empty entry
  uint32_t fk[kFront];
#pragma unroll
  for (int j = 0; j < kFront; ++j) fk[j] = fi[j] != kSentinelId ? order_key(fs[j] + 0.0f) : 0u;
  {
    const uint32_t hk = fk[0];
    const uint32_t wmn = wave_min_u32(hk ? hk : 0xFFFFFFFFu), wmx = wave_max_u32(hk);
    const int wc = __popcll(__ballot(hk != 0));
    if (lane == 0) {
      m.wmin[wave] = wmn;
      m.wmax[wave] = wmx;
      m.wcnt[wave] = wc;
    }
  }
  if (threadIdx.x < kHistBins) m.hist[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    m.n_cand = 0;
    m.n_deep = 0;
  }
  __syncthreads();

  // 2. the bound Tk (a score image): with more than k non-empty heads, the
  //    front entries are counted in 256 bins of images between the lowest
  //    and the highest head, and Tk is the lower edge of the highest bin at
  //    which the count from the top reaches k. The edges are images, so the
  //    count at Tk is exact: at least k entries reach Tk. (Every front entry at
  //    or above the k-th best head lies in the binned range.) With k heads
  //    or fewer, Tk = 1 and every non-empty entry counts.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  int nheads = 0;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    kmin = min(kmin, m.wmin[w]);
    kmax = max(kmax, m.wmax[w]);
    nheads += m.wcnt[w];
  }
  uint32_t Tk = 1u;
  if (nheads > k) {
    const uint32_t R = kmax - kmin;
    const int shift = R >= (uint32_t)kHistBins ? 24 - __clz(R) : 0;   // R >> shift < 256
#pragma unroll
    for (int j = 0; j < kFront; ++j)
      if (fk[j] >= kmin) atomicAdd(&m.hist[min((fk[j] - kmin) >> shift, (uint32_t)kHistBins - 1)], 1u);
    __syncthreads();
    // every wave: counts from the top; lane l holds bins 255 - 4l - i
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = m.hist[kHistBins - 1 - 4 * lane - i] + (i ? c[i - 1] : 0u);
    const uint32_t above = wave_incl_scan_u32(c[3]) - c[3];   // in lanes before this one
    const unsigned long long reach = __ballot(above + c[3] >= (uint32_t)k);
    const int l0 = __builtin_ctzll(reach);   // first lane whose bins reach k (nheads > k: one does)
    int i0 = 3;
#pragma unroll
    for (int i = 2; i >= 0; --i) i0 = above + c[i] >= (uint32_t)k ? i : i0;
    const int bstar = kHistBins - 1 - 4 * l0 - __builtin_amdgcn_readlane(i0, l0);
    Tk = kmin + ((uint32_t)bstar << shift);
  }
  // An entry counts when its image reaches Tk (empty entries never do).
  auto reaches = [&](float sc, int id) { return id != kSentinelId && order_key(sc + 0.0f) >= Tk; };
  {
    uint32_t pass = 0;
#pragma unroll
    for (int j = 0; j < kFront; ++j) pass |= (fk[j] != 0u && fk[j] >= Tk ? 1u : 0u) << j;
    // slots from a prefix over the wave's lanes of their counts (bit planes)
    const int cnt = __popc(pass);
    int before = 0, wave_total = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {
      const unsigned long long plane = __ballot((cnt >> bit) & 1);
      before += lanes_below(plane) << bit;
      wave_total += __popcll(plane) << bit;
    }
    int base = 0;
    if (wave_total) {
      if (lane == 0) base = atomicAdd(&m.n_cand, wave_total);
      base = __builtin_amdgcn_readfirstlane(base);
    }
    int slot = base + before;
#pragma unroll
    for (int j = 0; j < kFront; ++j) {
      if (pass & (1u << j)) {
        if (slot < kCandSlots) m.cand[slot] = cand_key(fs[j], fi[j]);
        ++slot;
      }
    }
    // a slice whose last front entry reaches the bound may hold more: the
    // rest of its list (L > F), or its raw scores (lists shorter than k)
    const bool more = L > F || (L < k && raw != nullptr);
    if (more && (pass >> (F - 1)) & 1u) {
      const int dl = atomicAdd(&m.n_deep, 1);
      m.deep[dl] = p;
      m.deep_key[dl] = cand_key(fs[F - 1], fi[F - 1]);
    }
  }
  __syncthreads();
  if (m.n_deep > 0) {
    // rare: one slice per wave at a time
    const int nd = m.n_deep;
    for (int dl = wave; dl < nd; dl += kMergeWaves) {
      const int q = m.deep[dl];
      if (L > F) {
        const int j = F + lane;
        const int jc = min(j, L - 1);
        const float sc = part_s[R + (int64_t)jc * n + q];
        const int id = j < L ? part_i[R + (int64_t)jc * n + q] : kSentinelId;
        const bool ps = reaches(sc, id);
        const unsigned long long mk = __ballot(ps);
        if (mk) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&m.n_cand, __popcll(mk));
          base = __shfl(base, 0);
          const int slot = base + lanes_below(mk);
          if (ps && slot < kCandSlots) m.cand[slot] = cand_key(sc, id);
        }
      } else {
        // the slice's raw scores below its list's last entry that reach T
        const int64_t lo = V * q / n, hi = V * (q + 1) / n;
        const uint64_t below = m.deep_key[dl];
        const float* rr = raw + b * V;
        float xs[kRawPerLane];
#pragma unroll
        for (int t = 0; t < kRawPerLane; ++t) xs[t] = rr[min(lo + t * kWave + lane, hi - 1)];
#pragma unroll
        for (int t = 0; t < kRawPerLane; ++t) {
          const int64_t v = lo + t * kWave + lane;
          const uint64_t key = v < hi ? cand_key(xs[t], (int)v) : 0ull;
          const bool ps = key != 0 && key < below && reaches(xs[t], (int)v);
          const unsigned long long mk = __ballot(ps);
          if (mk) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&m.n_cand, __popcll(mk));
            base = __shfl(base, 0);
            const int slot = base + lanes_below(mk);
            if (ps && slot < kCandSlots) m.cand[slot] = key;
          }
        }
      }
    }
    __syncthreads();
  }
  const int nc = m.n_cand;

  // 3. selection, with the rescoring in flight when it can be
  const bool fits = nc <= kCandSlots;
  const bool spec = RESCORE && fits && nc <= G * (kMergeWaves - 1);
  if (wave == 0) {
    if (fits) {
      select_candidates(m, nc, k);
    } else if (L == k) {
      float s;
      int i;
      merge_lists_seq(part_s + R, part_i + R, n, k, s, i);
      m.top_s[lane] = s;
      m.top_i[lane] = i;
    } else {
      // ties flag too many candidates: the k best of the row's raw scores,
      // 448 at a time, each chunk merged into the running best
      m.top_s[lane] = neg_inf();
      m.top_i[lane] = kSentinelId;
      const float* rr = raw + b * V;
      for (int64_t c0 = 0; c0 < V; c0 += 7 * kWave) {
        uint64_t key[8];
#pragma unroll
        for (int e = 0; e < 7; ++e) {
          const int64_t v = c0 + e * kWave + lane;
          key[e] = v < V ? cand_key(rr[v], (int)v) : 0ull;
        }
        key[7] = lane < k && m.top_i[lane] != kSentinelId ? cand_key(m.top_s[lane], m.top_i[lane]) : 0ull;
        wave_topk_emit<8>(key, k, m.tmp, m.top_s, m.top_i);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
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
      const int j = g * per + wave;
      if (wave < per && j < k) {
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

hipError_t launch_merge(int dtype, const float* part_s, const int* part_i, int n, int L, const float* raw,
                        int64_t V, int64_t B, int k, const void* W, const void* H, int d, int32_t* idx,
                        float* score, float* logits, hipStream_t stream) {
  if (n < 1 || n > kMaxLists || L < 1 || L > k) return hipErrorInvalidValue;
  if (L < k && (!raw || (V + n - 1) / n > kRawPerLane * kWave)) return hipErrorInvalidValue;
  const dim3 block(kMergeThreads);
  if (!logits) {
    const dim3 grid(1, (unsigned)B);
    hipLaunchKernelGGL((merge_kernel<uint16_t, false>), grid, block, 0, stream, part_s, part_i, n, L, raw, V, k,
                       (const uint16_t*)nullptr, (const uint16_t*)nullptr, d, idx, score, logits);
    return hipGetLastError();
  }
  // enough blocks that waves 1..7 of all of them can hold 2k candidates
  const int G = (2 * k + kMergeWaves - 2) / (kMergeWaves - 1);
  const dim3 grid((unsigned)G, (unsigned)B);
  if (dtype == 0)
    hipLaunchKernelGGL((merge_kernel<uint16_t, true>), grid, block, 0, stream, part_s, part_i, n, L, raw, V, k,
                       (const uint16_t*)W, (const uint16_t*)H, d, idx, score, logits);
  else
    hipLaunchKernelGGL((merge_kernel<float, true>), grid, block, 0, stream, part_s, part_i, n, L, raw, V, k,
                       (const float*)W, (const float*)H, d, idx, score, logits);
  return hipGetLastError();
}

}  // namespace lrh
