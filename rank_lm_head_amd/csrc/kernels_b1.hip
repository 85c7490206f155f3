// kernels_b1.hip — the draft-head call for one row in two launches, and the
// wide down-projection of the few-row path.
//
// The method ("EAGLE-4", section "Retrieve vocabulary candidates cheaply,
// then score them exactly"): z = Q . h, s[v] = P[v,:] . z for every
// vocabulary row, the k best ids under "higher score first, lower id on
// ties", then the exact logits W[id,:] . h of those k only. For one draft
// row the call is bound by reading P once (V x r bf16); what is left around
// that stream is latency, and this file cuts it to two launches:
//
//   down_wide_kernel  z = Q . h for up to 64 rows, one block per row of Q
//                     (two above 48 rows at r <= 256) and group of 8 rows
//                     (each reading whole rows of Q at once), and the reset
//                     of the one-row pass's completion counters.
//   draft1_kernel     one block per compute unit streams its vocabulary
//                     slice of P, takes the slice's best L = min(4, k)
//                     entries and, speculatively, the exact logit of the
//                     slice's best one (a row of W per block, gathered while
//                     the other entries are found). Each block then takes a
//                     ticket; the last block to finish merges all slice lists
//                     into the row's k best and fills in the few logits not
//                     computed yet.
//
// Completion uses two levels of device-scope counters: one per group of
// blocks that share blockIdx % 8 (the compute-die a block is dispatched to),
// then one for the groups, so no single address takes every block's
// atomic. The down-projection, which runs first in the same stream, zeroes
// them, so the call keeps no state in the workspace between calls.
#include "launch.h"
#include "merge.h"
#include "stream.h"

namespace lrh {

constexpr int kDownThreads = 256;
constexpr int kDieGroups = 8;       // blockIdx % 8: the compute-die of the block
constexpr int kSyncStride = 32;     // 32-bit words between counters (128 bytes)
constexpr uint32_t kNoLogit = 0xFFFFFFFFu;   // a speculative logit not written yet (a NaN no dot product gives)
constexpr int kSpecPolls = 8;                // re-reads of a speculative logit that had not landed
constexpr int kB1MaxRowsPerBlock = 16 * kWave;

// ------------------------------------------------------------ z = Q . h
// Block (j, g) computes z[b][jq] for the NQ rows jq = j * NQ .. of Q and the
// rows b of group g (NB rows from g * NB; up to 8 groups, so up to 64 rows
// in one launch). Its 256 threads read the rows of Q in 16-byte chunks, NL
// per thread per step of NL * 2048 columns (all of them and the matching
// chunks of the group's rows of h issued before the products); each wave
// sums its lanes, and thread (q, b) adds the four wave sums in a fixed order
// and rounds to bf16. Chunks past d read a clamped, valid address and are
// zeroed. (Four rows of Q per block, so that each chunk of h serves four
// products, measured slower at 64 rows: 9.1 against 8.5 us; the kernel is
// bound by the latency of its loads, not by L2 traffic.) Block 0 also zeroes
// `nsync` counters of the following score pass, and the blocks set its n_lgs
// speculative logits to kNoLogit ("not written yet").
template <int NB, int NQ, int NL>
__global__ void __launch_bounds__(kDownThreads) down_wide_kernel(const uint16_t* __restrict__ Q,
                                                                 const uint16_t* __restrict__ H, int r, int d,
                                                                 int B, uint16_t* __restrict__ Z,
                                                                 uint32_t* __restrict__ sync, int nsync,
                                                                 uint32_t* __restrict__ lgs, int n_lgs) {
  __shared__ float part[kDownThreads / kWave][NQ][NB];
  const int tid = threadIdx.x, wave = wave_id(), lane = tid & 63;
  const int j = blockIdx.x;
  if (blockIdx.y == 0) {
    if (j == 0 && tid < nsync) sync[tid * kSyncStride] = 0u;
    for (int e = j * kDownThreads + tid; e < n_lgs; e += gridDim.x * kDownThreads) lgs[e] = kNoLogit;
  }
  const int row0 = blockIdx.y * NB;
  H += (int64_t)row0 * d;
  Z += (int64_t)row0 * r;
  B -= row0;   // rows of this group (at least 1)
  const int j0 = j * NQ;
  float acc[NQ][NB];
#pragma unroll
  for (int a = 0; a < NQ; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = 0.f;
  for (int c0 = 0; c0 < d; c0 += NL * kDownThreads * 8) {
    int cols[NL];
    u32x4 qv[NQ][NL], hv[NB][NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int c = c0 + (t * kDownThreads + tid) * 8;
      cols[t] = c < d ? c : d - 8;
    }
#pragma unroll
    for (int a = 0; a < NQ; ++a)
#pragma unroll
      for (int t = 0; t < NL; ++t) qv[a][t] = load16(Q + (int64_t)(j0 + a < r ? j0 + a : j0) * d + cols[t]);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < NL; ++t) hv[b][t] = load16(H + (int64_t)(b < B ? b : 0) * d + cols[t]);
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const bool ok = c0 + (t * kDownThreads + tid) * 8 < d;
#pragma unroll
      for (int a = 0; a < NQ; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[a][b] = dot8_bf16(ok ? qv[a][t] : u32x4{0u, 0u, 0u, 0u}, hv[b][t], acc[a][b]);
    }
  }
#pragma unroll
  for (int a = 0; a < NQ; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float s = group_sum<kWave>(acc[a][b]);
      if (lane == 0) part[wave][a][b] = s;
    }
  __syncthreads();
  if (tid < NQ * NB) {
    const int a = tid / NB, b = tid % NB;
    if (b < B && j0 + a < r) {
      float z = part[0][a][b];
#pragma unroll
      for (int w = 1; w < kDownThreads / kWave; ++w) z += part[w][a][b];
      Z[(int64_t)b * r + j0 + a] = f32_to_bf16(z);
    }
  }
}

// ------------------------------------------------ device-coherent access
// The pass's blocks hand their results to its last block through memory.
// Device-scope relaxed atomic stores and loads are coherent at the device
// level (they do not stay in, or read from, one compute-die's write-back
// L2), so publishing needs no write-back of the L2: every wave's stores
// complete before the block's barrier (the explicit vmcnt wait), the
// block's ticket RMW follows the barrier, and the last block reads only
// after its ticket. A device-scope release fence would do the same through
// an L2 write-back, which costs far more per block.
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this wave's vector memory operations (its stores) completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// ------------------------------------------- one row: score, select, merge
constexpr int kB1List = 4;   // entries per slice list (min(4, k))
constexpr int kB1Spec = 2;   // of which the first ones get speculative logits

struct B1Smem {
  uint32_t hist[kHistBins];     // entries per bin of score images
  uint32_t wmin[kMergeWaves], wmax[kMergeWaves];
  int wcnt[kMergeWaves];
  alignas(16) uint64_t cand[kCandSlots];   // candidate keys
  float clog[kCandSlots];       // and their exact logits, where known
  uint8_t chas[kCandSlots];
  int csrc[kCandSlots];         // where its speculative logit lands (-1: none)
  int deep[kMaxLists];          // lists that may hold more than their entries
  uint64_t deep_key[kMaxLists]; // and the key of their last entry
  uint64_t tmp[kWave];
  float top_s[kWave];
  int top_i[kWave];
  int top_slot[kWave];          // candidate slot of each winner (-1: none)
  int rank[kWave];              // partial ranks of the first 64 candidates
  int miss[kWave];              // winners whose logit is still to compute
  int tops[kB1List];            // ids of the slice's best entries
  int rounds_done;              // of wave 0's selection rounds
  int ready;                    // waves whose list / raw-score stores have completed
  int decided;                  // the ticket has been taken (m.last is set)
  int n_cand, n_deep, n_miss, last;
};

// Appends the lanes' keys with `ps` to the candidate buffer, without a
// known logit (slots past its end are counted, not stored).
__device__ __forceinline__ void b1_push(B1Smem& m, bool ps, uint64_t key) {
  const int lane = threadIdx.x & 63;
  const unsigned long long mk = __ballot(ps);
  if (mk) {
    int base = 0;
    if (lane == 0) base = atomicAdd(&m.n_cand, __popcll(mk));
    base = __shfl(base, 0);
    const int slot = base + lanes_below(mk);
    if (ps && slot < kCandSlots) {
      m.cand[slot] = key;
      m.chas[slot] = 0;
      m.csrc[slot] = -1;
    }
  }
}

// Grid: n blocks of 512 threads (n <= 512, at most one per compute unit),
// block x owning the vocabulary slice [V*x/n, V*(x+1)/n) of at most E * 64
// rows, each of its 8 waves an eighth of it.
//  1. The slice's scores go to LDS (stream_scores).
//  2. Wave 0 takes the slice's L = min(4, k) best entries (SliceTop rounds)
//     and publishes them as candidate keys, entry j at keys[j * n + x]
//     (0 when the slice has fewer rows). With logits, waves 1 and 2 give
//     the first two entries their exact logits (lgs[j * n + x]),
//     speculatively: most of the row's winners are the first or second
//     entry of their slice. When L < k the other waves copy the scores to
//     raw[v] (the merge reads a slice's raw scores when more than L of its
//     entries may win).
//  3. Tickets: the block's RMW on its die group's counter, and the group's
//     last block one on the group counter. The block that completes the last
//     group is the last of the grid.
//  4. That block merges the lists (b1_merge) and writes idx, score and
//     logits, computing the logits of the few winners no slice had
//     computed (one wave per winner, the same row dot as the slices' and as
//     rescore_kernel, so the bits do not depend on who computed them).
// The k best of the n slice lists (L entries each, candidate keys at
// keys[j * n + p], read device-coherently) into m.top_s / m.top_i, with
// m.top_slot[r] the winner's candidate slot (its exact logit m.clog[slot]
// when m.chas[slot]); -1 when the winner came from the fallback.
//
// Take any bound T that at least k entries reach: an entry below T is
// preceded by k others and cannot win, and a list whose last entry is below
// T holds no more winners. T comes from a histogram of the entries' score
// images between the lowest and the highest head: the lower edge of the
// highest bin at which the count from the top reaches k (the edges are
// images, so at least k entries reach T). The entries that reach it (a few
// more than k) are the candidates; a list whose last entry reaches T may
// hold more, which its slice's raw scores give (rare). Each candidate's rank
// is the number of candidates that precede it, counted by every thread for
// its own candidate at once. Massive ties that overflow the candidate
// buffer fall back to a sequential selection over the raw scores (or, with
// lists as long as k, over the list entries).
__device__ __forceinline__ void b1_merge(B1Smem& m, const uint64_t* __restrict__ keys,
                                         const float* __restrict__ lgs, int n, int L,
                                         const float* __restrict__ raw, int64_t V, int k) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int p = threadIdx.x;
  uint64_t key[kB1List];
  float lg[kB1List];
#pragma unroll
  for (int j = 0; j < kB1List; ++j) {
    key[j] = p < n && j < L ? ld_dev(&keys[j * n + p]) : 0ull;
    lg[j] = lgs && p < n && j < L && j < kB1Spec ? ld_dev(&lgs[j * n + p]) : 0.f;
  }
  uint32_t img[kB1List];
#pragma unroll
  for (int j = 0; j < kB1List; ++j) img[j] = (uint32_t)(key[j] >> 32);   // 0 = empty
  {
    const uint32_t hk = img[0];
    const uint32_t wmn = wave_min_u32(hk ? hk : 0xFFFFFFFFu), wmx = wave_max_u32(hk);
    const int wc = __popcll(__ballot(hk != 0));
    if (lane == 0) {
      m.wmin[wave] = wmn;
      m.wmax[wave] = wmx;
      m.wcnt[wave] = wc;
    }
  }
  if (threadIdx.x < kHistBins) m.hist[threadIdx.x] = 0;
  if (threadIdx.x < kWave) m.rank[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    m.n_cand = 0;
    m.n_deep = 0;
  }
  __syncthreads();
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  int nheads = 0;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) {
    kmin = min(kmin, m.wmin[w]);
    kmax = max(kmax, m.wmax[w]);
    nheads += m.wcnt[w];
  }
  uint32_t T = 1u;
  if (nheads > k) {
    const uint32_t R = kmax - kmin;
    const int shift = R >= (uint32_t)kHistBins ? 24 - __clz(R) : 0;   // R >> shift < 256
#pragma unroll
    for (int j = 0; j < kB1List; ++j)
      if (img[j] >= kmin) atomicAdd(&m.hist[min((img[j] - kmin) >> shift, (uint32_t)kHistBins - 1)], 1u);
    __syncthreads();
    // every wave: counts from the top; lane l holds bins 255 - 4l - i
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = m.hist[kHistBins - 1 - 4 * lane - i] + (i ? c[i - 1] : 0u);
    const uint32_t above = wave_incl_scan_u32(c[3]) - c[3];
    const unsigned long long reach = __ballot(above + c[3] >= (uint32_t)k);
    const int l0 = __builtin_ctzll(reach);
    int i0 = 3;
#pragma unroll
    for (int i = 2; i >= 0; --i) i0 = above + c[i] >= (uint32_t)k ? i : i0;
    const int bstar = kHistBins - 1 - 4 * l0 - __builtin_amdgcn_readlane(i0, l0);
    T = kmin + ((uint32_t)bstar << shift);
  }
  {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < kB1List; ++j) cnt += img[j] != 0 && img[j] >= T;
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
    for (int j = 0; j < kB1List; ++j) {
      if (img[j] != 0 && img[j] >= T) {
        if (slot < kCandSlots) {
          m.cand[slot] = key[j];
          m.clog[slot] = lg[j];
          m.chas[slot] = lgs != nullptr && j < kB1Spec && __float_as_uint(lg[j]) != kNoLogit;
          m.csrc[slot] = lgs != nullptr && j < kB1Spec ? j * n + p : -1;
        }
        ++slot;
      }
    }
    if (raw && L >= 1 && img[L - 1] != 0 && img[L - 1] >= T) {
      const int dl = atomicAdd(&m.n_deep, 1);
      m.deep[dl] = p;
      m.deep_key[dl] = key[L - 1];
    }
  }
  __syncthreads();
  if (m.n_deep > 0) {
    // rare: the raw scores of a slice, below its list's last entry, that
    // reach T; one slice per wave at a time
    const int nd = m.n_deep;
    for (int dl = wave; dl < nd; dl += kMergeWaves) {
      const int q = m.deep[dl];
      const int64_t lo = V * q / n, hi = V * (q + 1) / n;
      const uint64_t below = m.deep_key[dl];
      for (int64_t c0 = lo; c0 < hi; c0 += 8 * kWave) {
        float xs[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) xs[t] = ld_dev(&raw[min(c0 + t * kWave + lane, hi - 1)]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t v = c0 + t * kWave + lane;
          const uint64_t kk = v < hi ? cand_key(xs[t], (int)v) : 0ull;
          b1_push(m, kk != 0 && kk < below && (uint32_t)(kk >> 32) >= T, kk);
        }
      }
    }
    __syncthreads();
  }
  const int nc = m.n_cand;
  if (nc <= kWave) {
    // rank of each candidate: the candidates that precede it, counted for
    // candidate `lane` by every wave over its eight (w * 8 .. w * 8 + 7)
    const uint64_t mine = lane < nc ? m.cand[lane] : 0ull;
    const u64x2* c2 = reinterpret_cast<const u64x2*>(m.cand + 8 * wave);
    int part = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u64x2 c = c2[j];
      part += (8 * wave + 2 * j < nc && c.x > mine) + (8 * wave + 2 * j + 1 < nc && c.y > mine);
    }
    if (lane < nc && part) atomicAdd(&m.rank[lane], part);
    __syncthreads();
    if (wave == 0) {
      const int r = lane < nc ? m.rank[lane] : kWave;
      if (r < k) {
        m.top_s[r] = key_score(mine);
        m.top_i[r] = key_id(mine);
        m.top_slot[r] = lane;
      }
      if (lane >= nc && lane < k) {   // fewer than k candidates: empty ranks
        m.top_s[lane] = neg_inf();
        m.top_i[lane] = kSentinelId;
        m.top_slot[lane] = -1;
      }
    }
  } else if (nc <= kCandSlots) {
    // rank of each candidate: the candidates that precede it
    if (p < nc) {
      const uint64_t mine = m.cand[p];
      int r = 0;
      const u64x2* c2 = reinterpret_cast<const u64x2*>(m.cand);
      int j = 0;
      for (; j + 2 <= nc; j += 2) {
        const u64x2 a = c2[j / 2];
        r += (a.x > mine) + (a.y > mine);
      }
      if (j < nc) r += m.cand[j] > mine;
      if (r < k) {
        m.top_s[r] = key_score(mine);
        m.top_i[r] = key_id(mine);
        m.top_slot[r] = p;
      }
    }
    if (p >= nc && p < k) {   // fewer than k candidates: empty ranks
      m.top_s[p] = neg_inf();
      m.top_i[p] = kSentinelId;
      m.top_slot[p] = -1;
    }
  } else if (wave == 0) {
    if (raw)
      select_keys_seq(V, k, [&](int64_t v) { return cand_key(ld_dev(&raw[v]), (int)v); }, m.top_s, m.top_i,
                      m.tmp);
    else
      select_keys_seq((int64_t)n * L, k, [&](int64_t e) { return ld_dev(&keys[e]); }, m.top_s, m.top_i, m.tmp);
    m.top_slot[lane] = -1;
  }
  __syncthreads();
}

template <int K, int E>
__global__ void __launch_bounds__(kMergeThreads) draft1_kernel(
    const uint16_t* __restrict__ P, const uint16_t* __restrict__ Z, int64_t V, int k, int L, int rescore,
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ H, int d, uint64_t* __restrict__ keys,
    float* __restrict__ lgs, float* __restrict__ raw, uint32_t* __restrict__ sync, int32_t* __restrict__ idx,
    float* __restrict__ score, float* __restrict__ logits) {
  __shared__ float sc[E * kWave];
  __shared__ B1Smem m;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int n = gridDim.x, x = blockIdx.x;
  const int64_t blo = V * x / n, bhi = V * (x + 1) / n;
  const int64_t wlo = blo + (bhi - blo) * wave / kMergeWaves;
  const int64_t whi = blo + (bhi - blo) * (wave + 1) / kMergeWaves;
  const int nrows = (int)(bhi - blo);

  // 1. scores of the slice
  if (threadIdx.x == 0) {
    m.rounds_done = 0;
    m.ready = 0;
    m.decided = 0;
  }
  stream_scores<K, 1>(P, Z, 1, blo, wlo, whi, sc, E * kWave);
  __syncthreads();

  // 2. the slice's best entries (wave 0, round by round); the exact logits
  // of the first kB1Spec of them, each started as soon as its round is done
  // (waves 1..kB1Spec wait on an LDS counter, which wave 0 always takes to
  // L); the raw copy (the remaining waves)
  auto lds_load = [](const int& v) { return __hip_atomic_load(&v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
  if (wave == 0) {
    SliceTop<E> st;
    st.load(sc, nrows);
    for (int r = 0; r < L; ++r) {
      const int id = st.round(r, (int)blo);
      if (lane == 0) {
        m.tops[r] = id;
        __hip_atomic_store(&m.rounds_done, r + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    if (lane < L) st_dev<uint64_t>(&keys[lane * n + x], st.my_i != kSentinelId ? cand_key(st.my_s, st.my_i) : 0ull);
  } else if (wave <= kB1Spec) {
    if (rescore && wave <= L) {
      while (lds_load(m.rounds_done) < wave) __builtin_amdgcn_s_sleep(1);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const int v = m.tops[wave - 1];
      if (v != kSentinelId) {
        const float lg = wave_row_dot<uint16_t>(W + (int64_t)v * d, H, d);
        if (lane == 0) st_dev(&lgs[(wave - 1) * n + x], lg);
      }
    }
  } else if (L < k) {
    for (int j = (wave - 1 - kB1Spec) * kWave + lane; j < nrows; j += (kMergeWaves - 1 - kB1Spec) * kWave)
      st_dev(&raw[blo + j], sc[j]);
  }

  // 3. tickets, once the lists and raw scores have landed. The speculative
  // logits are not waited for: the merge reads them again where they had
  // not landed (down_wide_kernel reset them to kNoLogit).
  if (wave != 1 && wave != 2) {
    wait_stores();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_fetch_add(&m.ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (threadIdx.x == 0) {
    while (lds_load(m.ready) < kMergeWaves - 2) __builtin_amdgcn_s_sleep(1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int g = x % kDieGroups;
    const uint32_t in_group = (uint32_t)((n - g + kDieGroups - 1) / kDieGroups);
    const uint32_t groups = (uint32_t)(n < kDieGroups ? n : kDieGroups);
    int is_last = 0;
    const uint32_t t = __hip_atomic_fetch_add(&sync[g * kSyncStride], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (t == in_group - 1) {
      const uint32_t t2 = __hip_atomic_fetch_add(&sync[kDieGroups * kSyncStride], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      is_last = t2 == groups - 1;
    }
    m.last = is_last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __hip_atomic_store(&m.decided, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  if (lane == 0)
    while (lds_load(m.decided) == 0) __builtin_amdgcn_s_sleep(1);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (!__builtin_amdgcn_readfirstlane(m.last)) return;   // block-uniform

  // 4. the merge, by the last block
  b1_merge(m, keys, rescore ? lgs : nullptr, n, L, L < k ? raw : nullptr, V, k);
  if (threadIdx.x < k) {
    const int r = threadIdx.x;
    const int v = m.top_i[r];
    idx[r] = v;
    if (score) score[r] = m.top_s[r];
  }
  if (!rescore) return;
  if (wave == 0) {
    const int r = lane;
    const int slot = r < k ? m.top_slot[r] : -1;
    const int v = r < k ? m.top_i[r] : kSentinelId;
    bool known = slot >= 0 && m.chas[slot];
    if (slot >= 0 && !known && m.csrc[slot] >= 0) {   // a speculative logit that had not landed yet
      const int src = m.csrc[slot];
      for (int polls = 0; polls < kSpecPolls && !known; ++polls) {
        const float g = ld_dev(&lgs[src]);
        if (__float_as_uint(g) != kNoLogit) {
          m.clog[slot] = g;
          known = true;
        } else {
          __builtin_amdgcn_s_sleep(4);
        }
      }
    }
    const bool need = v != kSentinelId && !known;
    const unsigned long long mk = __ballot(need);
    if (need) m.miss[lanes_below(mk)] = r;
    if (lane == 0) m.n_miss = __popcll(mk);
    if (r < k && !need) logits[r] = known ? m.clog[slot] : __builtin_nanf("");
  }
  __syncthreads();
  for (int t = wave; t < m.n_miss; t += kMergeWaves) {
    const int r = m.miss[t];
    const float lg = wave_row_dot<uint16_t>(W + (int64_t)m.top_i[r] * d, H, d);
    if (lane == 0) logits[r] = lg;
  }
}

// ================================================================ launchers

int b1_blocks(int64_t V, int n_cu) {
  int64_t n = (V + kWave - 1) / kWave;   // at least 64 rows per block
  if (n > n_cu) n = n_cu;
  if (n > kB1MaxLists) n = kB1MaxLists;
  return (int)(n < 1 ? 1 : n);
}

int b1_list_len(int k) { return k < kB1List ? k : kB1List; }

bool b1_path(int dtype, int64_t B, int64_t K, int64_t V, int n_cu) {
  if (dtype != 0 || B != 1 || K < 8 || K > 512 || (K & (K - 1)) != 0) return false;
  const int n = b1_blocks(V, n_cu);
  return (V + n - 1) / n <= kB1MaxRowsPerBlock;
}

// Chunks of 2048 columns per thread and step: the row in one step up to
// d = 8192, else four per step.
static int down_wide_loads(int d) {
  const int nl = (d + kDownThreads * 8 - 1) / (kDownThreads * 8);
  return nl < 4 ? nl : 4;
}

hipError_t launch_down_wide(const void* Q, const void* H, int r, int d, int64_t B, void* Z, uint32_t* sync,
                            int nsync, float* lgs, int n_lgs, hipStream_t stream) {
  if (B < 1 || B > kDownWideMaxB || nsync > kDownThreads || n_lgs < 0) return hipErrorInvalidValue;
  uint32_t* lg32 = reinterpret_cast<uint32_t*>(lgs);
  const int groups = (int)((B + kSmallB - 1) / kSmallB);
  // rows of Q per block: two above 48 rows of h at r <= 256 (8.0 -> 7.4 us
  // at 64 rows, r = 128; 12.6 -> 12.3 at r = 256; slower at 48 rows and
  // below, and at r = 512: 19.6 -> 22.2)
  const int nq = B > 48 && r <= 256 ? 2 : 1;
  const dim3 grid((unsigned)((r + nq - 1) / nq), (unsigned)groups), block(kDownThreads);
  const int nl = down_wide_loads(d);
  const uint16_t* q = (const uint16_t*)Q;
  const uint16_t* h = (const uint16_t*)H;
  uint16_t* z = (uint16_t*)Z;
#define LRH_DW(NB, NQ)                                                                                          \
  do {                                                                                                          \
    switch (nl) {                                                                                               \
      case 1: hipLaunchKernelGGL((down_wide_kernel<NB, NQ, 1>), grid, block, 0, stream, q, h, r, d, (int)B, z, sync, nsync, lg32, n_lgs); break; \
      case 2: hipLaunchKernelGGL((down_wide_kernel<NB, NQ, 2>), grid, block, 0, stream, q, h, r, d, (int)B, z, sync, nsync, lg32, n_lgs); break; \
      case 3: hipLaunchKernelGGL((down_wide_kernel<NB, NQ, 3>), grid, block, 0, stream, q, h, r, d, (int)B, z, sync, nsync, lg32, n_lgs); break; \
      default: hipLaunchKernelGGL((down_wide_kernel<NB, NQ, 4>), grid, block, 0, stream, q, h, r, d, (int)B, z, sync, nsync, lg32, n_lgs); break; \
    }                                                                                                           \
  } while (0)
  if (B == 1)
    LRH_DW(1, 1);
  else if (B == 2)
    LRH_DW(2, 1);
  else if (B <= 4)
    LRH_DW(4, 1);
  else if (nq == 2)
    LRH_DW(8, 2);
  else
    LRH_DW(8, 1);
#undef LRH_DW
  return hipGetLastError();
}

template <int K>
static hipError_t launch_draft1_k(const B1Args& a, hipStream_t stream, Timing t) {
  const int n = b1_blocks(a.V, a.n_cu);
  const int64_t rows = (a.V + n - 1) / n;
  const dim3 grid(n), block(kMergeThreads);
#define LRH_D1(E)                                                                                             \
  LRH_LAUNCH(t, (draft1_kernel<K, E>), grid, block, 0, stream, (const uint16_t*)a.P, (const uint16_t*)a.Z,      \
             a.V, a.k, a.L, a.logits != nullptr ? 1 : 0, (const uint16_t*)a.W, (const uint16_t*)a.H, a.d,      \
             a.keys, a.lgs, a.raw, a.sync, a.idx, a.score, a.logits)
  if (rows <= 4 * kWave)
    LRH_D1(4);
  else if (rows <= 10 * kWave)
    LRH_D1(10);
  else
    LRH_D1(16);
#undef LRH_D1
  return hipGetLastError();
}

hipError_t launch_draft1(const B1Args& a, hipStream_t stream, Timing t) {
  if (!b1_path(0, 1, a.K, a.V, a.n_cu) || a.k < 1 || a.k > kWave) return hipErrorInvalidValue;
  switch (a.K) {
    case 8: return launch_draft1_k<8>(a, stream, t);
    case 16: return launch_draft1_k<16>(a, stream, t);
    case 32: return launch_draft1_k<32>(a, stream, t);
    case 64: return launch_draft1_k<64>(a, stream, t);
    case 128: return launch_draft1_k<128>(a, stream, t);
    case 256: return launch_draft1_k<256>(a, stream, t);
    case 512: return launch_draft1_k<512>(a, stream, t);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace lrh
