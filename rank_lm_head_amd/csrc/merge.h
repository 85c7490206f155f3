// merge.h — the k best of a row's slice lists, and the exact row dot.
//
// After a score pass every draft row has n sorted lists (one per vocabulary
// slice) of its slice's L best ids. The pieces here find the row's k best
// overall in one block of 512 threads (one list per thread), for merge_kernel
// and for the last block of the batch-1 fused pass:
//
//  merge_collect     reads the leading entries of every list in one coalesced
//                    pass, finds a bound T that at least k of them reach (a
//                    histogram of score images) and gathers the entries that
//                    reach it (a few more than k) as candidate keys; lists
//                    whose last leading entry still reaches T are read further
//                    (their list, or their slice's scores: raw, or recomputed).
//  select_candidates ranks the candidates (wave 0).
//  select_raw_row    the fallback when ties flag more candidates than the
//                    buffer holds: the k best of the row's raw (or
//                    recomputed) scores.
//
// The order is the head's candidate order: higher score first, the lower id
// on equal scores ("EAGLE-4", section "Retrieve vocabulary candidates
// cheaply, then score them exactly", read as: the k best tokens, ties to the
// lower id).
#pragma once

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
// rounded up to 4, 8 or 10, so that no load is wasted on a short row);
// longer rows go in chunks of 10. Loads past d read a clamped, valid
// address and are zeroed, so none is predicated. For every U the lane's
// sum runs over its chunks in the same order, so every kernel that gives a
// candidate its exact logit through this function gets the same bits.
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
  return wave_row_dot_u<T, 10>(w, h, d);
}

// ---------------------------------------------------------------- merge
constexpr int kCandE = 8;                   // candidates per lane of wave 0
constexpr int kCandSlots = kCandE * kWave;
constexpr int kFront = 4;                   // leading entries of each list read up front
constexpr int kHistBins = 256;
constexpr int kRankSlots = 2 * kWave;       // candidates ranked directly

struct MergeSmem {
  uint32_t hist[kHistBins];   // front entries per bin of score images
  uint32_t wmin[kMergeWaves], wmax[kMergeWaves];
  int wcnt[kMergeWaves];
  uint64_t cand[kCandSlots];
  float spec[kCandSlots];     // exact logit of candidate slot j (this block's share)
  int slot_of[kWave];         // candidate slot of each winner
  uint64_t tmp[kRankSlots];
  int tslot[kRankSlots];
  float top_s[kWave];
  int top_i[kWave];
  int deep[kMaxLists];        // lists whose front entries all reach the bound
  uint64_t deep_key[kMaxLists];   // and the key of their last front entry
  int n_cand;
  int n_deep;
};

// Appends the lanes' keys with `ps` to the candidate buffer (slots past its
// end are counted, not stored).
__device__ __forceinline__ void push_cands(MergeSmem& m, bool ps, uint64_t key) {
  const int lane = threadIdx.x & 63;
  const unsigned long long mk = __ballot(ps);
  if (mk) {
    int base = 0;
    if (lane == 0) base = atomicAdd(&m.n_cand, __popcll(mk));
    base = __shfl(base, 0);
    const int slot = base + lanes_below(mk);
    if (ps && slot < kCandSlots) m.cand[slot] = key;
  }
}

// The scores of a row beyond its slice lists: the row's raw scores (raw),
// or, with raw == NULL and P != NULL, recomputed from P (V x K, bf16) and
// the row's z (K entries, bf16) on the matrix cores in the arithmetic of the
// score pass that made the lists (stream_mfma_tiles: per 16-row tile one
// v_mfma_f32_16x16x32_bf16 per 32 of K, accumulated in order from zero), so
// that a recomputed score equals the listed one bit for bit.
struct RowScores {
  const float* raw;
  const uint16_t* P;
  const uint16_t* z;
  int K;
};

// The row (0..63) whose recomputed score lane l holds after recompute64:
// column l & 15 of every output tile carries the same z, so lane l keeps
// output (l & 15) & 3 of tile (l & 15) >> 2, i.e. tile row 4 (l >> 4) + q.
__device__ __forceinline__ int recompute_row(int lane) {
  const int g = lane >> 4, col = lane & 15;
  return 16 * (col >> 2) + 4 * g + (col & 3);
}

// One wave: the scores of rows c0 + recompute_row(lane) (rows at or past hi
// are computed on row hi - 1 and are the caller's to drop).
__device__ __forceinline__ float recompute64(const RowScores& src, int64_t c0, int64_t hi) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, col = lane & 15;
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ks = src.K / 32;
  for (int t = 0; t < ks; ++t) {
    const u32x4 zb = load16(src.z + t * 32 + g * 8);
    u32x4 a[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int64_t row = min(c0 + 16 * c + col, hi - 1);
      a[c] = load16(src.P + row * src.K + t * 32 + g * 8);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[c]),
                                                       __builtin_bit_cast(bf16x8, zb), acc[c], 0, 0, 0);
  }
  float x = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) x = (col >> 2) == c && (col & 3) == q ? acc[c][q] : x;
  return x;
}

// Steps 1-2 of the merge of row b, by all 512 threads: list p (p < n <= 512)
// is read by thread p; entry j of list p sits at lists_s/i[lay.at(j, p)]. src (raw and P both NULL when L >= k) gives the
// row's scores, slice p being [V*p/n, V*(p+1)/n). Returns the candidate
// count (past kCandSlots: the buffer overflowed and only the count is right).
//
// Take any bound T that at least k list entries reach. Then an entry below
// T is preceded by k others and cannot win, and a list whose head is below T
// holds no winner. T comes from a histogram of the front entries' score
// images between the lowest and the highest head: the lower edge of the
// highest bin at which the count from the top reaches k. The edges are
// images, so at least k entries reach T. With k heads or fewer, T = 1 and
// every non-empty entry counts.
__device__ __forceinline__ int merge_collect(MergeSmem& m, const float* __restrict__ lists_s,
                                             const int* __restrict__ lists_i, int n, int L, ListLayout lay,
                                             const RowScores& src, int64_t V, int k) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int F = min(kFront, L);
  const int p = threadIdx.x;
  const int pc = min(p, n - 1);
  float fs[kFront];
  int fi[kFront];
#pragma unroll
  for (int j = 0; j < kFront; ++j) {
    const int jc = min(j, L - 1);
    fs[j] = lists_s[lay.at(jc, pc)];
    fi[j] = lists_i[lay.at(jc, pc)];
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
        if (slot < kCandSlots) {
          m.cand[slot] = cand_key(fs[j], fi[j]);
        }
        ++slot;
      }
    }
    // a slice whose last front entry reaches the bound may hold more: the
    // rest of its list (L > F), or its scores (lists shorter than k)
    const bool more = L > F || (L < k && (src.raw != nullptr || src.P != nullptr));
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
        for (int j0 = F; j0 < L; j0 += kWave) {
          const int j = j0 + lane;
          const int jc = min(j, L - 1);
          const float sc = lists_s[lay.at(jc, q)];
          const int id = j < L ? lists_i[lay.at(jc, q)] : kSentinelId;
          push_cands(m, reaches(sc, id), cand_key(sc, id));
        }
      } else {
        // the slice's scores below its list's last entry that reach T
        const int64_t lo = V * q / n, hi = V * (q + 1) / n;
        const uint64_t below = m.deep_key[dl];
        if (src.raw) {
          for (int64_t c0 = lo; c0 < hi; c0 += 8 * kWave) {
            float xs[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) xs[t] = src.raw[min(c0 + t * kWave + lane, hi - 1)];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int64_t v = c0 + t * kWave + lane;
              const uint64_t key = v < hi ? cand_key(xs[t], (int)v) : 0ull;
              push_cands(m, key != 0 && key < below && reaches(xs[t], (int)v), key);
            }
          }
        } else {
          for (int64_t c0 = lo; c0 < hi; c0 += kWave) {
            const float x = recompute64(src, c0, hi);
            const int64_t v = c0 + recompute_row(lane);
            const uint64_t key = v < hi ? cand_key(x, (int)v) : 0ull;
            push_cands(m, key != 0 && key < below && reaches(x, (int)v), key);
          }
        }
      }
    }
    __syncthreads();
  }
  return m.n_cand;
}

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

// Wave 0: the k best of `count` keys given by key_at(i) (0 = empty), taken
// 448 at a time, each chunk merged into the running best top_s / top_i
// (64 entries each; tmp is 64 words of LDS owned by the wave).
template <typename KeyAt>
__device__ __forceinline__ void select_keys_seq(int64_t count, int k, KeyAt key_at, float* top_s, int* top_i,
                                                uint64_t* tmp) {
  const int lane = threadIdx.x & 63;
  top_s[lane] = neg_inf();
  top_i[lane] = kSentinelId;
  for (int64_t c0 = 0; c0 < count; c0 += 7 * kWave) {
    uint64_t key[8];
#pragma unroll
    for (int e = 0; e < 7; ++e) {
      const int64_t v = c0 + e * kWave + lane;
      key[e] = v < count ? key_at(v) : 0ull;
    }
    key[7] = lane < k && top_i[lane] != kSentinelId ? cand_key(top_s[lane], top_i[lane]) : 0ull;
    wave_topk_emit<8>(key, k, tmp, top_s, top_i);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Wave 0, when ties flag more candidates than the buffer holds: the k best
// of the row's V scores, raw or recomputed (64 rows per recompute64, the
// rows of a chunk in recompute_row order).
__device__ __forceinline__ void select_raw_row(MergeSmem& m, const RowScores& src, int64_t V, int k) {
  if (src.raw) {
    const float* raw = src.raw;
    select_keys_seq(V, k, [&](int64_t v) { return cand_key(raw[v], (int)v); }, m.top_s, m.top_i, m.tmp);
    return;
  }
  const int lane = threadIdx.x & 63;
  m.top_s[lane] = neg_inf();
  m.top_i[lane] = kSentinelId;
  const int64_t perm = recompute_row(lane);
  for (int64_t c0 = 0; c0 < V; c0 += 7 * kWave) {
    uint64_t key[8];
#pragma unroll
    for (int e = 0; e < 7; ++e) {
      const int64_t r0 = c0 + e * kWave;
      key[e] = 0ull;
      if (r0 < V) {
        const float x = recompute64(src, r0, V);
        if (r0 + perm < V) key[e] = cand_key(x, (int)(r0 + perm));
      }
    }
    key[7] = lane < k && m.top_i[lane] != kSentinelId ? cand_key(m.top_s[lane], m.top_i[lane]) : 0ull;
    wave_topk_emit<8>(key, k, m.tmp, m.top_s, m.top_i);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

}  // namespace lrh
