// topk.h — candidate selection building blocks for the head's kernels.
//
// Order: (s1, i1) precedes (s2, i2) when s1 > s2, or s1 == s2 and i1 < i2
// (the k best tokens, ties to the lower id). Pieces:
//
//  * WaveSel: a wave's running best-k for up to NB draft rows, when the
//    wave's threshold is the same for all its lanes (a wave that owns whole
//    vocabulary rows). The list is kept sorted in registers (one pair per
//    lane), the k-th best in scalars, and rows that beat it are compacted
//    into an LDS buffer with a ballot; a full buffer is folded into the list
//    with a bitonic sort and a bitonic merge.
//
//  * wave_window_threshold / wave_topk_emit: the k best of up to a few
//    hundred keys held by one wave. A short bisection on the score values
//    finds a bound that between k and 64 keys reach; those are compacted
//    to LDS and each is placed by counting the keys that precede it, which
//    orders them as well (no sorting network on the hot path).
//
//  * wave_select_threshold: the exact k-th best by a full bisection, used
//    when ties keep the window from being reached.
//
//  * wave_top_few: the few best (a slice's leading entries) by repeated
//    wave-wide maxima of 32-bit score images.
//
//  * merge_lists_seq: a wave-wide fold of sorted lists, the fallback of the
//    merge kernel when too many entries tie at its threshold.
#pragma once

#include "device.h"

namespace lrh {

constexpr int kBuf = 64;            // per-row candidate buffer of a WaveSel

// ------------------------------------------------------------------ WaveSel
template <int NB>
struct WaveSel {
  float ls[NB];   // this lane's element of the sorted list
  int li[NB];
  float ts[NB];   // k-th best so far (wave-uniform)
  int ti[NB];
  int cnt[NB];    // buffered candidates (wave-uniform)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      ls[b] = neg_inf();
      li[b] = kSentinelId;
      ts[b] = neg_inf();
      ti[b] = kSentinelId;
      cnt[b] = 0;
    }
  }

  // Appends (s, v) of the lanes with `pass` to row b's buffer.
  __device__ __forceinline__ void push(int b, bool pass, float s, int v, float* bs, int* bi) {
    const unsigned long long m = __ballot(pass);
    if (m) {
      if (pass) {
        const int p = cnt[b] + lanes_below(m);
        bs[p] = s;
        bi[p] = v;
      }
      cnt[b] += __popcll(m);
    }
  }

  // Folds row b's buffer into its list and refreshes the k-th best.
  __device__ __forceinline__ void fold(int b, const float* bs, const int* bi, int k) {
    const int lane = threadIdx.x & 63;
    float s = neg_inf();
    int i = kSentinelId;
    if (lane < cnt[b]) {
      s = bs[lane];
      i = bi[lane];
    }
    bitonic_sort_desc(s, i);
    merge_reversed(s, i, __shfl(ls[b], kWave - 1 - lane), __shfl(li[b], kWave - 1 - lane));
    ls[b] = s;
    li[b] = i;
    ts[b] = readlane_f(s, k - 1);
    ti[b] = __builtin_amdgcn_readlane(i, k - 1);
    cnt[b] = 0;
  }
};

// ------------------------------------------------------- keys and counting
// A candidate as one 64-bit key: the order-preserving image of its score in
// the high word, the complement of its id in the low word. A larger key
// precedes a smaller one, exactly the candidate order; 0 marks an empty slot
// (every real key has a high word of at least 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t cand_key(float s, int id) {
  s = s + 0.0f;   // -0 and +0 are the same score
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ uint32_t order_key_inv(uint32_t u) {
  return (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
}
__device__ __forceinline__ float key_score(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ int wave_count(bool p) { return __popcll(__ballot(p)); }

// Wave-wide min / max of a 32-bit value: DPP inside each row of 16 lanes
// (pairs, quads, half rows, rows), then the four row results by readlane.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, Ctrl, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t rl(uint32_t x, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, lane);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));
  x = min(x, dpp_u32<0x4E>(x));
  x = min(x, dpp_u32<0x141>(x));
  x = min(x, dpp_u32<0x140>(x));
  return min(min(rl(x, 0), rl(x, 16)), min(rl(x, 32), rl(x, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u32<0xB1>(x));
  x = max(x, dpp_u32<0x4E>(x));
  x = max(x, dpp_u32<0x141>(x));
  x = max(x, dpp_u32<0x140>(x));
  return max(max(rl(x, 0), rl(x, 16)), max(rl(x, 32), rl(x, 48)));
}

// Inclusive prefix sum over the lanes of a wave (lane order): DPP row shifts
// by 1, 2, 4 and 8 inside each row of 16 lanes (lanes whose source falls
// outside the row add 0), then the totals of the rows below by readlane.
template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_shr_or_0(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_shr_or_0<0x111>(x);
  x += dpp_shr_or_0<0x112>(x);
  x += dpp_shr_or_0<0x114>(x);
  x += dpp_shr_or_0<0x118>(x);
  const int row = (threadIdx.x & 63) >> 4;
  const uint32_t r0 = rl(x, 15), r1 = rl(x, 31), r2 = rl(x, 47);
  x += row >= 1 ? r0 : 0u;
  x += row >= 2 ? r1 : 0u;
  x += row >= 3 ? r2 : 0u;
  return x;
}

// Wave-wide exact selection threshold over E keys per lane: returns T such
// that exactly min(k, #non-empty keys) keys satisfy key >= T.
//  1. Bisection on the score values inside [min, max] of the wave, counting
//     with ballots and stopping as soon as exactly k scores reach the bound.
//     The bound then separates the k-th and (k+1)-th scores, so a handful of
//     halvings of the value range usually suffice.
//  2. If the interval closes first (equal or adjacent scores at the
//     boundary), an exact search on the keys: their high words (score
//     images), then, among keys tied there, their low words (ids).
template <int E>
__device__ __forceinline__ uint64_t wave_select_threshold(const uint64_t (&key)[E], int k) {
  int valid = 0;
  float fmn = __builtin_inff(), fmx = -__builtin_inff();
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    valid += wave_count(key[e] != 0);
    sv[e] = key[e] != 0 ? key_score(key[e]) : -__builtin_inff();
    if (key[e] != 0) {
      fmn = fminf(fmn, sv[e]);
      fmx = fmaxf(fmx, sv[e]);
    }
  }
  if (valid <= k) return 1;
  fmn = __uint_as_float(order_key_inv(wave_min_u32(order_key(fmn))));
  fmx = __uint_as_float(order_key_inv(wave_max_u32(order_key(fmx))));
  // count(s >= flo) >= k > count(s >= fhi); flo = min reaches all valid
  float flo = fmn, fhi = fmx;
  int cnt_hi = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) cnt_hi += wave_count(sv[e] >= fhi);
  if (cnt_hi == k) return (uint64_t)order_key(fhi) << 32;
  if (cnt_hi < k) {
#pragma unroll 1
    for (int it = 0; it < 64; ++it) {
      const float mid = 0.5f * (flo + fhi);
      if (!(mid > flo && mid < fhi)) break;   // adjacent floats
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += wave_count(sv[e] >= mid);
      if (cnt == k) return (uint64_t)order_key(mid) << 32;
      if (cnt > k)
        flo = mid;
      else
        fhi = mid;
    }
  }
  // exact search on the keys inside the bracket found so far:
  // count(key high word >= lo) >= k > count(high word >= hi)
  uint32_t kh[E];
#pragma unroll
  for (int e = 0; e < E; ++e) kh[e] = (uint32_t)(key[e] >> 32);
  uint32_t lo = order_key(flo);
  const uint64_t hi0 = cnt_hi < k ? (uint64_t)order_key(fhi) : (uint64_t)order_key(fmx) + 1;
  uint64_t hi = hi0;
#pragma unroll 1
  while (hi - lo > 1) {
    const uint32_t mid = (uint32_t)(lo + (hi - lo) / 2);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += wave_count(key[e] != 0 && kh[e] >= mid);
    if (cnt >= k) {
      lo = mid;
      if (cnt == k) return (uint64_t)lo << 32;
    } else {
      hi = mid;
    }
  }
  // lo is the k-th largest high word and several keys share it
  int above = 0;
  uint32_t lmn = 0xFFFFFFFFu, lmx = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    above += wave_count(key[e] != 0 && kh[e] > lo);
    if (key[e] != 0 && kh[e] == lo) {
      lmn = min(lmn, (uint32_t)key[e]);
      lmx = max(lmx, (uint32_t)key[e]);
    }
  }
  const int need = k - above;
  uint32_t llo = wave_min_u32(lmn);
  uint64_t lhi = (uint64_t)wave_max_u32(lmx) + 1;
#pragma unroll 1
  while (lhi - llo > 1) {
    const uint32_t mid = (uint32_t)(llo + (lhi - llo) / 2);
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cnt += wave_count(key[e] != 0 && kh[e] == lo && (uint32_t)key[e] >= mid);
    if (cnt >= need) {
      llo = mid;
      if (cnt == need) break;
    } else {
      lhi = mid;
    }
  }
  return ((uint64_t)lo << 32) | llo;
}

// ------------------------------------------------ windowed selection
// A bound T with k <= #{key >= T} <= cap (cap <= 64) over E keys per lane,
// found by bisection on the score values: only the window has to be hit,
// not the gap between the k-th and (k+1)-th score, so a few halvings of the
// wave's value range suffice. Returns 1 (every non-empty key) when at most
// cap keys are non-empty; falls back to the exact k-th key when ties at the
// boundary keep the window out of reach.
template <int E>
__device__ __forceinline__ uint64_t wave_window_threshold(const uint64_t (&key)[E], int k, int cap) {
  int valid = 0;
  float fmn = __builtin_inff(), fmx = -__builtin_inff();
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    valid += wave_count(key[e] != 0);
    sv[e] = key[e] != 0 ? key_score(key[e]) : -__builtin_inff();
    if (key[e] != 0) {
      fmn = fminf(fmn, sv[e]);
      fmx = fmaxf(fmx, sv[e]);
    }
  }
  if (valid <= cap) return 1;
  fmn = __uint_as_float(order_key_inv(wave_min_u32(order_key(fmn))));
  fmx = __uint_as_float(order_key_inv(wave_max_u32(order_key(fmx))));
  // invariant: count(s >= flo) > cap and count(s >= fhi) < k
  float flo = fmn, fhi = fmx;
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += wave_count(sv[e] >= fhi);
  if (c >= k) {
    if (c <= cap) return (uint64_t)order_key(fhi) << 32;
  } else {
#pragma unroll 1
    for (int it = 0; it < 64; ++it) {
      const float mid = 0.5f * (flo + fhi);
      if (!(mid > flo && mid < fhi)) break;
      c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += wave_count(sv[e] >= mid);
      if (c >= k && c <= cap) return (uint64_t)order_key(mid) << 32;
      if (c > cap)
        flo = mid;
      else
        fhi = mid;
    }
  }
  return wave_select_threshold<E>(key, k);
}

// Places the n <= 64 distinct keys tmp[0 .. n) by counting, for each, the
// keys that precede it; tmp[n .. round_up(n, 8)) must hold zeros (an empty
// key precedes nothing). The keys are read eight at a time with broadcast
// LDS reads. The k best go to out_s/out_i[r * stride] (r = 0 .. k-1) in
// candidate order and empty entries fill ranks n .. k-1 when n < k.
// Returns the lane's rank (k or more when it holds no winner).
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int wave_rank_emit(const uint64_t* tmp, int n, int k, float* __restrict__ out_s,
                                              int* __restrict__ out_i, int64_t stride = 1) {
  const int lane = threadIdx.x & 63;
  const uint64_t mine = lane < n ? tmp[lane] : 0ull;
  const u64x2* t2 = reinterpret_cast<const u64x2*>(tmp);
  int r = 0;
  for (int t = 0; t < n; t += 16) {
    // 16 keys (8 broadcast reads) in flight; past n + 8 the reads hit
    // slots that may hold stale keys, so the second half is counted only
    // when it lies below round_up(n, 8)
    u64x2 a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = t2[t / 2 + q];
#pragma unroll
    for (int q = 0; q < 4; ++q) r += (a[q].x > mine) + (a[q].y > mine);
    if (t + 8 < n) {
#pragma unroll
      for (int q = 4; q < 8; ++q) r += (a[q].x > mine) + (a[q].y > mine);
    }
  }
  if (lane < n) {
    if (r < k) {
      out_s[r * stride] = key_score(mine);
      out_i[r * stride] = key_id(mine);
    }
  } else {
    r = k;
    if (lane < k) {
      out_s[lane * stride] = neg_inf();
      out_i[lane * stride] = kSentinelId;
    }
  }
  return r;
}

// Zeros tmp[n .. round_up(n, 8)) (n <= 64) and makes the wave's LDS writes
// visible to its own later reads.
__device__ __forceinline__ void pad_keys(uint64_t* tmp, int n) {
  const int lane = threadIdx.x & 63;
  if (lane >= n && lane < ((n + 7) & ~7)) tmp[lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// As wave_rank_emit for n <= 128 distinct keys, two per lane (tmp[lane] and
// tmp[lane + 64]); tmp[n .. round_up(n, 8)) must hold zeros. The ranks of
// the lane's two keys go to r[0], r[1] (k or more: no winner); k <= 64.
__device__ __forceinline__ void wave_rank_emit2(const uint64_t* tmp, int n, int k, float* __restrict__ out_s,
                                                int* __restrict__ out_i, int (&r)[2]) {
  const int lane = threadIdx.x & 63;
  uint64_t mine[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) mine[h] = lane + h * kWave < n ? tmp[lane + h * kWave] : 0ull;
  const u64x2* t2 = reinterpret_cast<const u64x2*>(tmp);
  r[0] = r[1] = 0;
  for (int t = 0; t < n; t += 16) {
    u64x2 a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = t2[t / 2 + q];
    const int qn = t + 8 < n ? 8 : 4;   // past round_up(n, 8) the slots may be stale
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < qn) {
#pragma unroll
        for (int h = 0; h < 2; ++h) r[h] += (a[q].x > mine[h]) + (a[q].y > mine[h]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (lane + h * kWave < n) {
      if (r[h] < k) {
        out_s[r[h]] = key_score(mine[h]);
        out_i[r[h]] = key_id(mine[h]);
      }
    } else {
      r[h] = k;
    }
  }
  if (lane >= n && lane < k) {   // fewer than k keys: empty ranks n .. k-1
    out_s[lane] = neg_inf();
    out_i[lane] = kSentinelId;
  }
}

// The k best of E keys per lane (distinct where non-empty), in candidate
// order, to out_s/out_i[r * stride] (r = 0 .. k-1); `tmp` is 64 words of
// LDS owned by the wave.
template <int E>
__device__ __forceinline__ void wave_topk_emit(const uint64_t (&key)[E], int k, uint64_t* tmp,
                                               float* __restrict__ out_s, int* __restrict__ out_i,
                                               int64_t stride = 1) {
  const uint64_t T = wave_window_threshold<E>(key, k, kWave);
  int n = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool sel = key[e] != 0 && key[e] >= T;
    const unsigned long long m = __ballot(sel);
    if (sel) {
      const int p = n + lanes_below(m);
      if (p < kWave) tmp[p] = key[e];
    }
    n += __popcll(m);
  }
  n = min(n, kWave);
  pad_keys(tmp, n);
  wave_rank_emit(tmp, n, k, out_s, out_i, stride);
}

// ------------------------------------------------- a few best by argmax
// The best entries of a slice's n <= E * 64 scores held in LDS (entry j at
// sc[j], token id id0 + j), one per round, in candidate order. Entry
// j = e * 64 + lane sits in lane `lane` as element e, so within a lane a
// lower e is a lower id. Each round takes the wave-wide maximum of the
// 32-bit score images (each lane offers its best element, the lowest e among
// equal ones), then the lanes holding it: almost always one, and otherwise
// the lowest id among them (smallest e, then lowest lane). The winner's
// element is cleared; round r leaves the winner in lane r (my_s, my_i).
template <int E>
struct SliceTop {
  uint32_t h[E];   // 0 = empty (no finite score maps to 0)
  float my_s;
  int my_i;

  __device__ __forceinline__ void load(const float* sc, int n) {
    const int lane = threadIdx.x & 63;
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = sc[min(e * kWave + lane, n - 1)];
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = e * kWave + lane < n ? order_key(v[e] + 0.0f) : 0u;
    my_s = neg_inf();
    my_i = kSentinelId;
  }

  // Round r; returns the winner's id (wave-uniform), or kSentinelId when
  // the slice has no entries left.
  __device__ __forceinline__ int round(int r, int id0) {
    const int lane = threadIdx.x & 63;
    uint32_t best = h[0];
    int be = 0;
#pragma unroll
    for (int e = 1; e < E; ++e) {
      const bool t = h[e] > best;
      best = t ? h[e] : best;
      be = t ? e : be;
    }
    const uint32_t M = wave_max_u32(best);
    if (M == 0) return kSentinelId;
    unsigned long long mk = __ballot(best == M);
    if (mk & (mk - 1)) {   // equal scores in several lanes
      const uint32_t me = wave_min_u32(best == M ? (uint32_t)be : 0xFFu);
      mk = __ballot(best == M && (uint32_t)be == me);
    }
    const int wl = __builtin_ctzll(mk);
    const int we = __builtin_amdgcn_readlane(be, wl);
#pragma unroll
    for (int e = 0; e < E; ++e) h[e] = (lane == wl && e == we) ? 0u : h[e];
    const int id = id0 + we * kWave + wl;
    if (lane == r) {
      my_s = __uint_as_float(order_key_inv(M));
      my_i = id;
    }
    return id;
  }
};

// The L best (L <= 64) of a slice's n <= E * 64 scores held in LDS, in
// candidate order, to out_s/out_i[r * stride] for r < L; ranks past n get
// empty entries.
template <int E>
__device__ __forceinline__ void wave_top_few(const float* sc, int n, int id0, int L, float* __restrict__ out_s,
                                             int* __restrict__ out_i, int64_t stride) {
  const int lane = threadIdx.x & 63;
  SliceTop<E> st;
  st.load(sc, n);
  for (int r = 0; r < L; ++r)
    if (st.round(r, id0) == kSentinelId) break;   // fewer than L entries
  if (lane < L) {
    out_s[lane * stride] = st.my_s;
    out_i[lane * stride] = st.my_i;
  }
}

// ------------------------------------------------------- sequential merge
// Where entry j of list p of a row's n sorted lists sits: depth-major (entry
// j of all lists together: entry stride n, list stride 1) or row-major (a
// list's entries together: entry stride 1, list stride = its length).
struct ListLayout {
  int64_t entry_stride, list_stride;
  __device__ __forceinline__ int64_t at(int j, int p) const { return j * entry_stride + p * list_stride; }
};

// Wave-wide fallback: folds every list into (s, i), the running best 64 in
// candidate order, skipping lists whose best entry does not beat the running
// k-th.
__device__ __forceinline__ void merge_lists_seq(const float* ps, const int* pi, int n, int k, ListLayout lay,
                                                float& s, int& i) {
  const int lane = threadIdx.x & 63;
  s = neg_inf();
  i = kSentinelId;
  const int j = kWave - 1 - lane;
  for (int p = 0; p < n; ++p) {
    const float head = ps[lay.at(0, p)];
    const int head_i = pi[lay.at(0, p)];
    const float ks = readlane_f(s, k - 1);
    const int ki = __builtin_amdgcn_readlane(i, k - 1);
    if (!precedes(head, head_i, ks, ki)) continue;
    float os = neg_inf();
    int oi = kSentinelId;
    if (j < k) {
      os = ps[lay.at(j, p)];
      oi = pi[lay.at(j, p)];
    }
    merge_reversed(s, i, os, oi);
  }
}

}  // namespace lrh
