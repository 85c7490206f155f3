// lrhead.hip — host side of the C ABI in include/lrhead.h.
//
// Every entry point validates its arguments on the host before it touches
// HIP, then enqueues the stage kernels on the caller's stream and returns.
// Nothing here allocates device memory or synchronises: the caller's
// workspace holds z and the per-slice candidate lists.
#include "lrhead.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>

#include "launch.h"

struct lrhead_s {
  uint32_t magic;
  int dtype;
  int64_t V, d, r, B_max;
  int k_max;
  const void* Q;
  const void* P;
  const void* W;
  char* ws;
  size_t ws_bytes;
  void* z;          // B_max x r, weight dtype
  float* part_s;    // candidate lists: rows x slices x k_max
  int* part_i;
  float* raw;       // raw scores of the streaming path: min(B_max, 8) x V
  uint64_t* b1_keys;  // one-row pass: slice lists (candidate keys)
  float* b1_lgs;      // one-row pass: their speculative exact logits
  uint32_t* sync;     // one-row pass: completion counters
  int n_cu;           // compute units of the device
  bool batch;       // bf16 with B_max > 4: the GEMM path's scratch exists
  lrh::BatchScratch bw;
  hipEvent_t ev_before;  // optional events attached to the score pass: its start
  hipEvent_t ev_after;   // and its end
};

static __device__ __align__(256) unsigned char scratch[size_t(LRHEAD_STATIC_SCRATCH_MB) << 20];

namespace {

constexpr uint32_t kMagic = 0x4c524844u;  // "LRHD"
constexpr int64_t kDownGemmRows = 256;     // rows from which z = Q . h may run on the GEMM kernel
constexpr int64_t kDownSplitMaxElems = 65536;   // ... when B * r is above this
// From this many (row, winner) pairs on, the merge rescores only the
// winners, after the ranking: its speculative rescoring of every candidate
// (a few more than k per row) reads more of W than it hides once many rows
// keep the chip busy. Cold calls at r = 128, speculative against not: k = 32:
// 45.5 against 38.6 us at 64 rows, 31.9 against 28.9 at 32, 27.3 against
// 28.0 at 24; k = 64: 29.2 against 26.1 at 16 rows, 24.1 against 25.5 at
// 12; k = 8: 32.6 against 33.7 at 64 rows. (A separate rescoring launch
// after a ranking-only merge measured 40.1 us at 64 rows, k = 32.)
constexpr int64_t kSpeculatePairsBelow = 1024;
constexpr int64_t kBMaxLimit = int64_t(1) << 20;

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LRHEAD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
size_t elem_bytes(int dtype) { return dtype == LRHEAD_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Layout {
  size_t z, part_s, part_i, raw, b1_keys, b1_lgs, sync, batch, total;
};

// Most candidate lists any call with B <= B_max writes (B x slices), over
// both the streaming and the matrix-core selection.
int64_t max_list_rows(int64_t B_max, int64_t V) {
  int64_t best = 0;
  for (int64_t B = 1; B <= B_max; ++B) {
    int64_t rows = B * lrh::plan_vsplit(B, V);
    if (B <= lrh::kRowsMaxB) {
      const int64_t small = B * lrh::small_blocks(V);
      if (small > rows) rows = small;
    }
    if (rows > best) best = rows;
  }
  return best;
}

Layout layout(int dtype, int64_t V, int64_t r, int64_t B_max, int k_max) {
  Layout L;
  L.z = 0;
  const size_t zb = align256(size_t(B_max) * size_t(r) * elem_bytes(dtype));
  // the merge reads whole 16-byte chunks, up to 12 bytes past the last list
  const size_t lists = align256(size_t(max_list_rows(B_max, V)) * size_t(k_max) * 4 + 16);
  L.part_s = zb;
  L.part_i = zb + lists;
  // raw scores of the streaming path (bf16 heads, B <= kSmallB rows)
  const int64_t raw_rows = dtype == LRHEAD_BF16 ? (B_max < lrh::kSmallB ? B_max : lrh::kSmallB) : 0;
  L.raw = zb + 2 * lists;
  L.b1_keys = L.raw + align256(size_t(raw_rows) * size_t(V) * 4);
  L.b1_lgs = L.b1_keys + align256(size_t(lrh::kB1MaxLists) * lrh::kB1MaxList * 8);
  L.sync = L.b1_lgs + align256(size_t(lrh::kB1MaxLists) * lrh::kB1MaxList * 4);
  L.batch = L.sync + align256(size_t(lrh::kB1Counters) * 128);
  L.total = L.batch;
  if (lrh::batch_path(dtype, B_max)) L.total += align256(lrh::batch_scratch_bytes(V, B_max));
  return L;
}

int check_shapes(int dtype, int64_t V, int64_t d, int64_t r, int64_t B_max, int k_max) {
  if (dtype != LRHEAD_BF16 && dtype != LRHEAD_FP32) return fail(LRHEAD_EDTYPE, "unknown dtype %d", dtype);
  if (V < 1 || V > INT32_MAX) return fail(LRHEAD_ERANGE, "V = %lld outside [1, 2^31)", (long long)V);
  if (d < 8 || d > LRHEAD_D_MAX || d % 8) return fail(LRHEAD_ERANGE, "d = %lld: need a multiple of 8 in [8, %d]", (long long)d, LRHEAD_D_MAX);
  if (r < 8 || r > LRHEAD_R_MAX || r % 8) return fail(LRHEAD_ERANGE, "r = %lld: need a multiple of 8 in [8, %d]", (long long)r, LRHEAD_R_MAX);
  if (B_max < 1 || B_max > kBMaxLimit) return fail(LRHEAD_ERANGE, "B_max = %lld outside [1, 2^20]", (long long)B_max);
  if (k_max < 1 || k_max > LRHEAD_K_MAX || k_max > V)
    return fail(LRHEAD_ERANGE, "k_max = %d outside [1, min(%d, V)]", k_max, LRHEAD_K_MAX);
  return LRHEAD_OK;
}

int check_handle(const lrhead_s* h) {
  if (!h || h->magic != kMagic) return fail(LRHEAD_EINVAL, "invalid handle");
  return LRHEAD_OK;
}

int check_rows(const lrhead_s* h, const void* H, int64_t B) {
  if (B < 0 || B > h->B_max) return fail(LRHEAD_ERANGE, "B = %lld outside [0, B_max = %lld]", (long long)B, (long long)h->B_max);
  if (B > 0 && !H) return fail(LRHEAD_EINVAL, "H is NULL");
  if (!aligned16(H)) return fail(LRHEAD_EALIGN, "H is not 16-byte aligned");
  return LRHEAD_OK;
}

int check_k(const lrhead_s* h, int k) {
  if (k < 1 || k > h->k_max) return fail(LRHEAD_ERANGE, "k = %d outside [1, k_max = %d]", k, h->k_max);
  return LRHEAD_OK;
}

int check_out(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(LRHEAD_EINVAL, "%s is NULL", name) : LRHEAD_OK;
  if (!aligned16(p)) return fail(LRHEAD_EALIGN, "%s is not 16-byte aligned", name);
  return LRHEAD_OK;
}

#define LRH_TRY(x)            \
  do {                        \
    const int rc_ = (x);      \
    if (rc_ != LRHEAD_OK) return rc_; \
  } while (0)

#define LRH_HIP(x, what)                 \
  do {                                   \
    const hipError_t e_ = (x);           \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// The caller's profiling events, attached to the score pass's dispatch.
lrh::Timing timing(const lrhead_s* h) { return lrh::Timing{h->ev_before, h->ev_after}; }

// Down-projection, score pass with per-slice selection, and the merge of
// the slice lists; with `logits`, the merge also rescores the winners.
int enqueue_head(lrhead_s* h, const void* H, int64_t B, int k, int32_t* idx, float* score, float* logits,
                 hipStream_t s) {
  if (lrh::b1_path(h->dtype, B, h->r, h->V, h->n_cu)) {
    // one row: the down-projection (which also resets the pass's counters),
    // then a single pass that scores, selects, merges and rescores
    LRH_HIP(lrh::launch_down_wide(h->Q, H, (int)h->r, (int)h->d, B, h->z, h->sync, lrh::kB1Counters, h->b1_lgs,
                                  2 * lrh::b1_blocks(h->V, h->n_cu), s),
            "down-projection launch");
    lrh::B1Args a;
    a.P = h->P;
    a.Z = h->z;
    a.V = h->V;
    a.K = (int)h->r;
    a.k = k;
    a.L = lrh::b1_list_len(k);
    a.W = h->W;
    a.H = H;
    a.d = (int)h->d;
    a.keys = h->b1_keys;
    a.lgs = h->b1_lgs;
    a.raw = h->raw;
    a.sync = h->sync;
    a.n_cu = h->n_cu;
    a.idx = idx;
    a.score = score;
    a.logits = logits;
    LRH_HIP(lrh::launch_draft1(a, s, timing(h)), "score/selection launch");
    return LRHEAD_OK;
  }
  const bool rows = lrh::rows_path(h->dtype, B, h->r, h->V);
  const bool streaming = rows || lrh::small_path(h->dtype, B, h->r, h->V);
  if (!streaming && lrh::batch_path(h->dtype, B)) {
    // many rows. Up to 64 rows the down-projection takes one block per row
    // of Q and group of 8 rows (one launch); above that it is a GEMM worth
    // the pipelined kernel. The sparse score array is written only later in
    // the call, so the
    // split down-projection keeps its partial sums there when they fit.
    // Measured crossover: the split kernel is faster up to B * r = 65536
    // (B = 256 at r = 256: 144 against 149 us per call; B = 512 at r = 256:
    // 219 against 209 us).
    const size_t part_bytes = size_t(lrh::down_split_parts((int)h->d)) * size_t(B) * size_t(h->r) * 4;
    if (B <= lrh::kDownWideMaxB)
      LRH_HIP(lrh::launch_down_wide(h->Q, H, (int)h->r, (int)h->d, B, h->z, nullptr, 0, nullptr, 0, s),
              "down-projection launch");
    else if (B >= kDownGemmRows && B * h->r > kDownSplitMaxElems)
      LRH_HIP(lrh::launch_down_gemm(h->Q, H, (int)h->r, (int)h->d, B, h->z, h->bw.S, h->bw.S_bytes, s),
              "down-projection launch");
    else if (part_bytes <= h->bw.S_bytes)
      LRH_HIP(lrh::launch_down_split(h->Q, H, (int)h->r, (int)h->d, B, h->z, h->bw.S, s), "down-projection launch");
    else
      LRH_HIP(lrh::launch_down(h->dtype, h->Q, H, (int)h->r, (int)h->d, B, h->z, s), "down-projection launch");
    LRH_HIP(lrh::launch_batch_select(h->P, h->z, h->V, (int)h->r, B, k, h->bw, idx, score, s, timing(h)),
            "score/selection launch");
    if (logits)
      LRH_HIP(lrh::launch_rescore(h->dtype, h->W, H, idx, B, k, h->V, (int)h->d, logits, s), "rescore launch");
    return LRHEAD_OK;
  }
  int n_lists, list_len = k;
  const float* raw = nullptr;
  if (streaming) {
    LRH_HIP(lrh::launch_down_wide(h->Q, H, (int)h->r, (int)h->d, B, h->z, nullptr, 0, nullptr, 0, s),
            "down-projection launch");
    if (rows) {
      // no raw scores: the merge recomputes a slice it needs more of
      LRH_HIP(lrh::launch_select_rows(h->P, h->z, h->V, (int)h->r, B, k, h->part_s, h->part_i, s, timing(h)),
              "score/selection launch");
    } else {
      LRH_HIP(lrh::launch_select_small(h->P, h->z, h->V, (int)h->r, B, k, h->part_s, h->part_i, h->raw, s,
                                       timing(h)),
              "score/selection launch");
      raw = h->raw;
    }
    n_lists = lrh::small_blocks(h->V);
    list_len = lrh::small_list_len(k);
  } else {
    LRH_HIP(lrh::launch_down(h->dtype, h->Q, H, (int)h->r, (int)h->d, B, h->z, s), "down-projection launch");
    n_lists = lrh::plan_vsplit(B, h->V);
    LRH_HIP(lrh::launch_select(h->dtype, h->P, h->z, h->V, (int)h->r, B, k, n_lists, h->part_s, h->part_i, s,
                               timing(h)),
            "score/selection launch");
  }
  LRH_HIP(lrh::launch_merge(h->dtype, h->part_s, h->part_i, n_lists, list_len, rows, raw, rows ? h->P : nullptr,
                            rows ? h->z : nullptr, (int)h->r, h->V, B, k, h->W, H, (int)h->d, idx, score, logits,
                            B * k < kSpeculatePairsBelow, s),
          "merge launch");
  return LRHEAD_OK;
}

// The checks and settings a handle needs from the current device: it must be
// gfx950; the GEMM kernels of row batches get their LDS limit raised; the
// one-row pass sizes its grid by the compute units.
int device_setup(int dtype, int64_t B_max, int* n_cu) {
  int dev = 0;
  LRH_HIP(hipGetDevice(&dev), "hipGetDevice");
  hipDeviceProp_t prop;
  LRH_HIP(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(LRHEAD_EDEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
  if (lrh::batch_path(dtype, B_max)) LRH_HIP(lrh::batch_init(), "GEMM kernel set-up");
  LRH_HIP(hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev), "hipDeviceGetAttribute");
  return LRHEAD_OK;
}

void fill_handle(lrhead_s* h, int dtype, int64_t V, int64_t d, int64_t r, const void* Q, const void* P,
                 const void* W, int64_t B_max, int k_max, void* workspace, size_t workspace_bytes, int n_cu) {
  const Layout L = layout(dtype, V, r, B_max, k_max);
  h->magic = kMagic;
  h->dtype = dtype;
  h->V = V;
  h->d = d;
  h->r = r;
  h->B_max = B_max;
  h->k_max = k_max;
  h->Q = Q;
  h->P = P;
  h->W = W;
  h->ws = static_cast<char*>(workspace);
  h->ws_bytes = workspace_bytes;
  h->z = h->ws + L.z;
  h->part_s = reinterpret_cast<float*>(h->ws + L.part_s);
  h->part_i = reinterpret_cast<int*>(h->ws + L.part_i);
  h->raw = reinterpret_cast<float*>(h->ws + L.raw);
  h->b1_keys = reinterpret_cast<uint64_t*>(h->ws + L.b1_keys);
  h->b1_lgs = reinterpret_cast<float*>(h->ws + L.b1_lgs);
  h->sync = reinterpret_cast<uint32_t*>(h->ws + L.sync);
  h->n_cu = n_cu;
  h->batch = lrh::batch_path(dtype, B_max);
  h->bw = h->batch ? lrh::batch_scratch(h->ws + L.batch, V, B_max) : lrh::BatchScratch{};
  h->ev_before = nullptr;
  h->ev_after = nullptr;
}

// ------------------------------------------------- allocation-free variant
// The workspace of lrhead_draft_static is `scratch` (file scope, below the
// namespace): one copy per GPU, resident until the process ends. In host
// code its name only stands for the symbol; its address on a device comes
// from hipGetSymbolAddress with that device current, looked up once per
// device and kept.
constexpr size_t kStaticScratchBytes = size_t(LRHEAD_STATIC_SCRATCH_MB) << 20;
constexpr int kMaxDevices = 64;
struct StaticDevice {
  bool ready;
  void* ptr;   // device address of `scratch` on this device
  int n_cu;
};
std::mutex g_static_mu;
StaticDevice g_static[kMaxDevices];

int static_device(int dtype, int64_t B, void** ptr, int* n_cu) {
  int dev = 0;
  LRH_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LRHEAD_EDEVICE, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& sd = g_static[dev];
  if (!sd.ready) {
    int cu = 0;
    LRH_TRY(device_setup(dtype, 1, &cu));
    void* p = nullptr;
    LRH_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    sd.ptr = p;
    sd.n_cu = cu;
    sd.ready = true;
  }
  if (lrh::batch_path(dtype, B)) LRH_HIP(lrh::batch_init(), "GEMM kernel set-up");
  *ptr = sd.ptr;
  *n_cu = sd.n_cu;
  return LRHEAD_OK;
}

}  // namespace

extern "C" {

size_t lrhead_workspace_bytes(int dtype, int64_t V, int64_t d, int64_t r, int64_t B_max, int k_max) {
  if (check_shapes(dtype, V, d, r, B_max, k_max) != LRHEAD_OK) return 0;
  return layout(dtype, V, r, B_max, k_max).total;
}

int lrhead_create(lrhead_t* out, int dtype, int64_t V, int64_t d, int64_t r, const void* Q, const void* P,
                  const void* W, int64_t B_max, int k_max, void* workspace, size_t workspace_bytes) {
  if (!out) return fail(LRHEAD_EINVAL, "out is NULL");
  *out = nullptr;
  LRH_TRY(check_shapes(dtype, V, d, r, B_max, k_max));
  if (!Q || !P || !W) return fail(LRHEAD_EINVAL, "Q, P and W must be non-NULL");
  if (!workspace) return fail(LRHEAD_EINVAL, "workspace is NULL");
  if (!aligned16(Q) || !aligned16(P) || !aligned16(W) || !aligned16(workspace))
    return fail(LRHEAD_EALIGN, "Q, P, W and workspace must be 16-byte aligned");
  const Layout L = layout(dtype, V, r, B_max, k_max);
  if (workspace_bytes < L.total)
    return fail(LRHEAD_EWORKSPACE, "workspace holds %zu bytes, needs %zu", workspace_bytes, L.total);
  int n_cu = 0;
  LRH_TRY(device_setup(dtype, B_max, &n_cu));
  lrhead_s* h = new (std::nothrow) lrhead_s;
  if (!h) return fail(LRHEAD_EINVAL, "out of host memory");
  fill_handle(h, dtype, V, d, r, Q, P, W, B_max, k_max, workspace, workspace_bytes, n_cu);
  *out = h;
  return LRHEAD_OK;
}

int lrhead_candidates(lrhead_t h, const void* H, int64_t B, int k, int32_t* idx, float* score, void* stream) {
  LRH_TRY(check_handle(h));
  LRH_TRY(check_rows(h, H, B));
  LRH_TRY(check_k(h, k));
  LRH_TRY(check_out(idx, "idx", B > 0));
  LRH_TRY(check_out(score, "score", false));
  if (B == 0) return LRHEAD_OK;
  return enqueue_head(h, H, B, k, idx, score, nullptr, static_cast<hipStream_t>(stream));
}

int fullhead_logits(lrhead_t h, const void* H, int64_t B, const int32_t* idx, int k, float* logits,
                    void* stream) {
  LRH_TRY(check_handle(h));
  LRH_TRY(check_rows(h, H, B));
  LRH_TRY(check_out(idx, "idx", false));
  if (idx) LRH_TRY(check_k(h, k));
  LRH_TRY(check_out(logits, "logits", B > 0));
  if (B == 0) return LRHEAD_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!idx) {
    LRH_HIP(lrh::launch_dense(h->dtype, h->W, H, h->V, (int)h->d, B, logits, s), "dense logits launch");
    return LRHEAD_OK;
  }
  LRH_HIP(lrh::launch_rescore(h->dtype, h->W, H, idx, B, k, h->V, (int)h->d, logits, s), "rescore launch");
  return LRHEAD_OK;
}

int fullhead_topk(lrhead_t h, const void* H, int64_t B, int k, int32_t* idx, float* logits, void* stream) {
  LRH_TRY(check_handle(h));
  LRH_TRY(check_rows(h, H, B));
  LRH_TRY(check_k(h, k));
  LRH_TRY(check_out(idx, "idx", B > 0));
  LRH_TRY(check_out(logits, "logits", B > 0));
  if (B == 0) return LRHEAD_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (lrh::batch_path(h->dtype, B)) {
    LRH_HIP(lrh::launch_batch_select(h->W, H, h->V, (int)h->d, B, k, h->bw, idx, logits, s, timing(h)),
            "full-head selection launch");
    return LRHEAD_OK;
  }
  int n_lists;
  if (lrh::small_long_path(h->dtype, B, h->d, h->V)) {
    n_lists = lrh::small_blocks(h->V);
    LRH_HIP(lrh::launch_select_long(h->W, H, h->V, (int)h->d, B, k, h->part_s, h->part_i, s, timing(h)),
            "full-head selection launch");
  } else {
    n_lists = lrh::plan_vsplit(B, h->V);
    LRH_HIP(lrh::launch_select(h->dtype, h->W, H, h->V, (int)h->d, B, k, n_lists, h->part_s, h->part_i, s,
                               timing(h)),
            "full-head selection launch");
  }
  LRH_HIP(lrh::launch_merge(h->dtype, h->part_s, h->part_i, n_lists, k, false, nullptr, nullptr, nullptr, 0, h->V, B,
                            k, nullptr, nullptr, (int)h->d, idx, logits, nullptr, false, s),
          "merge launch");
  return LRHEAD_OK;
}

int lrhead_draft(lrhead_t h, const void* H, int64_t B, int k, int32_t* idx, float* score, float* logits,
                 void* stream) {
  LRH_TRY(check_handle(h));
  LRH_TRY(check_rows(h, H, B));
  LRH_TRY(check_k(h, k));
  LRH_TRY(check_out(idx, "idx", B > 0));
  LRH_TRY(check_out(score, "score", false));
  LRH_TRY(check_out(logits, "logits", B > 0));
  if (B == 0) return LRHEAD_OK;
  return enqueue_head(h, H, B, k, idx, score, logits, static_cast<hipStream_t>(stream));
}

int lrhead_draft_static(int dtype, int64_t V, int64_t d, int64_t r, const void* Q, const void* P, const void* W,
                        const void* H, int64_t B, int k, int32_t* idx, float* score, float* logits, void* stream) {
  if (B < 0) return fail(LRHEAD_ERANGE, "B = %lld is negative", (long long)B);
  LRH_TRY(check_shapes(dtype, V, d, r, B > 0 ? B : 1, k));
  if (!Q || !P || !W) return fail(LRHEAD_EINVAL, "Q, P and W must be non-NULL");
  if (!aligned16(Q) || !aligned16(P) || !aligned16(W)) return fail(LRHEAD_EALIGN, "Q, P and W must be 16-byte aligned");
  if (B > 0 && !H) return fail(LRHEAD_EINVAL, "H is NULL");
  if (!aligned16(H)) return fail(LRHEAD_EALIGN, "H is not 16-byte aligned");
  LRH_TRY(check_out(idx, "idx", B > 0));
  LRH_TRY(check_out(score, "score", false));
  LRH_TRY(check_out(logits, "logits", B > 0));
  if (B == 0) return LRHEAD_OK;
  const size_t need = layout(dtype, V, r, B, k).total;
  if (need > kStaticScratchBytes)
    return fail(LRHEAD_EWORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu", need,
                kStaticScratchBytes);
  void* ws = nullptr;
  int n_cu = 0;
  LRH_TRY(static_device(dtype, B, &ws, &n_cu));
  lrhead_s h;
  fill_handle(&h, dtype, V, d, r, Q, P, W, B, k, ws, kStaticScratchBytes, n_cu);
  return enqueue_head(&h, H, B, k, idx, score, logits, static_cast<hipStream_t>(stream));
}

int lrhead_branch(const float* logits, const int32_t* idx, const float* parent, int64_t B, int k, int nb,
                  float* probs, int32_t* br_idx, float* br_prob, float* br_path, void* stream) {
  if (B < 0) return fail(LRHEAD_ERANGE, "B = %lld is negative", (long long)B);
  if (k < 1 || k > LRHEAD_K_MAX) return fail(LRHEAD_ERANGE, "k = %d outside [1, %d]", k, LRHEAD_K_MAX);
  if (nb < 1 || nb > k) return fail(LRHEAD_ERANGE, "nb = %d outside [1, k = %d]", nb, k);
  if (B == 0) return LRHEAD_OK;
  if (!logits || !idx || !probs || !br_idx || !br_prob || !br_path)
    return fail(LRHEAD_EINVAL, "logits, idx, probs, br_idx, br_prob and br_path must be non-NULL");
  LRH_HIP(lrh::launch_branch(logits, idx, parent, B, k, nb, probs, br_idx, br_prob, br_path,
                             static_cast<hipStream_t>(stream)),
          "branch launch");
  return LRHEAD_OK;
}

size_t lrhead_factor_workspace_bytes(int64_t V, int64_t d, int r) {
  if (V < 1 || d < 1 || r < 1 || r > LRHEAD_R_MAX || r > d || r > V || V > INT32_MAX || d > LRHEAD_D_MAX) return 0;
  return lrh::factor_workspace_bytes(V, d, r);
}

int lrhead_factor(const void* W, int64_t V, int64_t d, int r, int q, const float* omega, void* P, void* Q,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (V < 1 || V > INT32_MAX) return fail(LRHEAD_ERANGE, "V = %lld outside [1, 2^31)", (long long)V);
  if (d < 1 || d > LRHEAD_D_MAX) return fail(LRHEAD_ERANGE, "d = %lld outside [1, %d]", (long long)d, LRHEAD_D_MAX);
  if (r < 1 || r > LRHEAD_R_MAX || r > d || r > V)
    return fail(LRHEAD_ERANGE, "r = %d outside [1, min(%d, d, V)]", r, LRHEAD_R_MAX);
  if (q < 0 || q > 8) return fail(LRHEAD_ERANGE, "q = %d outside [0, 8]", q);
  if (!W || !omega || !P || !Q || !workspace)
    return fail(LRHEAD_EINVAL, "W, omega, P, Q and workspace must be non-NULL");
  if (!aligned16(W) || !aligned16(omega) || !aligned16(P) || !aligned16(Q) || !aligned16(workspace))
    return fail(LRHEAD_EALIGN, "W, omega, P, Q and workspace must be 16-byte aligned");
  const size_t need = lrh::factor_workspace_bytes(V, d, r);
  if (workspace_bytes < need) return fail(LRHEAD_EWORKSPACE, "workspace holds %zu bytes, needs %zu", workspace_bytes, need);
  LRH_HIP(lrh::batch_init(), "GEMM kernel set-up");   // the W-sized products run on the GEMM kernel
  LRH_HIP(lrh::launch_factor(W, V, d, r, q, omega, P, Q, workspace, static_cast<hipStream_t>(stream)),
          "factor launch");
  return LRHEAD_OK;
}

int lrhead_set_stage_events(lrhead_t h, void* before, void* after) {
  LRH_TRY(check_handle(h));
  if ((before == nullptr) != (after == nullptr))
    return fail(LRHEAD_EINVAL, "give both events or neither");
  h->ev_before = static_cast<hipEvent_t>(before);
  h->ev_after = static_cast<hipEvent_t>(after);
  return LRHEAD_OK;
}

void lrhead_destroy(lrhead_t h) {
  if (h && h->magic == kMagic) {
    h->magic = 0;
    delete h;
  }
}

const char* lrhead_strerror(int code) {
  switch (code) {
    case LRHEAD_OK: return "success";
    case LRHEAD_EINVAL: return "invalid argument";
    case LRHEAD_ERANGE: return "size outside the supported range";
    case LRHEAD_EDTYPE: return "unknown dtype";
    case LRHEAD_EALIGN: return "pointer not 16-byte aligned";
    case LRHEAD_EWORKSPACE: return "workspace too small";
    case LRHEAD_EHIP: return "HIP error";
    case LRHEAD_EDEVICE: return "device is not gfx950";
    default: return "unknown error code";
  }
}

const char* lrhead_last_error(void) { return g_err; }

}  // extern "C"
