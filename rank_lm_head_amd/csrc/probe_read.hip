// probe_read.hip — the achievable HBM read bandwidth of the GPU, as the
// denominator that sits beside the specification peak in the benchmark's
// roofline. Measurement only: built into its own library (libprobe.so), not
// part of the head's C ABI.
//
// A grid of blocks reads a buffer once with 16-byte non-temporal loads, each
// thread keeping 8 of them in flight (grid-stride: consecutive threads read
// consecutive 16 bytes, so every wave load is 1 KiB of contiguous memory).
// The words are folded into one value that is stored only if it matches a
// value the caller never uses, so no load is dead to the compiler and the
// probe writes (almost) nothing.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kInFlight = 8;

__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t key,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) v[t] = __builtin_nontemporal_load(p + i + t * stride);
#pragma unroll
    for (int t = 0; t < kInFlight; ++t) acc ^= v[t].x ^ v[t].y ^ v[t].z ^ v[t].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) at `buf` once on
// `stream` with `blocks` blocks of 512 threads. `sink` (4 bytes of device
// memory) is written only when the folded words equal `key`. Returns 0, or
// -1 for bad arguments, or the HIP error of the launch.
extern "C" int probe_read(const void* buf, size_t bytes, uint32_t key, uint32_t* sink, int blocks,
                          hipStream_t stream) {
  if (!buf || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15u) || blocks < 1) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const u32x4*>(buf),
                     bytes / 16, key, sink);
  return (int)hipGetLastError();
}
