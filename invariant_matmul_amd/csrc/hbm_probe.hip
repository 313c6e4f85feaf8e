// Streaming-read probe of HBM bandwidth, for the benchmark only (built as its
// own shared library, libimm_hbm_probe.so; the GEMM library neither links nor
// calls it).
//
// The decode-shaped products are bound by reading B once from HBM (the
// Tencent deterministic-inference article, "Split-K": decode at M = 1 is the
// memory-bound case).  This probe measures what a plain read of a buffer
// achieves on the part, as the ceiling those products are judged against:
// every lane reads 16-byte vectors in a grid-stride loop, eight loads in
// flight per lane, and folds them into one word so the loads cannot be
// removed; nothing else is written (the word is stored only if it matches a
// value the data never produces, so in practice the kernel writes nothing).
//
// C ABI (no torch types):
//   int imm_probe_read(const void* src, size_t bytes, unsigned* sink,
//                      int workgroups, int nontemporal, void* stream);
//     src: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned);
//     sink: device word written only in the impossible case above;
//     workgroups: grid size (256 threads each), 1 .. 65536;
//     nontemporal: 1 = loads marked non-temporal.
//     Returns 0, or -1 for a bad argument, or the HIP error of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;
constexpr unsigned kMagic = 0x9e3779b9u;

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* src, int64_t n16,
                                                              unsigned* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  unsigned acc = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  // full rounds of kInFlight loads, then the tail one load at a time
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kMagic) sink[0] = acc;
}

}  // namespace

extern "C" int imm_probe_read(const void* src, size_t bytes, unsigned* sink, int workgroups,
                              int nontemporal, void* stream) {
  if (!src || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
      workgroups < 1 || workgroups > 65536)
    return -1;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(src);
  if (nontemporal)
    hipLaunchKernelGGL(read_probe_kernel<true>, dim3(workgroups), dim3(kThreads), 0, s, p, n16, sink);
  else
    hipLaunchKernelGGL(read_probe_kernel<false>, dim3(workgroups), dim3(kThreads), 0, s, p, n16, sink);
  return (int)hipGetLastError();
}
