// The allocation-free split-K entry point, gemm_splitk_run_noalloc.
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the split-K
// partial sums go to a workspace that is part of the library itself, a
// file-scope device array of GEMM_NOALLOC_WORKSPACE_BYTES.  The loaded code
// object holds one copy of it on every GPU the library runs on, from the
// first use on that GPU until the process ends.
//
// In host code the array's name only stands for it: its device address on a
// GPU comes from hipGetSymbolAddress, looked up once per device (with that
// device current) on the entry point's first call there and kept in
// g_scratch.  Only that address is ever handed to kernels.
//
// Every call on one GPU shares that GPU's array and finds in it whatever the
// previous call left.  Nothing needs clearing: the partial kernel writes
// every element [s, m, n] (s < split_k, m < M, n < N) before the reduction
// kernel, later on the same stream, reads it.  Two calls that overlap on one
// GPU (different streams or host threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host_internal.h"

static __device__ __align__(256) char scratch[GEMM_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The address of this device's copy of the array (looked up on first use).
hipError_t scratch_on(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" gemm_status gemm_splitk_run_noalloc(gemm_plan_t p, const void* A, const void* B,
                                               void* C, void* stream) {
  gemm_status st = imm::check_run_args(p, A, B, C, nullptr);
  if (st != GEMM_OK || p->M == 0 || p->N == 0) return st;
  if (gemm_workspace_size(p) > GEMM_NOALLOC_WORKSPACE_BYTES) return GEMM_ERR_WORKSPACE;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return imm::record_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED;
  void* ws = nullptr;
  e = scratch_on(dev, &ws);
  if (e != hipSuccess) return imm::record_hip_error(e);
  return imm::splitk_run(p, A, B, nullptr, C, ws, GEMM_NOALLOC_WORKSPACE_BYTES, false,
                         static_cast<hipStream_t>(stream));
}
