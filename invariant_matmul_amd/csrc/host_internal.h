// Host-side helpers of the C ABI shared by api.cpp and noalloc.hip.
#pragma once

#include <hip/hip_runtime.h>

#include "imm_internal.h"

namespace imm {

// Host-side helpers of the C ABI (api.cpp).
// Records a HIP error as the thread's last error; returns GEMM_ERR_HIP.
gemm_status record_hip_error(hipError_t e);
// The checks of a run call that need no runtime: plan, NULL and alignment.
gemm_status check_run_args(const gemm_plan_s* p, const void* A, const void* B, const void* C,
                           const float* bias);
// The split-K product (partial kernel into `workspace`, then the reduction)
// with every check of gemm_splitk_run_bias; check_ws = false skips the
// device-allocation check of the workspace (the library's own scratch array,
// which the runtime's pointer queries do not describe).
gemm_status splitk_run(const gemm_plan_s* p, const void* A, const void* B, const float* bias,
                       void* C, void* workspace, size_t workspace_bytes, bool check_ws,
                       hipStream_t s);

}  // namespace imm
