// Device-side helper shared by the GEMV and GEMM kernels (included by .hip
// sources only: the host-side C-ABI layer never sees it).
#pragma once
#include <hip/hip_runtime.h>

namespace qt {

// Barrier that orders LDS accesses only: global loads in flight stay in
// flight.  __syncthreads() also waits for every outstanding global load,
// which would expose the latency of prefetches issued just before it.
// (LDS-direct loads still in flight are waited for: they write LDS.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace qt
