// Device-side half of the device-data checks, for the kernel translation units.  Each unit that
// includes this header gets its own error word (internal linkage): the first bad index a kernel of
// that unit meets is recorded as (code, where, value), and read_clear_error() hands it to the host.
#pragma once

#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace {

__device__ int32_t g_pkv_error[3];

// First caller wins; later errors are dropped until the host clears the word.
__device__ __forceinline__ void record_error(int32_t code, int32_t where, int32_t value) {
    if (atomicCAS(&g_pkv_error[0], 0, code) == 0) {
        g_pkv_error[1] = where;
        g_pkv_error[2] = value;
    }
}

// Copy this unit's error word to out[3] and clear it, on `stream`, then wait for the stream.
inline int read_clear_error(void* stream, int32_t* out) {
    static const int32_t zero[3] = {0, 0, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(g_pkv_error), sizeof zero, 0, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess)
        e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_pkv_error), zero, sizeof zero, 0, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "reading the device error word failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

}  // namespace
