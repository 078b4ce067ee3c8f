// launch.h -- kernel launch that reports its own status.
//
// hipLaunchKernel returns the status of this launch.  Reading hipGetLastError()
// after a triple-chevron launch instead would also pick up (and clear) an error
// left by an unrelated earlier HIP call of the caller, and report a launch that
// was in fact queued as failed.
#ifndef ETA_LAUNCH_H
#define ETA_LAUNCH_H

#include <hip/hip_runtime.h>

// Every kernel of this library takes one argument struct by value.
template <typename Args>
inline hipError_t launch_kernel(void (*kernel)(Args), dim3 grid, dim3 block, hipStream_t stream, Args args) {
    void* params[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0, stream);
}

#endif  // ETA_LAUNCH_H
