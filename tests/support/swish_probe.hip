// Test support: evaluates the encoder's Swish (rkv_swish.h, the same source the kernels
// compile) on an array, so that its error can be measured against fp64 on the host.
#include <hip/hip_runtime.h>

#include "rkv_swish.h"

namespace {
__global__ void swish_probe_kernel(const float* __restrict__ x, float* __restrict__ y, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = rkv::silu(x[i]);
}
}  // namespace

// x, y: device arrays of n floats. Returns 0, or the HIP error code of the launch.
extern "C" int rkv_swish_probe(const float* x, float* y, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(swish_probe_kernel, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), x,
                       y, n);
    return (int)hipGetLastError();
}
