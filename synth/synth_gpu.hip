// synth_gpu.hip -- device fill of the seeded synthetic inputs defined in
// synth.h, so that tens of GB of expert weights can be generated in place in
// HBM.  Input generation only; the values are bit-identical to synth_host.c
// (integer hashing plus one exact fp32 multiply per element).
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang force_cuda_host_device begin
#include "synth.h"
#pragma clang force_cuda_host_device end

__global__ void __launch_bounds__(256) synth_fill_gauss_kernel(float* __restrict__ out, uint64_t n,
                                                               uint64_t key, float sigma,
                                                               uint64_t idx0)
{
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        out[i] = synth_gauss(key, idx0 + i, sigma);
}

extern "C" int synth_gpu_fill_gauss(float* dev_out, uint64_t n, uint64_t key, float sigma,
                                    uint64_t idx0, void* stream)
{
    if (n == 0) return 0;
    if (dev_out == nullptr) return -1;
    uint64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(synth_fill_gauss_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, dev_out, n, key, sigma, idx0);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
