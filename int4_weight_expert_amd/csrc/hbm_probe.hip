// hbm_probe.hip -- a plain streaming-read kernel that measures the HBM read
// rate this part reaches, the ceiling the byte-bound MoE kernels are held
// against.  Not part of the MoE path: a separate library (libhbm_probe.so)
// that only the benchmark loads.
//
// Each thread reads 16-byte pieces with a grid stride, eight loads in
// flight, and folds them into one word so that the loads cannot be removed;
// a workgroup stores its word only if it equals a value no input produces
// here (the buffer is filled by the caller), so no store reaches memory in
// practice and the traffic is reads only.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ void __launch_bounds__(kThreads) k_stream_read(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink,
                                                         uint32_t never)
{
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int k = 0; k < kInFlight; ++k)
            v[k] = NT ? __builtin_nontemporal_load(&p[i + k * stride]) : p[i + k * stride];
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) at buf once with `blocks` workgroups of
// 256 threads, on `stream`, with plain (nt = 0) or non-temporal (nt = 1)
// loads; sink needs `blocks` words.  Returns a hipError_t value (0 =
// success).
int hbm_probe_read(const void* buf, size_t bytes, int blocks, int nt, uint32_t* sink,
                   uint32_t never, void* stream)
{
    if (!buf || !sink || blocks <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
    if (nt)
        hipLaunchKernelGGL(k_stream_read<true>, dim3(blocks), dim3(kThreads), 0,
                           (hipStream_t)stream, (const u32x4*)buf, bytes / 16, sink, never);
    else
        hipLaunchKernelGGL(k_stream_read<false>, dim3(blocks), dim3(kThreads), 0,
                           (hipStream_t)stream, (const u32x4*)buf, bytes / 16, sink, never);
    return (int)hipGetLastError();
}

}  // extern "C"
