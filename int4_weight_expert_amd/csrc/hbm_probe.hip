// hbm_probe.hip -- a plain streaming-read kernel that measures the HBM read
// rate this part reaches, the ceiling the byte-bound MoE kernels are held
// against, and a read of the one-token gate/up kernel's bytes in the access
// patterns of two slot layouts.  Not part of the MoE path: a
// separate library (libhbm_probe.so) that only the benchmark loads.
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

// The one-token gate/up launch's bytes read in three access patterns by the
// same workgroups (n_exp x 256 of 256 threads, 48 KB each as 12 16-byte
// loads per lane, all in flight at once), with the GLM expert shape (gate and
// up [2048][6144] int4): PATTERN 0 as a workgroup that owns 8 rows reads them
// from 64-row blocks of 1 KiB chunks (their 16-byte pieces of every chunk,
// 128 bytes out of each 1 KiB, the other rows read by other workgroups),
// PATTERN 2 the same in an order that puts the 8 workgroups sharing a 64-row
// block on one XCD (within each run of 64 workgroups the order transposed),
// PATTERN 1 each workgroup's 48 KB contiguous, as in the slot layout's 8-row
// groups.
constexpr int kPH = 6144, kPI = 2048, kPC = kPH / 32;

template <int PATTERN>
__global__ void __launch_bounds__(kThreads) k_pattern_read(const uint8_t* __restrict__ buf,
                                                           size_t exp_bytes, uint32_t* __restrict__ sink,
                                                           uint32_t never)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int p = blockIdx.x, q = PATTERN == 2 ? (p & ~63) + ((p & 7) << 3) + ((p >> 3) & 7) : p;
    const int sb = q % (kPI / 8), gi = q / (kPI / 8);
    const uint8_t* base = buf + (size_t)gi * exp_bytes;
    u32x4 v[12];
    if (PATTERN != 1) {
        const int b = sb >> 3, s8 = sb & 7, rr = lane & 7, j = lane >> 3, c0 = w * 48;
        const size_t off = (size_t)(s8 * 8 + rr) * 16 + (size_t)(2 * j) * 1024;
#pragma unroll
        for (int st = 0; st < 3; ++st)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const size_t so = (size_t)(c0 + st * 16 + h) * 1024;
                v[2 * st + h] = *(const u32x4*)(base + (size_t)b * kPC * 1024 + off + so);
                v[6 + 2 * st + h] = *(const u32x4*)(base + (size_t)kPI * kPH / 2 + (size_t)b * kPC * 1024 + off + so);
            }
    } else {
        const uint8_t* p = base + (size_t)sb * 49152 + (size_t)w * 12288;
#pragma unroll
        for (int i = 0; i < 12; ++i) v[i] = *(const u32x4*)(p + (size_t)i * 1024 + lane * 16);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 12; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
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

// Reads n_exp GLM-shape experts' gate and up codes (exp_bytes apart from buf,
// at least 12.6 MB each) in `pattern` 0 (8 rows' pieces of 64-row blocks),
// 1 (contiguous per workgroup: the 8-row groups) or 2 (0 with the workgroups
// sharing a block on one XCD); sink needs n_exp x 256 words.  Returns a
// hipError_t value (0 = success).
int hbm_probe_pattern(const void* buf, size_t exp_bytes, int n_exp, int pattern, uint32_t* sink,
                      uint32_t never, void* stream)
{
    if (!buf || !sink || n_exp <= 0 || exp_bytes < (size_t)kPI * kPH) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)(n_exp * (kPI / 8))), block(kThreads);
    if (pattern == 0)
        hipLaunchKernelGGL(k_pattern_read<0>, grid, block, 0, (hipStream_t)stream, (const uint8_t*)buf,
                           exp_bytes, sink, never);
    else if (pattern == 2)
        hipLaunchKernelGGL(k_pattern_read<2>, grid, block, 0, (hipStream_t)stream, (const uint8_t*)buf,
                           exp_bytes, sink, never);
    else
        hipLaunchKernelGGL(k_pattern_read<1>, grid, block, 0, (hipStream_t)stream, (const uint8_t*)buf,
                           exp_bytes, sink, never);
    return (int)hipGetLastError();
}

}  // extern "C"
