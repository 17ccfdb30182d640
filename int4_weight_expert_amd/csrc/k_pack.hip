// k_pack.hip -- load-time kernels: int4 quantise/pack, blob <-> slot layout,
// router weight layout.  None of these run inside a forward.
//
// Quantisers, cited by page title and section:
//   per-row symmetric int4: "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" §05
//     (quantize_rows: row absmax scale with a 1e-8 floor, codes by
//     round-to-nearest of w/s) and §06 (pack_int4: two codes per byte, the
//     first in the low nibble; np.rint == lrintf in §07, i.e. half to even);
//   affine int4 with group size 64: Edge0 write-up (magicnetworld.com) §三.
// Both decisions (code from a float) are taken in fp32 with IEEE
// round-to-nearest division and rint, the precision the pages use.
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint16_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int code_row(float w, float s)
{
    int v = (int)rintf(__fdiv_rn(w, s));
    return v > 7 ? 7 : (v < -7 ? -7 : v);
}

// One 256-thread workgroup per output row (grid-stride over rows).
__global__ void __launch_bounds__(256) k_pack_int4_rows(const float* __restrict__ w, int64_t O,
                                                        int64_t I, uint8_t* __restrict__ q,
                                                        float* __restrict__ s)
{
    __shared__ float red[4];
    const int tid = threadIdx.x;
    for (int64_t o = blockIdx.x; o < O; o += gridDim.x) {
        const float* wr = w + o * I;
        float amax = 0.0f;
        for (int64_t i = tid; i < I; i += 256) amax = fmaxf(amax, fabsf(wr[i]));
        amax = wave_max(amax);
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float sc = __fdiv_rn(amax, 7.0f);
        if (sc < 1e-8f) sc = 1e-8f;
        if (tid == 0) s[o] = sc;
        uint8_t* qr = q + o * (I / 2);
        for (int64_t j = tid; j < I / 2; j += 256) {
            int v0 = code_row(wr[2 * j], sc), v1 = code_row(wr[2 * j + 1], sc);
            qr[j] = (uint8_t)((v0 & 0xF) | ((v1 & 0xF) << 4));
        }
    }
}

// One wavefront per (row, group of 64 inputs); 4 groups per workgroup.
__global__ void __launch_bounds__(256) k_pack_affine_g64(const float* __restrict__ w, int64_t O,
                                                         int64_t I, uint8_t* __restrict__ q,
                                                         uint16_t* __restrict__ scmn)
{
    const int lane = threadIdx.x & 63;
    const int64_t G = I / 64;
    const int64_t total = O * G;
    for (int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); item < total;
         item += (int64_t)gridDim.x * 4) {
        const int64_t o = item / G, g = item % G;
        const float v = w[o * I + g * 64 + lane];
        const float lo = wave_min(v), hi = wave_max(v);
        const uint16_t sc16 = bf16_rne(__fdiv_rn(hi - lo, 15.0f));
        const uint16_t mn16 = bf16_rne(lo);
        const float scv = __uint_as_float((uint32_t)sc16 << 16);
        const float mnv = __uint_as_float((uint32_t)mn16 << 16);
        int c = 0;
        if (scv != 0.0f) {
            c = (int)rintf(__fdiv_rn(v - mnv, scv));
            c = c < 0 ? 0 : (c > 15 ? 15 : c);
        }
        const int c_hi = __shfl_down(c, 1);
        if ((lane & 1) == 0) q[o * (I / 2) + g * 32 + (lane >> 1)] = (uint8_t)(c | (c_hi << 4));
        if (lane == 0) {
            scmn[(o * G + g) * 2 + 0] = sc16;
            scmn[(o * G + g) * 2 + 1] = mn16;
        }
    }
}

// Blob matrix [O][In/2] bytes <-> slot interleave (see moe_internal.h).
// One thread per 16-byte chunk; `flip` = 0x88888888 for the row format.
__global__ void __launch_bounds__(256) k_interleave(const uint8_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, int64_t O,
                                                    int64_t In, uint32_t flip, int to_slot)
{
    const int64_t C = In / 32;
    const int64_t total = O * C;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t lane = idx & 63, c = (idx >> 6) % C, b = (idx >> 6) / C;
        const int64_t canon = (b * 64 + lane) * (In / 2) + c * 16;
        const int64_t inter = idx * 16;
        uint4 v = *(const uint4*)(src + (to_slot ? canon : inter));
        v.x ^= flip;
        v.y ^= flip;
        v.z ^= flip;
        v.w ^= flip;
        *(uint4*)(dst + (to_slot ? inter : canon)) = v;
    }
}

// Affine (scale, min) pairs: blob [O][G] <-> slot [O/64][G][64], 4 B each.
__global__ void __launch_bounds__(256) k_interleave_pairs(const uint32_t* __restrict__ src,
                                                          uint32_t* __restrict__ dst, int64_t O,
                                                          int64_t G, int to_slot)
{
    const int64_t total = O * G;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t lane = idx & 63, g = (idx >> 6) % G, b = (idx >> 6) / G;
        const int64_t canon = (b * 64 + lane) * G + g;
        if (to_slot) dst[idx] = src[canon];
        else dst[canon] = src[idx];
    }
}

// Router W [E][H] -> [Epad/64][H/4][64] float4 (rows >= E are zero).
__global__ void __launch_bounds__(256) k_router_layout(const float* __restrict__ W,
                                                       float4* __restrict__ wr, int E, int Epad,
                                                       int H)
{
    const int64_t C = H / 4;
    const int64_t total = (int64_t)Epad * C;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t lane = idx & 63, c = (idx >> 6) % C, b = (idx >> 6) / C;
        const int64_t row = b * 64 + lane;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < E) v = *(const float4*)(W + row * H + c * 4);
        wr[idx] = v;
    }
}

static unsigned grid_for(int64_t items, int64_t per_block)
{
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

hipError_t launch_pack_int4_rows(const float* w, int64_t O, int64_t I, uint8_t* q, float* s,
                                 hipStream_t st)
{
    hipLaunchKernelGGL(k_pack_int4_rows, dim3(grid_for(O, 1)), dim3(256), 0, st, w, O, I, q, s);
    return hipGetLastError();
}

hipError_t launch_pack_affine_g64(const float* w, int64_t O, int64_t I, uint8_t* q,
                                  uint16_t* scmn, hipStream_t st)
{
    hipLaunchKernelGGL(k_pack_affine_g64, dim3(grid_for(O * (I / 64), 4)), dim3(256), 0, st, w,
                       O, I, q, scmn);
    return hipGetLastError();
}

static hipError_t convert(const uint8_t* src, uint8_t* dst, int fmt, int H, int I, int to_slot,
                          hipStream_t st)
{
    const int64_t gq = (int64_t)I * (H / 2), dq = (int64_t)H * (I / 2);
    const uint32_t flip = fmt == MOE_W_INT4_ROW ? 0x88888888u : 0u;
    const int64_t mats[3][3] = {{0, I, H}, {gq, I, H}, {2 * gq, H, I}};  // offset, O, In
    for (auto& m : mats) {
        hipLaunchKernelGGL(k_interleave, dim3(grid_for(m[1] * (m[2] / 32), 256)), dim3(256), 0,
                           st, src + m[0], dst + m[0], m[1], m[2], flip, to_slot);
    }
    const int64_t sb = 2 * gq + dq;
    if (fmt == MOE_W_INT4_ROW) {
        hipError_t e = hipMemcpyAsync(dst + sb, src + sb, (size_t)(2 * I + H) * 4,
                                      hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return e;
    } else {
        const int64_t ga = (int64_t)I * (H / 64) * 4;
        const int64_t pm[3][3] = {{sb, I, H / 64}, {sb + ga, I, H / 64}, {sb + 2 * ga, H, I / 64}};
        for (auto& m : pm)
            hipLaunchKernelGGL(k_interleave_pairs, dim3(grid_for(m[1] * m[2], 256)), dim3(256), 0,
                               st, (const uint32_t*)(src + m[0]), (uint32_t*)(dst + m[0]), m[1],
                               m[2], to_slot);
    }
    return hipGetLastError();
}

hipError_t launch_blob_to_slot(const uint8_t* blob, uint8_t* slot, int fmt, int H, int I,
                               hipStream_t st)
{
    return convert(blob, slot, fmt, H, I, 1, st);
}

hipError_t launch_slot_to_blob(const uint8_t* slot, uint8_t* blob, int fmt, int H, int I,
                               hipStream_t st)
{
    return convert(slot, blob, fmt, H, I, 0, st);
}

hipError_t launch_router_to_internal(const float* W, float* wr, int E, int Epad, int H,
                                     hipStream_t st)
{
    hipLaunchKernelGGL(k_router_layout, dim3(grid_for((int64_t)Epad * (H / 4), 256)), dim3(256),
                       0, st, W, (float4*)wr, E, Epad, H);
    return hipGetLastError();
}

}  // namespace moe
