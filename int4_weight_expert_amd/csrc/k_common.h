// k_common.h -- device helpers shared by the forward kernels: int4 byte
// unpacking, buffer loads, wavefront reductions, agent-scope hand-off
// between workgroups.  Internal to the library.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// AND whose result the compiler cannot narrow, so that the byte conversions
// below stay single v_cvt_f32_ubyteN instructions.
__device__ __forceinline__ uint32_t and_opaque(uint32_t a, uint32_t mask)
{
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(mask), "v"(a));
    return r;
}

__device__ __forceinline__ float ub0(uint32_t u) { return (float)(u & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t u) { return (float)((u >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t u) { return (float)((u >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t u) { return (float)(u >> 24); }

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Activations read by every lane at the same address, and read-only for the
// whole kernel, go through the constant address space: scalar loads.
typedef const __attribute__((address_space(4))) float cf32;

__device__ __forceinline__ cf32* as_const(const float* p) { return (cf32*)p; }

// Weight streams use buffer loads: one SGPR resource per stream, the lane's
// 16-byte offset in one VGPR, the chunk offset as an SGPR/immediate.  A load
// outside the resource's range returns zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 8 codes of one dword against 8 activations read from LDS at a wave-uniform
// address (broadcast ds_read_b128).  Even columns sit in the low nibbles
// (value v), odd columns in the high nibbles (value 16 v): they go to
// separate accumulators and the odd one is scaled by 1/16 at the end.
__device__ __forceinline__ void dot8(uint32_t w, const float* xs, float& ae, float& ao)
{
    const float4 x0 = *(const float4*)xs, x1 = *(const float4*)(xs + 4);
    const uint32_t lo = and_opaque(w, 0x0F0F0F0Fu), hi = and_opaque(w, 0xF0F0F0F0u);
    ae = fmaf(ub0(lo), x0.x, ae);
    ao = fmaf(ub0(hi), x0.y, ao);
    ae = fmaf(ub1(lo), x0.z, ae);
    ao = fmaf(ub1(hi), x0.w, ao);
    ae = fmaf(ub2(lo), x1.x, ae);
    ao = fmaf(ub2(hi), x1.y, ao);
    ae = fmaf(ub3(lo), x1.z, ae);
    ao = fmaf(ub3(hi), x1.w, ao);
}

__device__ __forceinline__ void dot32(const uint4& w, const float* xs, float& ae, float& ao)
{
    dot8(w.x, xs, ae, ao);
    dot8(w.y, xs + 8, ae, ao);
    dot8(w.z, xs + 16, ae, ao);
    dot8(w.w, xs + 24, ae, ao);
}

// Data handed between workgroups of one kernel travels with agent-scope
// relaxed atomic accesses (sc1 loads/stores, coherent across the XCDs' L2s
// without writing back or invalidating whole caches).  An arrival first
// waits for the caller's stores to complete (s_waitcnt vmcnt(0)), then
// bumps the counter; whoever sees the last count reads everything.  The
// last arriver resets the counter for the next launch.
__device__ __forceinline__ void st_agent(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_agent(const float* p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// whole-workgroup arrival
__device__ __forceinline__ bool arrive_block(uint32_t* counter, uint32_t expected)
{
    __shared__ int s_last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == expected - 1;
    }
    __syncthreads();
    const bool last = s_last;
    if (last && threadIdx.x == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// single-wavefront arrival
__device__ __forceinline__ bool arrive_wave(uint32_t* counter, uint32_t expected)
{
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t prev = 0;
    if ((threadIdx.x & 63) == 0)
        prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    const bool last = prev == expected - 1;
    if (last && (threadIdx.x & 63) == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return last;
}

// Token j of an expert group: its token index t and its row r in h and in
// the down partials (routed assignment a = t*K + k uses row a; shared
// expert s uses T*K + s*T + t).
__device__ __forceinline__ void tok_rows(const Fwd& f, const int32_t* __restrict__ perm,
                                         const Group& g, int j, int& t, int& r)
{
    if (g.kind == 0) {
        const int a = perm[g.off + j];
        t = a / f.K;
        r = a;
    } else {
        t = j;
        r = f.T * f.K + g.off * f.T + j;
    }
}

}  // namespace moe
