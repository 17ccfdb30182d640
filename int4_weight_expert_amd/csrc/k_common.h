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

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
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

__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
    return make_uint2(v.x, v.y);
}

// Slot layout of an int4 matrix [O][In] (row and affine formats): 8-row
// groups.  Within group o / 8 the 16-byte pieces of its 8 rows for chunk c
// (32 inputs) are 128 contiguous bytes, chunk after chunk, so a group's
// codes are one run of C * 128 bytes (C = In / 32) and a 64-row block (8
// groups) is C * 1024 bytes.  Byte offset of row r's piece of chunk c,
// counted from the start of r's 64-row block (r < 64) or of the matrix:
__device__ __forceinline__ uint32_t blk_off(int r, int C, int c)
{
    return (uint32_t)(((r >> 3) * C + c) * 128 + (r & 7) * 16);
}
// Affine (scale, min) pairs, 4 bytes each, grouped the same way: row r's
// pair of input group g (64 inputs) at ((r / 8) * G + g) * 32 + (r % 8) * 4.
__device__ __forceinline__ uint32_t tab_off(int r, int G, int g)
{
    return (uint32_t)(((r >> 3) * G + g) * 32 + (r & 7) * 4);
}

__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
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

// ---------------------------------------------------------------------------
// fp16 dot path of the expert GEMVs.
//
// A dword of codes holds 8 nibbles n0..n7 (input i in bits 4i..4i+3).  Each
// nibble is moved to bits 4..7 of an fp16 whose exponent field is that of
// 1024 (0x6400): the half then reads exactly 1024 + 16 n.  One bit-field insert per
// pair builds (n0,n4) (n1,n5) (n2,n6) (n3,n7), and v_dot2_f32_f16 multiplies
// a pair with the matching pair of fp16 activations, accumulating in fp32.
// Activations are staged once per forward in spans of 64 inputs: each span
// is scaled by a power of two 2^k that puts its largest magnitude in
// [2^13, 2^14) (exact, no overflow), rounded to fp16 and stored in pair
// order, eight inputs per 16 bytes: x0 x4 x1 x5 x2 x6 x3 x7; beside it the
// span keeps (2^-k, sum of its fp16 values).  Over a span,
// sum (1024 + 16 n) x / 16 = sum n x + 64 sum x, and the kernels remove the
// 64 sum x term (plus the code offset) with the span's stored sum, then
// rescale by 2^-k.
// ---------------------------------------------------------------------------

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t NIB_MASK = 0x00F000F0u;

// The magic exponent lives in a VGPR (gfx9 VOP3 takes no literal, and the
// constant bus takes one SGPR: the mask).
__device__ __forceinline__ uint32_t magic_vgpr()
{
    uint32_t r;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(r));
    return r;
}

__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t c)
{
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(mask), "v"(a), "v"(c));
    return r;
}

// four fp16 pairs 1024 + 16 n of one dword of codes (v_bfi_b32 issues
// faster than v_and_or_b32 on gfx950)
__device__ __forceinline__ void nib_pairs(uint32_t w, uint32_t mv, uint32_t& p0, uint32_t& p1,
                                          uint32_t& p2, uint32_t& p3)
{
    p0 = bfi(NIB_MASK, w << 4, mv);
    p1 = bfi(NIB_MASK, w, mv);
    p2 = bfi(NIB_MASK, w >> 4, mv);
    p3 = bfi(NIB_MASK, w >> 8, mv);
}

// The same pairs in plain code, for matrix-core operands: the compiler
// inserts the wait states a matrix instruction needs after the vector ALU
// writes its source registers only for instructions it can see, not for
// the results of inline assembly (with nib_pairs feeding v_mfma directly,
// the few-token kernels read stale operands).
// mv holds 0x64006400 in a form the compiler cannot fold (Fwd::magic), so
// that each pair is one v_bfi_b32 it forms itself.
__device__ __forceinline__ void nib_pairs_mfma(uint32_t w, uint32_t mv, uint32_t& p0, uint32_t& p1,
                                               uint32_t& p2, uint32_t& p3)
{
    p0 = ((w << 4) & NIB_MASK) | (mv & ~NIB_MASK);
    p1 = (w & NIB_MASK) | (mv & ~NIB_MASK);
    p2 = ((w >> 4) & NIB_MASK) | (mv & ~NIB_MASK);
    p3 = ((w >> 8) & NIB_MASK) | (mv & ~NIB_MASK);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c,
                                  false);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi)
{
    h2_t v;
    v.x = lo;
    v.y = hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Stages one span of 64 activations held one per lane (lane i = input i):
// q16 receives the 64 fp16 values in pair order, *sc = (2^-k, sum).
__device__ __forceinline__ void stage_span64(float v, int lane, uint16_t* __restrict__ q16,
                                             float2* __restrict__ sc)
{
    const float m = wave_max(fabsf(v));
    int e;
    frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)
    e = max(e, -100);
    const _Float16 h = (_Float16)(v * ldexpf(1.0f, 14 - e));
    const float t = wave_sum((float)h);
    const int g = lane >> 3, p = lane & 7;
    q16[g * 8 + (p < 4 ? 2 * p : 2 * p - 7)] = __builtin_bit_cast(uint16_t, h);
    if (lane == 0) *sc = make_float2(ldexpf(1.0f, e - 14), t);
}

// One row of `len` fp32 values (len a multiple of 8), held by one
// wavefront, staged as fp16 with one power-of-two scale that puts its largest
// magnitude in [2^13, 2^14): q[len/8] in pair order and *s = (2^-k, sum of
// the fp16 values).  Lane l holds 8-value groups l, l + 64, ... (NG of them,
// NG >= len / 512), all loaded before anything else.  Also returns the
// row's fp32 sum and sum of squares (wavefront totals).
template <int NG>
__device__ __forceinline__ void stage_row(const float* __restrict__ row, int len, int lane,
                                          uint4* __restrict__ q, float2* __restrict__ s,
                                          float& sum, float& ss)
{
    const float4* r4 = (const float4*)row;
    const int ng = len / 8;
    float4 a[NG], b[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane + 64 * i;
        a[i] = b[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (g < ng) {
            a[i] = r4[2 * g];
            b[i] = r4[2 * g + 1];
        }
    }
    float m = 0.f, su = 0.f, sq = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const float v[8] = {a[i].x, a[i].y, a[i].z, a[i].w, b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            m = fmaxf(m, fabsf(v[k]));
            su += v[k];
            sq = fmaf(v[k], v[k], sq);
        }
    }
    m = wave_max(m);
    sum = wave_sum(su);
    ss = wave_sum(sq);
    int e;
    frexpf(m, &e);
    e = max(e, -100);
    const float sc = ldexpf(1.0f, 14 - e);
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int g = lane + 64 * i;
        if (g < ng) {
            const _Float16 h0 = (_Float16)(a[i].x * sc), h1 = (_Float16)(a[i].y * sc);
            const _Float16 h2 = (_Float16)(a[i].z * sc), h3 = (_Float16)(a[i].w * sc);
            const _Float16 h4 = (_Float16)(b[i].x * sc), h5 = (_Float16)(b[i].y * sc);
            const _Float16 h6 = (_Float16)(b[i].z * sc), h7 = (_Float16)(b[i].w * sc);
            q[g] = make_uint4(pack_h2(h0, h4), pack_h2(h1, h5), pack_h2(h2, h6), pack_h2(h3, h7));
            t += (((float)h0 + (float)h1) + ((float)h2 + (float)h3)) +
                 (((float)h4 + (float)h5) + ((float)h6 + (float)h7));
        }
    }
    t = wave_sum(t);
    if (lane == 0) *s = make_float2(ldexpf(1.0f, e - 14), t);
}

// Data handed between workgroups of one kernel travels with agent-scope
// relaxed atomic accesses (sc1 loads/stores, coherent across the XCDs' L2s
// without writing back or invalidating whole caches).  An arrival first
// waits for the caller's stores to complete (s_waitcnt vmcnt(0)), then
// bumps the counter; whoever sees the last count reads everything.  The
// last arriver resets the counter for the next launch.
// Why this orders the hand-off without release/acquire: (1) the compiler
// may reorder relaxed atomics to different addresses, so a compiler-only
// fence (__atomic_signal_fence, no instruction) sits on both sides of the
// arrival and keeps the data stores before it and the reader's loads after
// it in program order; (2) in hardware, vmcnt(0) returns only once every
// earlier vector store has been acknowledged by the memory level that makes
// it agent-coherent (sc1), and the counter update is issued after that;
// (3) the reader's sc1 loads miss the non-coherent caches and are issued
// only after its fetch_add has returned the last count (a value dependence
// through the branch).  An agent-scope acq_rel would instead write back
// and invalidate the whole L2, which costs more than the hand-off.
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
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return last;
}

// Whole-workgroup arrival for many workgroups arriving together: workgroup
// p arrives on sub-counter p % 16 (each on a 256-byte line of its own, 64
// words apart), the last of each sub-counter on the top counter (word
// 16 * 64); true for the last of all.  Each counter is reset by its last
// arriver.  (Atomics on one address serialise: one counter for all costs
// about 12 ns per workgroup.)
__device__ __forceinline__ bool arrive_block_h(uint32_t* cnt, uint32_t n)
{
    __shared__ int s_last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t sub = blockIdx.x % 16u, members = n / 16u + (sub < n % 16u ? 1u : 0u);
        int last = 0;
        if (__hip_atomic_fetch_add(&cnt[sub * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            members - 1) {
            __hip_atomic_store(&cnt[sub * 64], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t subs = n < 16u ? n : 16u;
            if (__hip_atomic_fetch_add(&cnt[16 * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                subs - 1) {
                __hip_atomic_store(&cnt[16 * 64], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = 1;
            }
        }
        s_last = last;
    }
    __syncthreads();
    const bool last = s_last;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return last;
}

// single-wavefront arrival
__device__ __forceinline__ bool arrive_wave(uint32_t* counter, uint32_t expected)
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t prev = 0;
    if ((threadIdx.x & 63) == 0)
        prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    const bool last = prev == expected - 1;
    if (last && (threadIdx.x & 63) == 0)
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return last;
}

// A token whose sum of squares is not finite (x holds a NaN or an infinity,
// or magnitudes whose squares overflow fp32) sets the range status bit
// (moe_status reports MOE_E_RANGE); its outputs are then unspecified.
__device__ __forceinline__ void flag_range(const Fwd& f, float ss)
{
    if (!(ss <= 3.402823466e38f)) atomicOr(&f.status[0], (uint32_t)STATUS_RANGE);
}

// Wave-uniform copies (SGPRs) of values the compiler cannot prove uniform:
// group descriptors and token indices read from memory by every lane.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ Group uni_group(const Group* __restrict__ GR, int gi)
{
    const Group g = GR[gi];
    Group u;
    const uint64_t p = (uint64_t)(uintptr_t)g.base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    u.base = (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    u.cnt = uni(g.cnt);
    u.off = uni(g.off);
    u.kind = uni(g.kind);
    u.expert = uni(g.expert);
    return u;
}

// Token j of an expert group: its token index t and its row r in h and in
// the expert outputs (routed assignment a = t*K + k uses row a; shared
// expert s uses T*K + s*T + t).  Wave-uniform.
__device__ __forceinline__ void tok_rows(const Fwd& f, const int32_t* __restrict__ perm,
                                         const Group& g, int j, int& t, int& r)
{
    if (g.kind == 0) {
        const int a = uni(perm[g.off + j]);
        t = a / f.K;
        r = a;
    } else {
        t = j;
        r = f.T * f.K + g.off * f.T + j;
    }
}

}  // namespace moe
