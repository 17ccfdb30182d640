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
//
// Sources: fp32, bf16, or FP8 E4M3 (fn) codes with one fp32 inverse scale
// per 128 x 128 block, the checkpoint's form ("惊呆了！…" §06, FP8 block
// decode: fp8 value times its block's inverse scale, one fp32 multiply).
// The FP8 decode is gfx950's v_cvt_pk_f32_fp8, which decodes the fn
// variant exactly (checked against every code by the parity tests).
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

// Element (o, i) of a source matrix [O][I], decoded to fp32.  nbi = number
// of 128-wide block columns of the FP8 inverse scales.
template <int SRC>
__device__ __forceinline__ float src_elem(const void* __restrict__ w,
                                          const float* __restrict__ sinv, int64_t o, int64_t i,
                                          int64_t I, int64_t nbi)
{
    if constexpr (SRC == MOE_SRC_F32) {
        return ((const float*)w)[o * I + i];
    } else if constexpr (SRC == MOE_SRC_BF16) {
        return __uint_as_float((uint32_t)((const uint16_t*)w)[o * I + i] << 16);
    } else {
        const int b = ((const uint8_t*)w)[o * I + i];
        return __builtin_amdgcn_cvt_f32_fp8(b, 0) * sinv[(o >> 7) * nbi + (i >> 7)];
    }
}

// Any even I: one 256-thread workgroup per output row (grid-stride over rows).
template <int SRC>
__global__ void __launch_bounds__(256) k_pack_int4_rows(const void* __restrict__ w,
                                                        const float* __restrict__ sinv, int64_t O,
                                                        int64_t I, uint8_t* __restrict__ q,
                                                        float* __restrict__ s)
{
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t nbi = (I + 127) >> 7;
    for (int64_t o = blockIdx.x; o < O; o += gridDim.x) {
        float amax = 0.0f;
        for (int64_t i = tid; i < I; i += 256)
            amax = fmaxf(amax, fabsf(src_elem<SRC>(w, sinv, o, i, I, nbi)));
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
            int v0 = code_row(src_elem<SRC>(w, sinv, o, 2 * j, I, nbi), sc);
            int v1 = code_row(src_elem<SRC>(w, sinv, o, 2 * j + 1, I, nbi), sc);
            qr[j] = (uint8_t)((v0 & 0xF) | ((v1 & 0xF) << 4));
        }
    }
}

// ---------------------------------------------------------------------------
// Tiled requantiser for I a multiple of 32 up to 8192 (the expert shapes).
// A workgroup of 4 wavefronts takes 8 consecutive rows of one matrix, 2 per
// wavefront.  Lane l holds the 16-input units l, l + 64, ... of its row
// (each unit one coalesced 16-byte FP8 load, 32 bytes of bf16, 64 of fp32)
// in registers, so each element is read once; the row maximum is a
// wavefront max.  Codes go out as 8 bytes per unit: in the blob layout
// directly (consecutive lanes, consecutive bytes); in the slot interleave
// through LDS, so that each store writes the 8 rows' 16-byte pieces of one
// 32-input chunk, 128 contiguous bytes.  8-row tiles keep every tile of an
// expert resident at once (no partial second round of workgroups).
//
// Code = rint(fl(w / s)) with w = fl(v * bs) for FP8 (bs its block's
// inverse scale).  With y = fl(1/s) (correctly rounded, once per row), the
// quotient is q0 = w*y refined once, q = fma(fma(-s, q0, w), y, q0).  Only
// codes matter, and they can differ from the IEEE quotient's only where
// w/s lies within a few ulps of a half-integer; for every divisor
// significand and every dividend within 24 ulps of k*s (k = 0.5 .. 7.5) this
// sequence gives the IEEE quotient's code (exhaustive host check, with a
// test of its own), and the device parity tests compare every code with
// the oracle's IEEE division.  Adding 1.5 * 2^23 (+ 8 for the slot's offset
// binary) rounds to the nearest integer, ties to even, and leaves the code
// in the low byte, since s = fl(amax/7) bounds |w/s| by 7 plus an ulp.
// ---------------------------------------------------------------------------
struct RqMat {
    const void* src;     // [O][In] source elements
    const float* sinv;   // FP8 inverse scales [ceil(O/128)][ceil(In/128)]
    uint8_t* q;          // codes (blob rows or the slot's matrix)
    float* s;            // [O] row scales
    int O, In;
};

struct RqArgs {
    RqMat m[3];
    int tiles[3];        // 8-row tiles per matrix
};

constexpr int RQ_ROWS = 8;                        // rows per workgroup
constexpr int RQ_TSTRIDE = RQ_ROWS * 16 + 16;     // LDS bytes per 32-input chunk (padded)

template <int SRC> struct RqUnit;  // 16-byte loads per 16-input unit
template <> struct RqUnit<MOE_SRC_FP8_E4M3> { static constexpr int N = 1; };
template <> struct RqUnit<MOE_SRC_BF16> { static constexpr int N = 2; };
template <> struct RqUnit<MOE_SRC_F32> { static constexpr int N = 4; };

// Largest |value| of one unit, before the block scale.  FP8 and bf16 are
// sign-magnitude, so with the sign cleared their order is the integers'
// order (and rounding the product by a positive scale keeps it: max fl(|v|
// * bs) = fl(max|v| * bs)).
template <int SRC>
__device__ __forceinline__ float rq_unit_amax(const uint4 (&r)[RqUnit<SRC>::N])
{
    if constexpr (SRC == MOE_SRC_FP8_E4M3) {
        const uint32_t w[4] = {r[0].x & 0x7F7F7F7Fu, r[0].y & 0x7F7F7F7Fu, r[0].z & 0x7F7F7F7Fu,
                               r[0].w & 0x7F7F7F7Fu};
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = max(m, max(w[k] & 0xFFu, (w[k] >> 8) & 0xFFu));
            m = max(m, max((w[k] >> 16) & 0xFFu, w[k] >> 24));
        }
        return __builtin_amdgcn_cvt_f32_fp8((int)m, 0);
    } else if constexpr (SRC == MOE_SRC_BF16) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w[4] = {r[j].x, r[j].y, r[j].z, r[j].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
        }
        return __uint_as_float(m << 16);
    } else {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = fmaxf(m, fmaxf(fmaxf(fabsf(__uint_as_float(r[j].x)), fabsf(__uint_as_float(r[j].y))),
                               fmaxf(fabsf(__uint_as_float(r[j].z)), fabsf(__uint_as_float(r[j].w)))));
        return m;
    }
}

// Inputs 8h .. 8h+7 of a unit, decoded to fp32 (before the block scale).
template <int SRC>
__device__ __forceinline__ void rq_decode8(const uint4 (&r)[RqUnit<SRC>::N], int h, float (&v)[8])
{
    if constexpr (SRC == MOE_SRC_FP8_E4M3) {
        const uint32_t w[2] = {h ? r[0].z : r[0].x, h ? r[0].w : r[0].y};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
            v[4 * k + 0] = lo[0];
            v[4 * k + 1] = lo[1];
            v[4 * k + 2] = hi[0];
            v[4 * k + 3] = hi[1];
        }
    } else if constexpr (SRC == MOE_SRC_BF16) {
        const uint4 u = r[h];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(w[k] << 16);
            v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 u = r[2 * h + j];
            v[4 * j + 0] = __uint_as_float(u.x);
            v[4 * j + 1] = __uint_as_float(u.y);
            v[4 * j + 2] = __uint_as_float(u.z);
            v[4 * j + 3] = __uint_as_float(u.w);
        }
    }
}

// 8 codes (+ off) as nibbles, input 0 in the low nibble.  y = q + 1.5*2^23
// + off holds rint(q) + off in its low byte (two's complement).
__device__ __forceinline__ uint32_t rq_pack8(const float (&q)[8], float magic)
{
    uint32_t y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = __float_as_uint(q[e] + magic);
    const uint32_t ev = __builtin_amdgcn_perm(y[2], y[0], 0x0C0C0400u) |
                        __builtin_amdgcn_perm(y[6], y[4], 0x04000C0Cu);
    const uint32_t od = __builtin_amdgcn_perm(y[3], y[1], 0x0C0C0400u) |
                        __builtin_amdgcn_perm(y[7], y[5], 0x04000C0Cu);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

template <int SRC, bool SLOT>
__global__ void __launch_bounds__(RQ_ROWS * 32) k_requant_rows(RqArgs a)
{
    constexpr int NU = RqUnit<SRC>::N;
    constexpr int ESZ = SRC == MOE_SRC_FP8_E4M3 ? 1 : (SRC == MOE_SRC_BF16 ? 2 : 4);
    extern __shared__ __align__(16) uint8_t rq_tile[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int t = blockIdx.x, mi = 0;
    if (t >= a.tiles[0]) {
        t -= a.tiles[0];
        mi = 1;
        if (t >= a.tiles[1]) {
            t -= a.tiles[1];
            mi = 2;
        }
    }
    const RqMat m = a.m[mi];
    const int o0 = t * RQ_ROWS;
    const int U = m.In >> 4, C = m.In >> 5, nbi = (m.In + 127) >> 7;
    const float magic = SLOT ? 12582920.0f : 12582912.0f;  // 1.5 * 2^23 (+ 8)
#pragma unroll 1
    for (int rr = 0; rr < 2; ++rr) {
        const int ro = 2 * wv + rr, o = o0 + ro;
        if (o >= m.O) break;
        const uint8_t* row = (const uint8_t*)m.src + (size_t)o * m.In * ESZ;
        uint4 raw[8][NU];
        float bs[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int u = min(lane + 64 * k, U - 1);  // past the row end: reread its last unit
#pragma unroll
            for (int j = 0; j < NU; ++j) raw[k][j] = ((const uint4*)(row + (size_t)u * 16 * ESZ))[j];
            bs[k] = SRC == MOE_SRC_FP8_E4M3 ? m.sinv[(size_t)(o >> 7) * nbi + (u >> 3)] : 1.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (lane + 64 * k < U) {
                const float um = rq_unit_amax<SRC>(raw[k]);
                amax = fmaxf(amax, SRC == MOE_SRC_FP8_E4M3 ? um * bs[k] : um);
            }
        amax = wave_max(amax);
        float sc = __fdiv_rn(amax, 7.0f);
        if (sc < 1e-8f) sc = 1e-8f;
        const float rinv = __fdiv_rn(1.0f, sc);
        if (lane == 0) m.s[o] = sc;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int u = lane + 64 * k;
            if (u < U) {
                uint32_t nib[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float v[8], q[8];
                    rq_decode8<SRC>(raw[k], h, v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float w = SRC == MOE_SRC_FP8_E4M3 ? v[e] * bs[k] : v[e];
                        const float q0 = w * rinv;
                        q[e] = fmaf(fmaf(-sc, q0, w), rinv, q0);
                    }
                    nib[h] = rq_pack8(q, magic);
                }
                if (SLOT)
                    *(uint2*)(rq_tile + (u >> 1) * RQ_TSTRIDE + ro * 16 + (u & 1) * 8) =
                        make_uint2(nib[0], nib[1]);
                else
                    *(uint2*)(m.q + (size_t)o * (m.In / 2) + (size_t)u * 8) = make_uint2(nib[0], nib[1]);
            }
        }
    }
    if (SLOT) {  // every matrix's O is a multiple of 64, so the tile is full
        // the tile's 8 rows are one 8-row group of the slot layout: C * 128
        // contiguous bytes
        __syncthreads();
        uint8_t* gq = m.q + (size_t)(o0 >> 3) * C * 128;
        for (int i = threadIdx.x; i < C * RQ_ROWS; i += RQ_ROWS * 32) {
            const int c = i / RQ_ROWS, r = i % RQ_ROWS;
            *(uint4*)(gq + ((size_t)c * RQ_ROWS + r) * 16) =
                *(const uint4*)(rq_tile + c * RQ_TSTRIDE + r * 16);
        }
    }
}

// Per-row int8 ("惊呆了！…" §05 quantize_rows with bits = 8): s = max|w|/127
// floored at 1e-8, code = rint(w / s) clamped to [-128, 127], q [O][I] int8.
// One 256-thread workgroup per row.
template <int SRC>
__global__ void __launch_bounds__(256) k_pack_int8_rows(const void* __restrict__ w,
                                                        const float* __restrict__ sinv, int64_t O,
                                                        int64_t I, int8_t* __restrict__ q,
                                                        float* __restrict__ s)
{
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t nbi = (I + 127) >> 7;
    for (int64_t o = blockIdx.x; o < O; o += gridDim.x) {
        float amax = 0.0f;
        for (int64_t i = tid; i < I; i += 256)
            amax = fmaxf(amax, fabsf(src_elem<SRC>(w, sinv, o, i, I, nbi)));
        amax = wave_max(amax);
        if ((tid & 63) == 0) red[tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float sc = __fdiv_rn(amax, 127.0f);
        if (sc < 1e-8f) sc = 1e-8f;
        if (tid == 0) s[o] = sc;
        for (int64_t i = tid; i < I; i += 256) {
            int v = (int)rintf(__fdiv_rn(src_elem<SRC>(w, sinv, o, i, I, nbi), sc));
            q[o * I + i] = (int8_t)(v > 127 ? 127 : (v < -128 ? -128 : v));
        }
    }
}

// One wavefront per (row, group of 64 inputs); 4 groups per workgroup.
template <int SRC>
__global__ void __launch_bounds__(256) k_pack_affine_g64(const void* __restrict__ w,
                                                         const float* __restrict__ sinv, int64_t O,
                                                         int64_t I, uint8_t* __restrict__ q,
                                                         uint16_t* __restrict__ scmn)
{
    const int lane = threadIdx.x & 63;
    const int64_t G = I / 64;
    const int64_t total = O * G;
    const int64_t nbi = (I + 127) >> 7;
    for (int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); item < total;
         item += (int64_t)gridDim.x * 4) {
        const int64_t o = item / G, g = item % G;
        const float v = src_elem<SRC>(w, sinv, o, g * 64 + lane, I, nbi);
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

// Blob matrix [O][In/2] bytes <-> slot interleave (see moe_internal.h):
// groups of R rows, the 16-byte pieces of a group's rows for one chunk of 32
// inputs contiguous, chunk after chunk (R = 8 for the int4 formats; R = 64
// for int8 matrices, passed as int4 matrices of twice the width).  One
// thread per 16-byte chunk; `flip` = 0x88888888 for the row format.
template <int R>
__global__ void __launch_bounds__(256) k_interleave(const uint8_t* __restrict__ src,
                                                    uint8_t* __restrict__ dst, int64_t O,
                                                    int64_t In, uint32_t flip, int to_slot)
{
    const int64_t C = In / 32;
    const int64_t total = O * C;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t r = idx % R, c = (idx / R) % C, grp = (idx / R) / C;
        const int64_t canon = (grp * R + r) * (In / 2) + c * 16;
        const int64_t inter = idx * 16;
        uint4 v = *(const uint4*)(src + (to_slot ? canon : inter));
        v.x ^= flip;
        v.y ^= flip;
        v.z ^= flip;
        v.w ^= flip;
        *(uint4*)(dst + (to_slot ? inter : canon)) = v;
    }
}

// Affine (scale, min) pairs: blob [O][G] <-> slot [O/8][G][8], 4 B each.
__global__ void __launch_bounds__(256) k_interleave_pairs(const uint32_t* __restrict__ src,
                                                          uint32_t* __restrict__ dst, int64_t O,
                                                          int64_t G, int to_slot)
{
    const int64_t total = O * G;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t r = idx & 7, g = (idx >> 3) % G, grp = (idx >> 3) / G;
        const int64_t canon = (grp * 8 + r) * G + g;
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

// Router W [E][H] -> the large-T router's split fp16 copy.  Each expert row
// is scaled by 2^k (its largest magnitude then in [2^13, 2^14), exact) and
// each scaled weight v is held as hi = fp16(v) and lo = fp16(v - hi), 22
// significant bits together.  Layout [Epad/32][H/16][64][2] uint4: lane
// l = 32 h + m of expert block b holds expert 32 b + m, inputs 16 s + 8 h ..
// 16 s + 8 h + 7 in order, hi then lo (the B operands of a 32 x 32 x 16
// fp16 matrix-core step).  Rows >= E are zero; s16[e] = (2^k, 2^-k).
__global__ void __launch_bounds__(256) k_router_rowscale(const float* __restrict__ W, int E,
                                                         int H, float2* __restrict__ s16)
{
    __shared__ float s_m[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    float m = 0.f;
    if (e < E)
        for (int k = tid; k < H; k += 256) m = fmaxf(m, fabsf(W[(size_t)e * H + k]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((tid & 63) == 0) s_m[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) {
        m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
        int ex = 0;
        int k = 0;
        if (m > 0.f && m <= 3.402823466e38f) {
            (void)frexpf(m, &ex);  // m in [2^(ex-1), 2^ex)
            k = 14 - ex;
            k = k > 100 ? 100 : k < -100 ? -100 : k;
        }
        s16[e] = make_float2(ldexpf(1.f, k), ldexpf(1.f, -k));
    }
}

__global__ void __launch_bounds__(256) k_router_split(const float* __restrict__ W,
                                                      const float2* __restrict__ s16,
                                                      uint4* __restrict__ w16, int E, int Epad,
                                                      int H)
{
    const int64_t S = H / 16;
    const int64_t total = (int64_t)(Epad / 32) * S * 64;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int l = (int)(idx & 63);
        const int64_t s = (idx >> 6) % S, b = (idx >> 6) / S;
        const int64_t e = b * 32 + (l & 31);
        uint32_t hi[4] = {0u, 0u, 0u, 0u}, lo[4] = {0u, 0u, 0u, 0u};
        if (e < E) {
            const float sc = s16[e].x;
            const float* src = W + e * H + s * 16 + (l >> 5) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hp = 0u, lp = 0u;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float v = src[2 * i + j] * sc;
                    const _Float16 a = (_Float16)v;
                    const _Float16 r = (_Float16)(v - (float)a);
                    hp |= (uint32_t)__builtin_bit_cast(uint16_t, a) << (16 * j);
                    lp |= (uint32_t)__builtin_bit_cast(uint16_t, r) << (16 * j);
                }
                hi[i] = hp;
                lo[i] = lp;
            }
        }
        w16[2 * idx] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        w16[2 * idx + 1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
}

static unsigned grid_for(int64_t items, int64_t per_block)
{
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The tiled kernel covers In a multiple of 32 up to 8192 with 16-byte
// aligned rows.
static bool rq_fast_ok(const void* src, const void* q, int64_t O, int64_t In)
{
    return In > 0 && In % 32 == 0 && In <= 8192 && O < (1 << 30) && aligned16(src) &&
           aligned16(q);
}

template <bool SLOT>
static hipError_t launch_rq(int src, const RqArgs& a, hipStream_t st)
{
    int maxC = 0;
    for (int i = 0; i < 3; ++i)
        if (a.tiles[i] > 0 && a.m[i].In / 32 > maxC) maxC = a.m[i].In / 32;
    const dim3 grid(a.tiles[0] + a.tiles[1] + a.tiles[2]), block(RQ_ROWS * 32);
    const size_t lds = SLOT ? (size_t)maxC * RQ_TSTRIDE : 0;
    switch (src) {
    case MOE_SRC_F32:
        hipLaunchKernelGGL((k_requant_rows<MOE_SRC_F32, SLOT>), grid, block, lds, st, a);
        break;
    case MOE_SRC_BF16:
        hipLaunchKernelGGL((k_requant_rows<MOE_SRC_BF16, SLOT>), grid, block, lds, st, a);
        break;
    case MOE_SRC_FP8_E4M3:
        hipLaunchKernelGGL((k_requant_rows<MOE_SRC_FP8_E4M3, SLOT>), grid, block, lds, st, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant_rows(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                               uint8_t* q, float* s, hipStream_t st)
{
    if (rq_fast_ok(w, q, O, I)) {
        RqArgs a{};
        a.m[0] = RqMat{w, sinv, q, s, (int)O, (int)I};
        a.tiles[0] = (int)((O + RQ_ROWS - 1) / RQ_ROWS);
        return launch_rq<false>(src, a, st);
    }
    const dim3 grid(grid_for(O, 1)), block(256);
    switch (src) {
    case MOE_SRC_F32:
        hipLaunchKernelGGL(k_pack_int4_rows<MOE_SRC_F32>, grid, block, 0, st, w, sinv, O, I, q, s);
        break;
    case MOE_SRC_BF16:
        hipLaunchKernelGGL(k_pack_int4_rows<MOE_SRC_BF16>, grid, block, 0, st, w, sinv, O, I, q, s);
        break;
    case MOE_SRC_FP8_E4M3:
        hipLaunchKernelGGL(k_pack_int4_rows<MOE_SRC_FP8_E4M3>, grid, block, 0, st, w, sinv, O, I, q,
                           s);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant_affine(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                                 uint8_t* q, uint16_t* scmn, hipStream_t st)
{
    const dim3 grid(grid_for(O * (I / 64), 4)), block(256);
    switch (src) {
    case MOE_SRC_F32:
        hipLaunchKernelGGL(k_pack_affine_g64<MOE_SRC_F32>, grid, block, 0, st, w, sinv, O, I, q,
                           scmn);
        break;
    case MOE_SRC_BF16:
        hipLaunchKernelGGL(k_pack_affine_g64<MOE_SRC_BF16>, grid, block, 0, st, w, sinv, O, I, q,
                           scmn);
        break;
    case MOE_SRC_FP8_E4M3:
        hipLaunchKernelGGL(k_pack_affine_g64<MOE_SRC_FP8_E4M3>, grid, block, 0, st, w, sinv, O, I,
                           q, scmn);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_requant_int8_rows(const void* w, int src, const float* sinv, int64_t O,
                                    int64_t I, int8_t* q, float* s, hipStream_t st)
{
    const dim3 grid(grid_for(O, 1)), block(256);
    switch (src) {
    case MOE_SRC_F32:
        hipLaunchKernelGGL(k_pack_int8_rows<MOE_SRC_F32>, grid, block, 0, st, w, sinv, O, I, q, s);
        break;
    case MOE_SRC_BF16:
        hipLaunchKernelGGL(k_pack_int8_rows<MOE_SRC_BF16>, grid, block, 0, st, w, sinv, O, I, q, s);
        break;
    case MOE_SRC_FP8_E4M3:
        hipLaunchKernelGGL(k_pack_int8_rows<MOE_SRC_FP8_E4M3>, grid, block, 0, st, w, sinv, O, I, q,
                           s);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool requant_slot_ok(const void* wg, const void* wu, const void* wd, const uint8_t* slot, int H,
                     int I)
{
    const int64_t gq = (int64_t)I * (H / 2);
    return rq_fast_ok(wg, slot, I, H) && rq_fast_ok(wu, slot + gq, I, H) &&
           rq_fast_ok(wd, slot + 2 * gq, H, I);
}

// Row format: the three matrices of one expert in one launch, codes and
// scales written straight into the slot.
hipError_t launch_requant_slot(int src, const void* wg, const void* wu, const void* wd,
                               const float* sg, const float* su, const float* sd, int H, int I,
                               uint8_t* slot, hipStream_t st)
{
    const int64_t gq = (int64_t)I * (H / 2), dq = (int64_t)H * (I / 2);
    float* sc = (float*)(slot + 2 * gq + dq);
    RqArgs a{};
    a.m[0] = RqMat{wg, sg, slot, sc, I, H};
    a.m[1] = RqMat{wu, su, slot + gq, sc + I, I, H};
    a.m[2] = RqMat{wd, sd, slot + 2 * gq, sc + 2 * I, H, I};
    a.tiles[0] = a.tiles[1] = I / RQ_ROWS;
    a.tiles[2] = H / RQ_ROWS;
    return launch_rq<true>(src, a, st);
}

static hipError_t convert(const uint8_t* src, uint8_t* dst, int fmt, int H, int I, int to_slot,
                          uint32_t flip, hipStream_t st)
{
    if (fmt == MOE_W_INT8_ROW) {
        // int8 matrices [O][In]: 64-row blocks of 16-input chunks, codes offset
        // binary (q + 128 = byte ^ 0x80); the interleave of an int4 matrix of
        // twice the width has exactly that layout
        const int64_t m8 = (int64_t)I * H;
        const int64_t mats[3][3] = {{0, I, H}, {m8, I, H}, {2 * m8, H, I}};
        for (auto& m : mats)
            hipLaunchKernelGGL(k_interleave<64>, dim3(grid_for(m[1] * (m[2] / 16), 256)), dim3(256), 0,
                               st, src + m[0], dst + m[0], m[1], 2 * m[2], 0x80808080u, to_slot);
        const hipError_t e = hipMemcpyAsync(dst + 3 * m8, src + 3 * m8, (size_t)(2 * I + H) * 4,
                                            hipMemcpyDeviceToDevice, st);
        return e != hipSuccess ? e : hipGetLastError();
    }
    const int64_t gq = (int64_t)I * (H / 2), dq = (int64_t)H * (I / 2);
    const int64_t mats[3][3] = {{0, I, H}, {gq, I, H}, {2 * gq, H, I}};  // offset, O, In
    for (auto& m : mats) {
        hipLaunchKernelGGL(k_interleave<8>, dim3(grid_for(m[1] * (m[2] / 32), 256)), dim3(256), 0,
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

static uint32_t blob_flip(int fmt)
{
    return fmt == MOE_W_INT4_ROW ? 0x88888888u : (fmt == MOE_W_INT8_ROW ? 0x80808080u : 0u);
}

hipError_t launch_blob_to_slot(const uint8_t* blob, uint8_t* slot, int fmt, int H, int I,
                               hipStream_t st)
{
    return convert(blob, slot, fmt, H, I, 1, blob_flip(fmt), st);
}

hipError_t launch_slot_to_blob(const uint8_t* slot, uint8_t* blob, int fmt, int H, int I,
                               hipStream_t st)
{
    return convert(slot, blob, fmt, H, I, 0, blob_flip(fmt), st);
}

// The converter's container (row format, codes already offset binary, the
// slot's own coding): interleave only.
hipError_t launch_container_to_slot(const uint8_t* staged, uint8_t* slot, int H, int I,
                                    hipStream_t st)
{
    return convert(staged, slot, MOE_W_INT4_ROW, H, I, 1, 0u, st);
}

hipError_t launch_router_to_internal(const float* W, float* wr, int E, int Epad, int H,
                                     hipStream_t st)
{
    hipLaunchKernelGGL(k_router_layout, dim3(grid_for((int64_t)Epad * (H / 4), 256)), dim3(256),
                       0, st, W, (float4*)wr, E, Epad, H);
    return hipGetLastError();
}

hipError_t launch_router_split(const float* W, uint4* w16, float2* w16s, int E, int Epad, int H,
                               hipStream_t st)
{
    hipLaunchKernelGGL(k_router_rowscale, dim3(Epad), dim3(256), 0, st, W, E, H, w16s);
    hipLaunchKernelGGL(k_router_split, dim3(grid_for((int64_t)(Epad / 32) * (H / 16) * 64, 256)),
                       dim3(256), 0, st, W, (const float2*)w16s, w16, E, Epad, H);
    return hipGetLastError();
}

}  // namespace moe
