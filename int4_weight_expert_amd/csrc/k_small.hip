// k_small.hip -- the decode-size forward (few tokens): router GEMV with
// wavefront top-k and bucketing, fused int4 gate/up GEMV with SiLU*up, and
// the int4 down GEMV with a deterministic weighted combine.
//
// What is computed, cited by page title and section:
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11: the router is
//     an fp32 GEMV, sigmoid(logit) + correction bias picks the top-K (a strict
//     greater-than scan, so equal scores go to the lower id), the weight is
//     the plain sigmoid times the routed scale; the batch's experts are
//     deduplicated so each is read once; each expert is SwiGLU
//     (gate/up -> silu(g)*u -> down) and its output is added with its weight;
//     §04 siluf(x) = x/(1+exp(-x)) and the double-accumulated rmsnorm.
//   Edge0 write-up (magicnetworld.com) §七: the chosen sigmas are
//     renormalised, w_i = s * sigma_i / (sum sigma + 1e-20); §三: affine int4
//     with group size 64.
//   GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6c/6d: the shared
//     expert is always active and is added to the routed sum.
//
// Roofline: all three kernels are HBM-bound at decode sizes.  The GEMVs read
// each resident expert byte once (weights as 1 KiB coalesced wavefront
// loads, activations as wave-uniform scalar loads), unpack two codes per
// byte with one AND per 8 codes and one v_cvt_f32_ubyteN per code, and
// accumulate in fp32 with v_fmac (18 VALU operations per 8 weights).
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

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

// 8 codes of one dword against 8 activations.  Even columns sit in the low
// nibbles (value v), odd columns in the high nibbles (value 16 v): they go
// to separate accumulators and the odd one is scaled by 1/16 at the end.
__device__ __forceinline__ void dot8(uint32_t w, const float* __restrict__ xs, float& ae, float& ao)
{
    const uint32_t lo = and_opaque(w, 0x0F0F0F0Fu), hi = and_opaque(w, 0xF0F0F0F0u);
    ae = fmaf(ub0(lo), xs[0], ae);
    ao = fmaf(ub0(hi), xs[1], ao);
    ae = fmaf(ub1(lo), xs[2], ae);
    ao = fmaf(ub1(hi), xs[3], ao);
    ae = fmaf(ub2(lo), xs[4], ae);
    ao = fmaf(ub2(hi), xs[5], ao);
    ae = fmaf(ub3(lo), xs[6], ae);
    ao = fmaf(ub3(hi), xs[7], ao);
}

__device__ __forceinline__ void dot32(const uint4& w, const float* __restrict__ xs, float& ae,
                                      float& ao)
{
    dot8(w.x, xs, ae, ao);
    dot8(w.y, xs + 8, ae, ao);
    dot8(w.z, xs + 16, ae, ao);
    dot8(w.w, xs + 24, ae, ao);
}

// Token j of a group: its token index t and its row r in h / ystage
// (routed assignment a = t*K + k uses row a; shared expert s uses
// T*K + s*T + t).
__device__ __forceinline__ void tok_rows(const Fwd& f, const Group& g, int j, int& t, int& r)
{
    if (g.kind == 0) {
        const int a = f.perm[g.off + j];
        t = a / f.K;
        r = a;
    } else {
        t = j;
        r = f.T * f.K + g.off * f.T + j;
    }
}

__device__ __forceinline__ uint32_t ord_float(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Router tail (one 256-thread workgroup): token statistics, sigmoid, bias,
// top-K per token, weights, bucketing into expert groups, slot resolution.
// Used by the small-T router (after the last partial arrives) for T <= 16.
// ---------------------------------------------------------------------------

template <int NT>
__device__ void router_tail(const Fwd& f)
{
    __shared__ float s_c[NT][256];
    __shared__ float s_sig[NT][256];
    __shared__ float s_rs[NT];
    __shared__ int s_ids[NT * 8];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_nact;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = f.T, H = f.H, E = f.E, K = f.K, Epad = f.Epad;

    // 1. token statistics: sum, RMSNorm factor, sums of 64-column groups
    for (int t = w; t < T; t += 4) {
        const float* xt = f.x + (size_t)t * H;
        float sum = 0.f, ss = 0.f;
        for (int i0 = 0; i0 < H; i0 += 256) {
            const float4 v = *(const float4*)(xt + i0 + lane * 4);
            float gs = (v.x + v.y) + (v.z + v.w);
            sum += gs;
            ss = fmaf(v.x, v.x, ss);
            ss = fmaf(v.y, v.y, ss);
            ss = fmaf(v.z, v.z, ss);
            ss = fmaf(v.w, v.w, ss);
            gs += __shfl_xor(gs, 1);
            gs += __shfl_xor(gs, 2);
            gs += __shfl_xor(gs, 4);
            gs += __shfl_xor(gs, 8);
            if ((lane & 15) == 0) f.xgs[(size_t)t * (H / 64) + (i0 >> 6) + (lane >> 4)] = gs;
        }
        sum = wave_sum(sum);
        ss = wave_sum(ss);
        if (lane == 0) {
            const float rs = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
            f.tok[t].xsum = sum;
            f.tok[t].rscale = rs;
            s_rs[t] = rs;
        }
    }
    __syncthreads();

    // 2. logits (fixed-order sum of the K-slice partials), sigmoid, score
    if (tid < Epad) {
        for (int t = 0; t < T; ++t) {
            float l = 0.f;
            for (int s = 0; s < f.S; ++s) l += f.part[((size_t)s * T + t) * Epad + tid];
            l *= s_rs[t];
            float sig = 0.f, c = -INFINITY;
            if (tid < E) {
                sig = 1.0f / (1.0f + expf(-l));
                c = sig + f.bias[tid];
            }
            s_c[t][tid] = c;
            s_sig[t][tid] = sig;
        }
    }
    for (int e = tid; e < 256; e += 256) s_cnt[e] = 0;
    __syncthreads();

    // 3. top-K per token: K rounds of a wavefront argmax over 64-bit keys
    //    (score order, then lower id), one wavefront per token
    for (int t = w; t < T; t += 4) {
        uint32_t taken = 0;
        float ssum = 0.f;
        for (int kk = 0; kk < K; ++kk) {
            unsigned long long best = 0ull;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int e = lane + 64 * m;
                if (e < Epad && !(taken & (1u << m))) {
                    const unsigned long long key =
                        ((unsigned long long)ord_float(s_c[t][e]) << 32) | (uint32_t)(0xFFFFu - e);
                    best = key > best ? key : best;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const unsigned long long other = __shfl_xor(best, o);
                best = other > best ? other : best;
            }
            const int e = 0xFFFF - (int)(best & 0xFFFFu);
            if ((e & 63) == lane) taken |= 1u << (e >> 6);
            if (lane == 0) s_ids[t * K + kk] = e;
            ssum += s_sig[t][e];
        }
        if (lane < K) {
            const int e = s_ids[t * K + lane];
            const float sg = s_sig[t][e];
            const float wv = f.norm_topk ? f.routed_scale * (sg / (ssum + 1e-20f)) : f.routed_scale * sg;
            f.ids[t * K + lane] = e;
            f.wts[t * K + lane] = wv;
        }
    }
    __syncthreads();

    // 4. bucketing: counts, exclusive scan, stable scatter, active groups
    const int n = T * K;
    if (tid < n) atomicAdd(&s_cnt[s_ids[tid]], 1);
    __syncthreads();
    if (w == 0) {
        int c4[4], a4[4], sc = 0, sa = 0;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            c4[m] = s_cnt[lane * 4 + m];
            a4[m] = c4[m] > 0;
            sc += c4[m];
            sa += a4[m];
        }
        int ic = sc, ia = sa;  // inclusive wavefront scans
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int pc = __shfl_up(ic, o), pa = __shfl_up(ia, o);
            if (lane >= o) {
                ic += pc;
                ia += pa;
            }
        }
        int rc = ic - sc, ra = ia - sa;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            s_off[lane * 4 + m] = rc;
            s_act[lane * 4 + m] = a4[m] ? ra : -1;
            rc += c4[m];
            ra += a4[m];
        }
        if (lane == 63) {
            s_off[256] = rc;
            s_nact = ra;
        }
    }
    __syncthreads();
    if (tid < n) {
        const int e = s_ids[tid];
        int rank = 0;
        for (int a = 0; a < tid; ++a) rank += s_ids[a] == e;
        f.perm[s_off[e] + rank] = tid;
    }
    if (tid < E) {
        f.cnt[tid] = s_cnt[tid];
        f.off[tid] = s_off[tid];
        if (tid == 0) f.off[E] = s_off[E];
        const int idx = s_act[tid];
        if (idx >= 0) {
            f.active[idx] = tid;
            const int slot = f.tbl[tid];
            Group g;
            g.base = slot >= 0 ? f.pool + (size_t)slot * f.slot_bytes : nullptr;
            g.cnt = s_cnt[tid];
            g.off = s_off[tid];
            g.kind = 0;
            g.expert = tid;
            f.groups[f.n_shared + idx] = g;
            if (slot < 0) {
                atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
                const int code = f.layer * E + tid;
                atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
            }
        }
    }
    if (tid < f.n_shared) {
        Group g;
        g.base = f.shared + (size_t)tid * f.slot_bytes;
        g.cnt = T;
        g.off = tid;
        g.kind = 1;
        g.expert = -1;
        f.groups[tid] = g;
    }
    if (tid == 0) {
        f.n_active[0] = s_nact;
        f.n_groups[0] = f.n_shared + s_nact;
    }
}

// ---------------------------------------------------------------------------
// Small-T router: split-K GEMV over the interleaved router weights.
// Workgroup (b, q) = expert block b (64 experts, one per lane) and K-slices
// 4q..4q+3 (one per wavefront).  Partials go to f.part; the last workgroup
// to arrive runs router_tail.
// ---------------------------------------------------------------------------

template <int NT>
__global__ void __launch_bounds__(256) k_router_small(Fwd f)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x, s = blockIdx.y * 4 + w;
    const int H = f.H, T = f.T, CH = H / 4;
    const int cs = CH / f.S, c0 = s * cs;
    const float4* wr = (const float4*)f.wr + (size_t)b * CH * 64 + lane;
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.f;
    int c = c0;
    for (; c + 4 <= c0 + cs; c += 4) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = wr[(size_t)(c + u) * 64];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j < T) {
                const float* xs = f.x + (size_t)j * H + c * 4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    acc[j] = fmaf(v[u].x, xs[4 * u + 0], acc[j]);
                    acc[j] = fmaf(v[u].y, xs[4 * u + 1], acc[j]);
                    acc[j] = fmaf(v[u].z, xs[4 * u + 2], acc[j]);
                    acc[j] = fmaf(v[u].w, xs[4 * u + 3], acc[j]);
                }
            }
        }
    }
    for (; c < c0 + cs; ++c) {
        const float4 v = wr[(size_t)c * 64];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j < T) {
                const float* xs = f.x + (size_t)j * H + c * 4;
                acc[j] = fmaf(v.x, xs[0], acc[j]);
                acc[j] = fmaf(v.y, xs[1], acc[j]);
                acc[j] = fmaf(v.z, xs[2], acc[j]);
                acc[j] = fmaf(v.w, xs[3], acc[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
        if (j < T) f.part[((size_t)s * T + j) * f.Epad + b * 64 + lane] = acc[j];

    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&f.counters[0], 1u);
        s_last = prev == gridDim.x * gridDim.y - 1;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (threadIdx.x == 0) f.counters[0] = 0;
    router_tail<NT>(f);
}

// ---------------------------------------------------------------------------
// Gate/up GEMV: workgroup (b, g) computes h = silu(g)*u for the 64 rows
// 64b..64b+63 of group g's expert and every token of the group; NW
// wavefronts split the input columns and meet in LDS.
// ---------------------------------------------------------------------------

template <int FMT, int NT, int NW>
__global__ void __launch_bounds__(NW * 64) k_gateup(Fwd f)
{
    const int b = blockIdx.x, gi = blockIdx.y;
    if (gi >= f.n_groups[0]) return;
    const Group grp = f.groups[gi];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = f.H, I = f.I, C = H / 32;
    const int row = b * 64 + lane;
    __shared__ float red[NT][2][NW][64];

    const int c0 = (w * C) / NW, c1 = ((w + 1) * C) / NW;
    const uint4* qg = (const uint4*)grp.base + (size_t)b * C * 64 + lane;
    const uint4* qu = (const uint4*)(grp.base + (size_t)I * H / 2) + (size_t)b * C * 64 + lane;

    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        if (grp.base == nullptr) {
            for (int j = w; j < nj; j += NW) {
                int t, r;
                tok_rows(f, grp, p0 + j, t, r);
                f.h[(size_t)r * I + row] = 0.f;
                if (lane == 0) f.hgs[(size_t)r * (I / 64) + b] = 0.f;
            }
            continue;
        }
        const float* xp[NT];
        int tt[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int t = 0, r = 0;
            if (j < nj) tok_rows(f, grp, p0 + j, t, r);
            tt[j] = t;
            xp[j] = f.x + (size_t)t * H;
        }
        float ge[NT], go[NT], ue[NT], uo[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) ge[j] = go[j] = ue[j] = uo[j] = 0.f;

        if (FMT == MOE_W_INT4_ROW) {
            int c = c0;
            for (; c + 4 <= c1; c += 4) {
                uint4 vg[4], vu[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    vg[u] = qg[(size_t)(c + u) * 64];
                    vu[u] = qu[(size_t)(c + u) * 64];
                }
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    if (j < nj) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float* xs = xp[j] + (c + u) * 32;
                            dot32(vg[u], xs, ge[j], go[j]);
                            dot32(vu[u], xs, ue[j], uo[j]);
                        }
                    }
                }
            }
            for (; c < c1; ++c) {
                const uint4 vg = qg[(size_t)c * 64], vu = qu[(size_t)c * 64];
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
                        const float* xs = xp[j] + c * 32;
                        dot32(vg, xs, ge[j], go[j]);
                        dot32(vu, xs, ue[j], uo[j]);
                    }
            }
        } else {
            // affine: groups of 64 inputs = 2 chunks; scale/min per (row, group)
            const int G = H / 64;
            const uint32_t* ag =
                (const uint32_t*)(grp.base + (size_t)3 * H * I / 2) + (size_t)b * G * 64 + lane;
            const uint32_t* au = ag + (size_t)I * G;
            for (int gq = c0 / 2; gq < c1 / 2; ++gq) {
                const uint4 g0 = qg[(size_t)(2 * gq) * 64], g1 = qg[(size_t)(2 * gq + 1) * 64];
                const uint4 u0 = qu[(size_t)(2 * gq) * 64], u1 = qu[(size_t)(2 * gq + 1) * 64];
                const uint32_t pg = ag[(size_t)gq * 64], pu = au[(size_t)gq * 64];
                const float scg = __uint_as_float(pg << 16), mng = __uint_as_float(pg & 0xFFFF0000u);
                const float scu = __uint_as_float(pu << 16), mnu = __uint_as_float(pu & 0xFFFF0000u);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
                        const float* xs = xp[j] + gq * 64;
                        float ae = 0.f, ao = 0.f, be = 0.f, bo = 0.f;
                        dot32(g0, xs, ae, ao);
                        dot32(g1, xs + 32, ae, ao);
                        dot32(u0, xs, be, bo);
                        dot32(u1, xs + 32, be, bo);
                        const float sx = f.xgs[(size_t)tt[j] * G + gq];
                        ge[j] = fmaf(scg, fmaf(ao, 0.0625f, ae), fmaf(mng, sx, ge[j]));
                        ue[j] = fmaf(scu, fmaf(bo, 0.0625f, be), fmaf(mnu, sx, ue[j]));
                    }
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            red[j][0][w][lane] = fmaf(go[j], 0.0625f, ge[j]);
            red[j][1][w][lane] = fmaf(uo[j], 0.0625f, ue[j]);
        }
        __syncthreads();
        for (int j = w; j < nj; j += NW) {
            float G = 0.f, U = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) {
                G += red[j][0][v][lane];
                U += red[j][1][v][lane];
            }
            int t, r;
            tok_rows(f, grp, p0 + j, t, r);
            const TokStat ts = f.tok[t];
            if (FMT == MOE_W_INT4_ROW) {
                const float* sg = (const float*)(grp.base + (size_t)3 * H * I / 2);
                G = (G - 8.0f * ts.xsum) * sg[row];
                U = (U - 8.0f * ts.xsum) * sg[I + row];
            }
            G *= ts.rscale;
            U *= ts.rscale;
            const float hv = G / (1.0f + expf(-G)) * U;
            f.h[(size_t)r * I + row] = hv;
            const float hs = wave_sum(hv);
            if (lane == 0) f.hgs[(size_t)r * (I / 64) + b] = hs;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Down GEMV + combine: workgroup (b, g) computes y for output rows
// 64b..64b+63 of group g's expert for every token of the group into ystage;
// the last group to finish row block b combines all groups for all tokens
// in a fixed order (shared experts, then routed experts in rank order).
// ---------------------------------------------------------------------------

template <int FMT, int NT, int NW>
__global__ void __launch_bounds__(NW * 64) k_down(Fwd f)
{
    const int b = blockIdx.x, gi = blockIdx.y;
    const int n_groups = f.n_groups[0];
    if (gi >= n_groups) return;
    const Group grp = f.groups[gi];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = f.H, I = f.I, C = I / 32, GI = I / 64;
    const int row = b * 64 + lane;
    __shared__ float red[NT][NW][64];
    __shared__ int s_last;

    const int c0 = (w * C) / NW, c1 = ((w + 1) * C) / NW;
    const uint4* qd = (const uint4*)(grp.base + (size_t)I * H) + (size_t)b * C * 64 + lane;

    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        if (grp.base == nullptr) {
            for (int j = w; j < nj; j += NW) {
                int t, r;
                tok_rows(f, grp, p0 + j, t, r);
                f.ystage[(size_t)r * H + row] = 0.f;
            }
            continue;
        }
        const float* hp[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int t = 0, r = 0;
            if (j < nj) tok_rows(f, grp, p0 + j, t, r);
            hp[j] = f.h + (size_t)r * I;
        }
        float ye[NT], yo[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) ye[j] = yo[j] = 0.f;

        if (FMT == MOE_W_INT4_ROW) {
            int c = c0;
            for (; c + 4 <= c1; c += 4) {
                uint4 vd[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) vd[u] = qd[(size_t)(c + u) * 64];
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
#pragma unroll
                        for (int u = 0; u < 4; ++u) dot32(vd[u], hp[j] + (c + u) * 32, ye[j], yo[j]);
                    }
            }
            for (; c < c1; ++c) {
                const uint4 vd = qd[(size_t)c * 64];
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) dot32(vd, hp[j] + c * 32, ye[j], yo[j]);
            }
        } else {
            const uint32_t* ad = (const uint32_t*)(grp.base + (size_t)3 * H * I / 2) +
                                 (size_t)2 * I * (H / 64) + (size_t)b * GI * 64 + lane;
            for (int gq = c0 / 2; gq < c1 / 2; ++gq) {
                const uint4 d0 = qd[(size_t)(2 * gq) * 64], d1 = qd[(size_t)(2 * gq + 1) * 64];
                const uint32_t pd = ad[(size_t)gq * 64];
                const float sc = __uint_as_float(pd << 16), mn = __uint_as_float(pd & 0xFFFF0000u);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
                        const float* hs = hp[j] + gq * 64;
                        float ae = 0.f, ao = 0.f;
                        dot32(d0, hs, ae, ao);
                        dot32(d1, hs + 32, ae, ao);
                        const float sh = f.hgs[(size_t)(hp[j] - f.h) / I * GI + gq];
                        ye[j] = fmaf(sc, fmaf(ao, 0.0625f, ae), fmaf(mn, sh, ye[j]));
                    }
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) red[j][w][lane] = fmaf(yo[j], 0.0625f, ye[j]);
        __syncthreads();
        for (int j = w; j < nj; j += NW) {
            float Y = 0.f;
#pragma unroll
            for (int v = 0; v < NW; ++v) Y += red[j][v][lane];
            int t, r;
            tok_rows(f, grp, p0 + j, t, r);
            if (FMT == MOE_W_INT4_ROW) {
                float hsum = 0.f;
                for (int q = 0; q < GI; ++q) hsum += f.hgs[(size_t)r * GI + q];
                const float* sd = (const float*)(grp.base + (size_t)3 * H * I / 2) + 2 * I;
                Y = (Y - 8.0f * hsum) * sd[row];
            }
            f.ystage[(size_t)r * H + row] = Y;
        }
        __syncthreads();
    }

    // arrival; the last group of this row block combines
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicAdd(&f.counters[1 + b], 1u);
        s_last = prev == (uint32_t)(n_groups - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const int T = f.T, K = f.K;
    for (int t = w; t < T; t += NW) {
        float m = 0.f;
        for (int s = 0; s < f.n_shared; ++s) m += f.ystage[(size_t)(T * K + s * T + t) * H + row];
        for (int k = 0; k < K; ++k)
            m = fmaf(f.wts[t * K + k], f.ystage[(size_t)(t * K + k) * H + row], m);
        if (f.residual) m = f.x[(size_t)t * H + row] + m;
        f.out[(size_t)t * H + row] = m;
    }
    if (threadIdx.x == 0) f.counters[1 + b] = 0;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_router_small(const Fwd& f, hipStream_t st)
{
    const dim3 grid(f.Epad / 64, f.S / 4), block(256);
    if (f.T <= 1) hipLaunchKernelGGL(k_router_small<1>, grid, block, 0, st, f);
    else if (f.T <= 2) hipLaunchKernelGGL(k_router_small<2>, grid, block, 0, st, f);
    else if (f.T <= 4) hipLaunchKernelGGL(k_router_small<4>, grid, block, 0, st, f);
    else if (f.T <= 8) hipLaunchKernelGGL(k_router_small<8>, grid, block, 0, st, f);
    else hipLaunchKernelGGL(k_router_small<16>, grid, block, 0, st, f);
    return hipGetLastError();
}

template <int FMT>
static void gateup_dispatch(const Fwd& f, dim3 grid, hipStream_t st)
{
    if (f.T <= 1) hipLaunchKernelGGL((k_gateup<FMT, 1, 4>), grid, dim3(256), 0, st, f);
    else if (f.T <= 2) hipLaunchKernelGGL((k_gateup<FMT, 2, 4>), grid, dim3(256), 0, st, f);
    else if (f.T <= 4) hipLaunchKernelGGL((k_gateup<FMT, 4, 4>), grid, dim3(256), 0, st, f);
    else hipLaunchKernelGGL((k_gateup<FMT, 8, 4>), grid, dim3(256), 0, st, f);
}

template <int FMT>
static void down_dispatch(const Fwd& f, dim3 grid, hipStream_t st)
{
    if (f.T <= 1) hipLaunchKernelGGL((k_down<FMT, 1, 4>), grid, dim3(256), 0, st, f);
    else if (f.T <= 2) hipLaunchKernelGGL((k_down<FMT, 2, 4>), grid, dim3(256), 0, st, f);
    else if (f.T <= 4) hipLaunchKernelGGL((k_down<FMT, 4, 4>), grid, dim3(256), 0, st, f);
    else hipLaunchKernelGGL((k_down<FMT, 8, 4>), grid, dim3(256), 0, st, f);
}

hipError_t launch_gateup_gemv(const Fwd& f, int max_groups, hipStream_t st)
{
    const dim3 grid(f.I / 64, max_groups);
    if (f.fmt == MOE_W_INT4_ROW) gateup_dispatch<MOE_W_INT4_ROW>(f, grid, st);
    else gateup_dispatch<MOE_W_INT4_AFFINE_G64>(f, grid, st);
    return hipGetLastError();
}

hipError_t launch_down_gemv(const Fwd& f, int max_groups, hipStream_t st)
{
    const dim3 grid(f.H / 64, max_groups);
    if (f.fmt == MOE_W_INT4_ROW) down_dispatch<MOE_W_INT4_ROW>(f, grid, st);
    else down_dispatch<MOE_W_INT4_AFFINE_G64>(f, grid, st);
    return hipGetLastError();
}

}  // namespace moe
