// k_large.hip -- router and bucketing for large token counts (prefill):
// per-token statistics, an fp32 router GEMM, one-wavefront-per-token top-K,
// and a single-workgroup stable counting sort of the T*K assignments.
//
// Cited by page title and section: "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型"
// (reader.mx) §11 (sigmoid + bias picks, plain sigmoid weighs, strict
// greater-than scan so equal scores go to the lower id; the batch expert
// union that reads each expert once); Edge0 write-up §七 (renormalised
// weights with the 1e-20 term); "初始化与权重加载" (colibrì analysis) §1.2
// (a single expert group: n_group == 1).
#include "k_common.h"

namespace moe {

__device__ __forceinline__ float wsum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ uint32_t ordf(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The large-T router's power of two for a token's x: 2^k with sqrt(ss) 2^k
// in [2^11, 2^12), so every scaled |x| stays below 2^12 (1 when ss is 0 or
// not finite).
__device__ __forceinline__ float router_xscale(float ss)
{
    const float u = sqrtf(ss);
    if (!(u > 0.f && u <= 3.402823466e38f)) return 1.f;
    int ex = 0;
    (void)frexpf(u, &ex);  // u in [2^(ex-1), 2^ex)
    int k = 12 - ex;
    k = k > 100 ? 100 : k < -100 ? -100 : k;
    return ldexpf(1.f, k);
}

// Per-token sum and RMSNorm factor, and x staged for the grouped GEMM: the
// whole row as fp16 with one power-of-two scale (largest magnitude in
// [2^13, 2^14)), in pair order, and its sum; one wavefront per token.  H
// must be a multiple of 256.
template <int NG>
__global__ void __launch_bounds__(256) k_tokstats(Fwd f)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= f.T) return;
    const int H = f.H;
    const float* xt = f.x + (size_t)t * H;
    float sum = 0.f, ss = 0.f;
    stage_row<NG>(xt, H, lane, f.xq + (size_t)t * (H / 8), f.xrow + t, sum, ss);
    if (lane == 0) {
        f.tok[t].xsum = sum;
        f.tok[t].rscale = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
        f.tok[t].xscale = router_xscale(ss);
        flag_range(f, ss);
    }
}

// Per-token sum and RMSNorm factor, and x staged for the expert GEMVs as
// fp16 spans of 64 (each with its own power-of-two scale), by a 256-thread
// workgroup: wavefront w takes spans w NS .. (w + 1) NS - 1 (NS = H / 256)
// with eight loads in flight at a time, the four wavefronts' sums added in
// wavefront order.
__device__ void stage_token_spans(const Fwd& f, int t)
{
    __shared__ float s_ts[4][2];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int H = f.H, NS = H / 256;
    const float* xt = f.x + (size_t)t * H;
    float sum = 0.f, ss = 0.f;
    for (int s0 = 0; s0 < NS; s0 += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xt[(size_t)(w * NS + min(s0 + i, NS - 1)) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s0 + i < NS) {
                const int s = w * NS + s0 + i;
                sum += v[i];
                ss = fmaf(v[i], v[i], ss);
                stage_span64(v[i], lane, (uint16_t*)(f.xq + (size_t)t * (H / 8) + s * 8),
                             f.xsc + (size_t)t * (H / 64) + s);
            }
    }
    sum = wsum(sum);
    ss = wsum(ss);
    if (lane == 0) {
        s_ts[w][0] = sum;
        s_ts[w][1] = ss;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        sum = (s_ts[0][0] + s_ts[1][0]) + (s_ts[2][0] + s_ts[3][0]);
        ss = (s_ts[0][1] + s_ts[1][1]) + (s_ts[2][1] + s_ts[3][1]);
        f.tok[t].xsum = sum;
        f.tok[t].rscale = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
        f.tok[t].xscale = router_xscale(ss);
        flag_range(f, ss);
    }
}

// one workgroup per token
__global__ void __launch_bounds__(256) k_tokspans(Fwd f) { stage_token_spans(f, blockIdx.x); }

// Router logits for many tokens on the fp16 matrix cores.  Each fp32
// operand v is carried as two fp16 parts, hi = fp16(v) and lo = fp16(v - hi)
// (22 significant bits together), after an exact power-of-two scale: x per
// token (its statistics' xscale), the weights per expert (the split copy
// made when the router is set).  A 32 x 32 x 16 step takes three products
// into one fp32 accumulator, hi.hi, hi.lo and lo.hi (lo.lo, about 2^-22 of
// the product, is left out); the partial logit is the sum times both
// inverse scales.
// Workgroup = 128 tokens x every expert x one of rslices slices of the H
// inputs.  Workgroup p (on XCD p mod 8) takes slice p mod rslices, so with
// 8 or more slices the workgroups of an XCD read only their own slices'
// weights, which stay in that XCD's L2.  x goes through LDS already split
// (double-buffered chunks of 32 inputs, token-minor so the operand reads are
// conflict-free); wavefront w takes experts 32w..32w+31 for the four
// 32-token blocks, its weight operands straight from the split copy.  x and
// the weights are fetched four chunks ahead.  Each slice's partial logits go
// to a plane of their own; k_topk sums the planes in slice order.
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int RTILE = 128;  // tokens per workgroup of the large-T router
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

template <int NW>
__global__ void __launch_bounds__(64 * NW) k_router_h16(Fwd f)
{
    constexpr int TT = RTILE, TB = TT / 32;  // tokens per workgroup, 32-token blocks
    // [buffer][step of 16 inputs][input half][token] of 4 fp16 pairs: hi, lo
    __shared__ uint4 xh[2][2][2][TT], xl[2][2][2][TT];
    __shared__ float s_xs[TT];
    constexpr int NTHR = 64 * NW, NX = TT * 8;  // x float4 per chunk
    constexpr int NR = (NX + NTHR - 1) / NTHR;  // ... per thread
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = f.H, T = f.T, Epad = f.Epad, R = f.rslices;
    const int p = blockIdx.y * gridDim.x + blockIdx.x;
    const int slice = p % R, t0 = (p / R) * TT;
    const int h = lane >> 5, m = lane & 31;
    const int KC = H / R;  // inputs per slice, a multiple of 32
    const int kb = slice * KC, NCH = KC / 32;
    // the lane's (hi, lo) operand pair of step s: wb[s * 128]
    const uint4* wb = f.wr16 + ((size_t)w * (H / 16) + kb / 16) * 128 + lane * 2;
    for (int i = tid; i < TT; i += NTHR) s_xs[i] = t0 + i < T ? f.tok[t0 + i].xscale : 1.f;
    // x loader: pair i = tid + r NTHR -> token i >> 3, float4 i & 7 of the
    // chunk; token and pair indices clamped (a padded token's row is read
    // but its logits are not stored), so the loads carry no branch
    const float4* xr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int i = min(tid + r * NTHR, NX - 1);
        xr[r] = (const float4*)(f.x + (size_t)min(t0 + (i >> 3), T - 1) * H + kb) + (i & 7);
    }
    __syncthreads();
    auto load_x = [&](int ch, float4 (&v)[NR]) {
#pragma unroll
        for (int r = 0; r < NR; ++r) v[r] = xr[r][ch * 8];
    };
    // inputs 4j..4j+3 of the chunk: step j >> 2, half (j >> 1) & 1, pairs
    // 2 (j & 1) and 2 (j & 1) + 1 of that half's 8 inputs
    auto store_x = [&](int buf, const float4 (&v)[NR]) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int i = tid + r * NTHR;
            if (NR * NTHR == NX || i < NX) {
                const int tok = i >> 3, j = i & 7;
                const float sc = s_xs[tok];
                const float a0 = v[r].x * sc, a1 = v[r].y * sc, a2 = v[r].z * sc, a3 = v[r].w * sc;
                const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1, h2 = (_Float16)a2,
                               h3 = (_Float16)a3;
                const _Float16 l0 = (_Float16)(a0 - (float)h0), l1 = (_Float16)(a1 - (float)h1),
                               l2 = (_Float16)(a2 - (float)h2), l3 = (_Float16)(a3 - (float)h3);
                uint2* dh = (uint2*)&xh[buf][j >> 2][(j >> 1) & 1][tok] + (j & 1);
                uint2* dl = (uint2*)&xl[buf][j >> 2][(j >> 1) & 1][tok] + (j & 1);
                *dh = make_uint2(pack_h2(h0, h1), pack_h2(h2, h3));
                *dl = make_uint2(pack_h2(l0, l1), pack_h2(l2, l3));
            }
        }
    };
    f32x16 acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = (f32x16){};
    // x and weights of chunks ch .. ch + RP - 1 in flight, in slot ch % RP
    // (chunk indices clamped past the end, so the loads carry no branch)
    constexpr int RP = 4;
    float4 xv[RP][NR];
    uint4 bw[RP][2][2];  // [slot][step][hi, lo]
#pragma unroll
    for (int k = 0; k < RP; ++k) {
        const int c = min(k, NCH - 1);
        load_x(c, xv[k]);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            bw[k][st][0] = wb[(2 * c + st) * 128];
            bw[k][st][1] = wb[(2 * c + st) * 128 + 1];
        }
    }
    store_x(0, xv[0]);
    load_x(min(RP, NCH - 1), xv[0]);
    __syncthreads();
#pragma unroll 1
    for (int ch0 = 0; ch0 < NCH; ch0 += RP) {
#pragma unroll
        for (int k = 0; k < RP; ++k) {
            const int ch = ch0 + k;
            const int k1 = (k + 1) % RP;
            // chunk ch + 1 into the other buffer (free since the last barrier),
            // then its slot refetches chunk ch + 1 + RP
            if (ch + 1 < NCH) store_x((ch + 1) & 1, xv[k1]);
            load_x(min(ch + 1 + RP, NCH - 1), xv[k1]);
            if (ch < NCH) {
                const int buf = ch & 1;
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const h16x8 bh = __builtin_bit_cast(h16x8, bw[k][st][0]);
                    const h16x8 bl = __builtin_bit_cast(h16x8, bw[k][st][1]);
                    // hi.hi, then hi.lo, then lo.hi, each over the token
                    // blocks (no accumulator is used twice in a row)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const h16x8 ah = __builtin_bit_cast(h16x8, xh[buf][st][h][32 * tb + m]);
                        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[tb], 0, 0, 0);
                    }
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const h16x8 ah = __builtin_bit_cast(h16x8, xh[buf][st][h][32 * tb + m]);
                        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc[tb], 0, 0, 0);
                    }
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const h16x8 al = __builtin_bit_cast(h16x8, xl[buf][st][h][32 * tb + m]);
                        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc[tb], 0, 0, 0);
                    }
                }
            }
            const int cn = min(ch + RP, NCH - 1);
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bw[k][st][0] = wb[(2 * cn + st) * 128];
                bw[k][st][1] = wb[(2 * cn + st) * 128 + 1];
            }
            __syncthreads();
        }
    }
    // entry (reg j, lane l) of a 32 x 32 tile: token (j/4)*8 + (l/32)*4 + j%4,
    // expert l%32
    const int e = 32 * w + m;
    const float winv = f.wr16s[e].y;
    float* plane = f.logits + (size_t)slice * T * Epad;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int tl = 32 * tb + (j >> 2) * 8 + h * 4 + (j & 3);
            const int t = t0 + tl;
            if (t < T) plane[(size_t)t * Epad + e] = acc[tb][j] * (winv / s_xs[tl]);
        }
}

// Router logits for a few tokens (2 .. 16): workgroup e holds expert e's
// row of the row-major router copy in registers (thread l: float4 columns
// l, l + 256, ...) and takes the tokens TT at a time, every token's loads in
// flight together; the 4 wavefronts' sums meet in LDS in wavefront order
// and go to logit plane 0.  Workgroup t < T also forms token t's statistics
// (sum, RMSNorm factor, range check) and stages its x for the expert
// kernels: the whole row with one power-of-two scale (ROWS, the
// matrix-core path) or in spans of 64.
constexpr int RT_TT = 4;

template <int Q, int NG, bool ROWS>
__global__ void __launch_bounds__(256) k_router_t(Fwd f)
{
    __shared__ float s_red[RT_TT][4];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, e = blockIdx.x;
    const int H = f.H, H4 = H / 4, T = f.T;
    if (e < f.E) {
        const float4* wr = (const float4*)(f.wr_rows + (size_t)e * H);
        float4 wv[Q];
#pragma unroll
        for (int k = 0; k < Q; ++k) {
            const int c = tid + 256 * k;
            wv[k] = c < H4 ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int t0 = 0; t0 < T; t0 += RT_TT) {
            float acc[RT_TT];
#pragma unroll
            for (int j = 0; j < RT_TT; ++j) {
                const float4* xr = (const float4*)(f.x + (size_t)min(t0 + j, T - 1) * H);
                float4 xv[Q];
#pragma unroll
                for (int k = 0; k < Q; ++k) xv[k] = xr[min(tid + 256 * k, H4 - 1)];
                float a = 0.f;
#pragma unroll
                for (int k = 0; k < Q; ++k)
                    if (tid + 256 * k < H4) {
                        a = fmaf(wv[k].x, xv[k].x, a);
                        a = fmaf(wv[k].y, xv[k].y, a);
                        a = fmaf(wv[k].z, xv[k].z, a);
                        a = fmaf(wv[k].w, xv[k].w, a);
                    }
                acc[j] = wave_sum(a);
            }
            if (lane == 0)
#pragma unroll
                for (int j = 0; j < RT_TT; ++j) s_red[j][w] = acc[j];
            __syncthreads();
            if (tid < RT_TT && t0 + tid < T)
                f.logits[(size_t)(t0 + tid) * f.Epad + e] =
                    (s_red[tid][0] + s_red[tid][1]) + (s_red[tid][2] + s_red[tid][3]);
            __syncthreads();
        }
    }
    if (e < T) {
        if (ROWS) {
            if (w == 0) {
                float sum, ss;
                stage_row<NG>(f.x + (size_t)e * H, H, lane, f.xq + (size_t)e * (H / 8), f.xrow + e,
                              sum, ss);
                if (lane == 0) {
                    f.tok[e].xsum = sum;
                    f.tok[e].rscale = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
                    flag_range(f, ss);
                }
            }
        } else {
            stage_token_spans(f, e);
        }
    }
}

__global__ void __launch_bounds__(256) k_topk(Fwd f)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= f.T) return;
    const int E = f.E, K = f.K, Epad = f.Epad;
    const float rs = f.tok[t].rscale;
    // the router's slice partials of the lane's 4 experts, summed in slice
    // order, 8 slices (32 loads) in flight at a time (plane indices clamped,
    // the clamped ones then zeroed); expert slots past E (padding of Epad)
    // are read but not used
    float lg[4] = {0.f, 0.f, 0.f, 0.f};
    const int R = f.rslices;
    for (int s0 = 0; s0 < R; s0 += 8) {
        float v[4][8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = min(lane + 64 * m, Epad - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[m][i] = f.logits[((size_t)min(s0 + i, R - 1) * f.T + t) * Epad + e];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 8; ++i) lg[m] += s0 + i < R ? v[m][i] : 0.f;
    }
    float c[4], sg[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        c[m] = -INFINITY;
        sg[m] = 0.f;
        if (e < E) {
            const float l = lg[m] * rs;
            if (f.scoring == MOE_SCORE_SOFTMAX) {
                sg[m] = l;  // the probability follows below
            } else {
                sg[m] = 1.0f / (1.0f + expf(-l));
                c[m] = sg[m] + f.bias[e];
            }
        }
    }
    // softmax scoring: probabilities over all experts (shifted by the largest
    // logit); they weigh and select, no bias
    if (f.scoring == MOE_SCORE_SOFTMAX) {
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (lane + 64 * m < E) mx = fmaxf(mx, sg[m]);
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sg[m] = lane + 64 * m < E ? expf(sg[m] - mx) : 0.f;
            z += sg[m];
        }
        z = wsum(z);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            if (lane + 64 * m < E) {
                sg[m] = sg[m] / z;
                c[m] = sg[m];
            }
    }
    // group-limited selection: a group's score is the fp32 sum of its two
    // largest c; a group is kept when fewer than topk_group groups rank above
    // it (greater score, or equal score and lower index: the strictly-greater
    // scan's order); the other groups' experts are excluded
    if (f.n_group > 1) {
        __shared__ float s_c[4][256];
        __shared__ float s_gs[4][64];
        const int wv = threadIdx.x >> 6, NG = f.n_group, GS = E / NG;
#pragma unroll
        for (int m = 0; m < 4; ++m) s_c[wv][lane + 64 * m] = c[m];
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wavefront's writes are visible to it
        __builtin_amdgcn_wave_barrier();
        if (lane < NG) {
            float a = -INFINITY, b2 = -INFINITY;
#pragma unroll 8
            for (int e = lane * GS; e < (lane + 1) * GS; ++e) {
                const float v = s_c[wv][e];
                b2 = fmaxf(b2, fminf(a, v));
                a = fmaxf(a, v);
            }
            s_gs[wv][lane] = a + b2;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __builtin_amdgcn_wave_barrier();
        uint64_t kept = 0ull;
        if (lane < NG) {
            const float mine = s_gs[wv][lane];
            int rank = 0;
            for (int h = 0; h < NG; ++h) {
                const float o = s_gs[wv][h];
                rank += (o > mine) || (o == mine && h < lane);
            }
            kept = rank < f.topk_group;
        }
        kept = __ballot(kept != 0ull);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = lane + 64 * m;
            if (e < E && !((kept >> (e / GS)) & 1ull)) c[m] = -INFINITY;
        }
    }
    uint32_t taken = 0;
    float ssum = 0.f, mysig = 0.f;
    int myid = 0;
    for (int kk = 0; kk < K; ++kk) {
        unsigned long long best = 0ull;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = lane + 64 * m;
            if (e < Epad && !(taken & (1u << m))) {
                const unsigned long long key =
                    ((unsigned long long)ordf(c[m]) << 32) | (uint32_t)(0xFFFFu - e);
                best = key > best ? key : best;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const unsigned long long other = __shfl_xor(best, o);
            best = other > best ? other : best;
        }
        const int e = 0xFFFF - (int)(best & 0xFFFFu);
        const int owner = e & 63, m = e >> 6;
        float s_e = 0.f;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
            if (mm == m) s_e = sg[mm];
        s_e = __shfl(s_e, owner);
        if (lane == owner) taken |= 1u << m;
        ssum += s_e;
        if (lane == kk) {
            myid = e;
            mysig = s_e;
        }
    }
    if (lane < K) {
        const float wv = f.norm_topk ? f.routed_scale * (mysig / (ssum + 1e-20f))
                                     : f.routed_scale * mysig;
        f.ids[(size_t)t * K + lane] = myid;
        f.wts[(size_t)t * K + lane] = wv;
    }
}

// Stable counting sort of the T*K assignments by expert (one workgroup of
// 1024 threads).  Wavefront w owns the w-th of 16 contiguous segments of the
// assignments and walks it 64 at a time: the lanes holding the same expert
// id are found with 8 ballots over the id's bits, and the lowest of them
// keeps the wavefront's running count of that expert in its own LDS row.
// Pass 1 counts (LDS atomics); a prefix over the 16 wavefronts per expert and
// a scan over the experts give every (wavefront, expert) its first position;
// pass 2 repeats the walk and writes each assignment at its expert's offset
// plus the number of earlier assignments of that expert, so the order of
// assignment indices is kept.  If `groups` is set, also builds the forward's
// expert groups (shared experts first, then active experts ascending) and
// flags selected experts without a slot.
__device__ __forceinline__ unsigned long long same_expert(int e, bool valid)
{
    unsigned long long same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool on = (e >> bit) & 1;
        const unsigned long long bb = __ballot(on);
        same &= on ? bb : ~bb;
    }
    return same;
}

__global__ void __launch_bounds__(1024) k_bucket(const int32_t* __restrict__ ids, int n, int E,
                                                 int32_t* cnt, int32_t* off, int32_t* perm,
                                                 int32_t* active, int32_t* n_active, Fwd f,
                                                 int build_groups)
{
    constexpr int BU = 8;  // rounds whose ids are loaded together
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_nact;
    __shared__ int wcnt[16][256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    const int seg = ((n + 15) / 16 + 63) / 64 * 64;  // assignments per wavefront
    const int a0 = w * seg, a1 = min(n, a0 + seg);
    const int rounds = a1 > a0 ? (a1 - a0 + 63) / 64 : 0;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int pass = 0; pass < 2; ++pass) {
        for (int r0 = 0; r0 < rounds; r0 += BU) {
            int ev[BU];
#pragma unroll
            for (int u = 0; u < BU; ++u) {
                const int a = a0 + (r0 + u) * 64 + lane;
                ev[u] = a < a1 ? ids[a] : -1;
            }
#pragma unroll
            for (int u = 0; u < BU; ++u) {
                if (r0 + u >= rounds) break;
                const int a = a0 + (r0 + u) * 64 + lane;
                int e = ev[u];
                const bool valid = e >= 0 && e < E;
                if (pass == 0) {  // counts only: order does not matter
                    if (valid) atomicAdd(&wcnt[w][e], 1);
                    continue;
                }
                if (!valid) e = 0;
                const unsigned long long same = same_expert(e, valid);
                const int rank = __popcll(same & below);
                // every lane reads the running count before its lowest lane
                // (rank 0) advances it
                const int before = wcnt[w][e];
                if (valid) perm[s_off[e] + before + rank] = a;
                if (valid && rank == 0) wcnt[w][e] = before + __popcll(same);
            }
        }
        if (pass == 1) break;
        __syncthreads();
        // per expert: the wavefronts' first positions and the total
        if (tid < 256) {
            int run = 0;
            for (int v = 0; v < 16; ++v) {
                const int c = wcnt[v][tid];
                wcnt[v][tid] = run;
                run += c;
            }
            s_cnt[tid] = run;
        }
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
            int ic = sc, ia = sa;
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
    }
    __syncthreads();
    if (tid < E) {
        cnt[tid] = s_cnt[tid];
        off[tid] = s_off[tid];
        if (s_act[tid] >= 0) active[s_act[tid]] = tid;
    }
    if (tid == 0) {
        off[E] = s_off[E];
        n_active[0] = s_nact;
    }
    if (!build_groups) return;
    if (tid < E && s_act[tid] >= 0) {
        const int slot = f.tbl[tid];
        Group g;
        g.base = slot >= 0 ? f.pool + (size_t)slot * f.slot_bytes : nullptr;
        g.cnt = s_cnt[tid];
        g.off = s_off[tid];
        g.kind = 0;
        g.expert = tid;
        f.groups[f.n_shared + s_act[tid]] = g;
        if (slot == -1) {  // missing (a remote expert, -2, is skipped quietly)
            atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
            const int code = f.layer * E + tid;
            atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
        }
    }
    if (tid < f.n_shared) {
        Group g;
        g.base = f.shared + (size_t)tid * f.shared_bytes;
        g.cnt = f.T;
        g.off = tid;
        g.kind = 1;
        g.expert = -1;
        f.groups[tid] = g;
    }
    if (tid == 0) {
        f.n_groups[0] = f.n_shared + s_nact;
    }
}

// up to 16 tokens (each workgroup takes the tokens 4 at a time; beyond 16
// the matrix-core router with more H slices measured faster)
bool router_t_ok(int T, int H, const float* wr_rows)
{
    return T >= 2 && T <= 16 && wr_rows != nullptr && H <= 8192;
}

template <int Q>
static hipError_t router_t_go(const Fwd& f, hipStream_t st)
{
    const dim3 grid((unsigned)std::max(f.E, f.T)), block(256);
    if (!f.row_staging) return launch_k(k_router_t<Q, 1, false>, grid, block, 0, st, f);
    const int ng = (f.H + 511) / 512;
    if (ng <= 1) return launch_k(k_router_t<Q, 1, true>, grid, block, 0, st, f);
    if (ng <= 2) return launch_k(k_router_t<Q, 2, true>, grid, block, 0, st, f);
    if (ng <= 4) return launch_k(k_router_t<Q, 4, true>, grid, block, 0, st, f);
    if (ng <= 8) return launch_k(k_router_t<Q, 8, true>, grid, block, 0, st, f);
    if (ng <= 12) return launch_k(k_router_t<Q, 12, true>, grid, block, 0, st, f);
    return launch_k(k_router_t<Q, 16, true>, grid, block, 0, st, f);
}

hipError_t launch_router_large(const Fwd& f, hipStream_t st, int stage)
{
    if (f.rslices == 1) {  // a few tokens: the row router (logits and staging), then top-K
        switch (stage) {
        case 0: {
            const int q = (f.H + 1023) / 1024;
            if (q <= 1) return router_t_go<1>(f, st);
            if (q <= 2) return router_t_go<2>(f, st);
            if (q <= 4) return router_t_go<4>(f, st);
            if (q <= 6) return router_t_go<6>(f, st);
            return router_t_go<8>(f, st);
        }
        case 1: return hipSuccess;
        default: break;
        }
    }
    switch (stage) {
    case 0: {
        const dim3 grid((f.T + 3) / 4), block(256);
        if (!f.row_staging) return launch_k(k_tokspans, dim3((unsigned)f.T), block, 0, st, f);
        const int ng = (f.H + 511) / 512;  // 8-value groups per lane (H <= 8192 here)
        if (ng <= 1) return launch_k(k_tokstats<1>, grid, block, 0, st, f);
        if (ng <= 2) return launch_k(k_tokstats<2>, grid, block, 0, st, f);
        if (ng <= 4) return launch_k(k_tokstats<4>, grid, block, 0, st, f);
        if (ng <= 8) return launch_k(k_tokstats<8>, grid, block, 0, st, f);
        if (ng <= 12) return launch_k(k_tokstats<12>, grid, block, 0, st, f);
        return launch_k(k_tokstats<16>, grid, block, 0, st, f);
    }
    case 1:
        if (f.wr16 == nullptr || f.wr16s == nullptr) return hipErrorInvalidValue;
    {
        const dim3 grid((f.T + RTILE - 1) / RTILE, (unsigned)f.rslices), block(64 * (f.Epad / 32));
        switch (f.Epad / 32) {
        case 2: return launch_k(k_router_h16<2>, grid, block, 0, st, f);
        case 4: return launch_k(k_router_h16<4>, grid, block, 0, st, f);
        case 6: return launch_k(k_router_h16<6>, grid, block, 0, st, f);
        case 8: return launch_k(k_router_h16<8>, grid, block, 0, st, f);
        default: return hipErrorInvalidValue;
        }
    }
    case 2: return launch_k(k_topk, dim3((f.T + 3) / 4), dim3(256), 0, st, f);
    default:
        return launch_k(k_bucket, dim3(1), dim3(1024), 0, st, (const int32_t*)f.ids, f.T * f.K,
                        f.E, f.cnt, f.off, f.perm, f.active, f.n_active, f, 1);
    }
}

int router_slices(int T, int H)
{
    const int tiles = (T + RTILE - 1) / RTILE;
    int s = ROUTER_SLICES;
    while (s < ROUTER_SLICES_MAX && tiles * 2 * s <= 256 && (H / 32) % (2 * s) == 0) s *= 2;
    return s;
}

// rslices * T: at most ROUTER_SLICES * T; with more slices the grid has at
// most 256 workgroups of RTILE tokens, so rslices * T <= 128 * 256.
size_t router_logit_rows(int Tmax)
{
    return std::max<size_t>((size_t)ROUTER_SLICES * Tmax,
                            std::min<size_t>((size_t)ROUTER_SLICES_MAX * Tmax, 32768));
}

hipError_t launch_bucket(const int32_t* ids, int T, int K, int E, int32_t* cnt, int32_t* off,
                         int32_t* perm, int32_t* active, int32_t* n_active, hipStream_t st)
{
    Fwd f{};
    hipLaunchKernelGGL(k_bucket, dim3(1), dim3(1024), 0, st, ids, T * K, E, cnt, off, perm, active,
                       n_active, f, 0);
    return hipGetLastError();
}

}  // namespace moe
