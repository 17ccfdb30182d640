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

// Per-token sum, RMSNorm factor and sums of 64-column groups; one
// wavefront per token.  H must be a multiple of 256.
template <int NG>
__global__ void __launch_bounds__(256) k_tokstats(Fwd f)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= f.T) return;
    const int H = f.H;
    const float* xt = f.x + (size_t)t * H;
    float sum = 0.f, ss = 0.f;
    if constexpr (NG > 0) {
        // grouped GEMM: the whole row as fp16 with one power-of-two scale
        // (largest magnitude in [2^13, 2^14)), in pair order, and its sum
        stage_row<NG>(xt, H, lane, f.xq + (size_t)t * (H / 8), f.xrow + t, sum, ss);
    } else {
        // expert GEMVs: fp16 spans of 64
        for (int s = 0; s < H / 64; ++s) {
            const float v = xt[s * 64 + lane];
            sum += v;
            ss = fmaf(v, v, ss);
            stage_span64(v, lane, (uint16_t*)(f.xq + (size_t)t * (H / 8) + s * 8),
                         f.xsc + (size_t)t * (H / 64) + s);
        }
        sum = wsum(sum);
        ss = wsum(ss);
    }
    if (lane == 0) {
        f.tok[t].xsum = sum;
        f.tok[t].rscale = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
    }
}

// Router logits for many tokens on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products, fp32 accumulation).  Workgroup =
// 32 tokens x 64 experts; its 8 wavefronts each take one eighth of the H
// inputs, with two accumulator pairs (even and odd steps) per 32-expert
// block, and the slices are summed in LDS in a fixed order.  Per step of 8
// inputs a lane loads one float4 of x (4 consecutive inputs of its token)
// and one float4 of the interleaved router weights per 32-expert block; the
// lanes of the lower half take inputs k..k+3, the upper half k+4..k+7, so
// MFMA step j pairs inputs k+j and k+4+j in both operands.
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(512) k_router_mfma(Fwd f)
{
    __shared__ float red[8][2 * 16 * 64];  // [wave][block][reg][lane]
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = f.H, T = f.T;
    const int t0 = blockIdx.x * 32, eb = blockIdx.y;
    const int h = lane >> 5, m = lane & 31;
    const int row = t0 + m;
    const float4* xr = row < T ? (const float4*)(f.x + (size_t)row * H) : nullptr;
    const float4* wb = (const float4*)f.wr + (size_t)eb * (H / 4) * 64;
    const int KW = H / 8;  // inputs per wavefront (H is a multiple of 256)
    f32x16 acc[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[b][0] = acc[b][1] = (f32x16){};
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 2
    for (int k = w * KW; k < (w + 1) * KW; k += 8) {
        const int q = (k >> 2) + h;  // float4 index of this lane's 4 inputs
        const float4 a = xr ? xr[q] : z;
        const float4 b0 = wb[(size_t)q * 64 + m];
        const float4 b1 = wb[(size_t)q * 64 + 32 + m];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b0.x, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b1.x, acc[1][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b0.y, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b1.y, acc[1][1], 0, 0, 0);
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b0.z, acc[0][0], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b1.z, acc[1][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b0.w, acc[0][1], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b1.w, acc[1][1], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) red[w][(b * 16 + j) * 64 + lane] = acc[b][0][j] + acc[b][1][j];
    __syncthreads();
    // output (token, expert) of entry (block b, reg j, lane l):
    // token (j/4)*8 + (l/32)*4 + j%4, expert b*32 + l%32
    for (int i = threadIdx.x; i < 2 * 16 * 64; i += 512) {
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) v += red[s][i];
        const int b = i >> 10, j = (i >> 6) & 15, l = i & 63;
        const int t = t0 + (j >> 2) * 8 + (l >> 5) * 4 + (j & 3);
        if (t < T) f.logits[(size_t)t * f.Epad + eb * 64 + b * 32 + (l & 31)] = v;
    }
}

__global__ void __launch_bounds__(256) k_topk(Fwd f)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= f.T) return;
    const int E = f.E, K = f.K, Epad = f.Epad;
    const float rs = f.tok[t].rscale;
    float c[4], sg[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int e = lane + 64 * m;
        c[m] = -INFINITY;
        sg[m] = 0.f;
        if (e < E) {
            const float l = f.logits[(size_t)t * Epad + e] * rs;
            sg[m] = 1.0f / (1.0f + expf(-l));
            c[m] = sg[m] + f.bias[e];
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
// 1024 threads).  Within a 1024-assignment chunk, each wavefront finds the
// lanes holding the same expert id with 8 ballots over the id's bits; a
// per-expert running prefix over wavefronts and chunks keeps the order of
// assignment indices.  If `groups` is set, also builds the forward's expert
// groups (shared experts first, then active experts ascending) and flags
// selected experts without a slot.
__global__ void __launch_bounds__(1024) k_bucket(const int32_t* __restrict__ ids, int n, int E,
                                                 int32_t* cnt, int32_t* off, int32_t* perm,
                                                 int32_t* active, int32_t* n_active, Fwd f,
                                                 int build_groups)
{
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_run[256];
    __shared__ int s_nact;
    __shared__ int wcnt[16][256];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid < 256) {
        s_cnt[tid] = 0;
        s_run[tid] = 0;
    }
    __syncthreads();
    for (int a = tid; a < n; a += 1024) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
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
    for (int base = 0; base < n; base += 1024) {
        for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        const int a = base + tid;
        int e = a < n ? ids[a] : -1;
        const bool valid = e >= 0 && e < E;
        if (!valid) e = 0;
        unsigned long long same = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (e >> bit) & 1;
            const unsigned long long bb = __ballot(on);
            same &= on ? bb : ~bb;
        }
        const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int rank = __popcll(same & below);
        if (valid && rank == 0) wcnt[w][e] = __popcll(same);
        __syncthreads();
        if (tid < 256) {
            int run = s_run[tid];
            for (int v = 0; v < 16; ++v) {
                const int c = wcnt[v][tid];
                wcnt[v][tid] = run;
                run += c;
            }
            s_run[tid] = run;
        }
        __syncthreads();
        if (valid) perm[s_off[e] + wcnt[w][e] + rank] = a;
        __syncthreads();
    }
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
        if (slot < 0) {
            atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
            const int code = f.layer * E + tid;
            atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
        }
    }
    if (tid < f.n_shared) {
        Group g;
        g.base = f.shared + (size_t)tid * f.slot_bytes;
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

hipError_t launch_router_large(const Fwd& f, hipStream_t st, int stage)
{
    switch (stage) {
    case 0: {
        const dim3 grid((f.T + 3) / 4), block(256);
        if (!f.row_staging) return launch_k(k_tokstats<0>, grid, block, 0, st, f);
        const int ng = (f.H + 511) / 512;  // 8-value groups per lane (H <= 8192 here)
        if (ng <= 1) return launch_k(k_tokstats<1>, grid, block, 0, st, f);
        if (ng <= 2) return launch_k(k_tokstats<2>, grid, block, 0, st, f);
        if (ng <= 4) return launch_k(k_tokstats<4>, grid, block, 0, st, f);
        if (ng <= 8) return launch_k(k_tokstats<8>, grid, block, 0, st, f);
        if (ng <= 12) return launch_k(k_tokstats<12>, grid, block, 0, st, f);
        return launch_k(k_tokstats<16>, grid, block, 0, st, f);
    }
    case 1:
        return launch_k(k_router_mfma, dim3((f.T + 31) / 32, f.Epad / 64), dim3(512), 0, st, f);
    case 2: return launch_k(k_topk, dim3((f.T + 3) / 4), dim3(256), 0, st, f);
    default:
        return launch_k(k_bucket, dim3(1), dim3(1024), 0, st, (const int32_t*)f.ids, f.T * f.K,
                        f.E, f.cnt, f.off, f.perm, f.active, f.n_active, f, 1);
    }
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
