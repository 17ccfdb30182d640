// k_small.hip -- the decode-size router (few tokens): split-K router GEMV
// with the token statistics, then (in the last workgroup to finish) sigmoid,
// correction bias, wavefront top-k, renormalised weights and the
// token->expert bucketing that feeds the expert GEMVs.
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
// Roofline: HBM-bound (the router weights, 6.3 MB for the GLM shape) plus the
// latency of the serial tail (one workgroup).
#include "k_common.h"

namespace moe {

__device__ __forceinline__ uint32_t ord_float(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Router tail (one workgroup, one thread per expert): token statistics,
// sigmoid, bias, top-K per token, weights, bucketing into expert groups,
// slot resolution.  Runs after the last router partial arrives (T <= 16).
// Selection: the score key of expert e is (score, then lower id) packed in
// 64 bits; its rank is the number of keys above it, computed by every
// expert in parallel from LDS broadcasts, and experts of rank < K are the
// choice in rank order -- the same set and order as K strict greater-than
// scans.
// ---------------------------------------------------------------------------

template <int NT>
__device__ void router_tail(const Fwd& f)
{
    __shared__ unsigned long long s_key[NT][256];
    __shared__ float s_sig[NT][256];
    __shared__ float s_rs[NT];
    __shared__ int s_ids[NT * 8];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_nact;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nthr = blockDim.x;
    const int T = f.T, H = f.H, E = f.E, K = f.K, Epad = f.Epad;
    // independent loads first: bias and slot of this thread's expert
    float bias_e = 0.f;
    int slot_e = -1;
    if (tid < E) {
        bias_e = f.bias[tid];
        slot_e = f.tbl[tid];
    }
    // 1. token statistics: fixed-order sums of the per-slice partials
    if (tid < T) {
        float a[32], c[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            a[i] = i < f.S ? ld_agent(&f.tpart[((size_t)i * T + tid) * 2 + 0]) : 0.f;
            c[i] = i < f.S ? ld_agent(&f.tpart[((size_t)i * T + tid) * 2 + 1]) : 0.f;
        }
        float sum = 0.f, ss = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            sum += a[i];
            ss += c[i];
        }
        const float rs = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
        f.tok[tid].xsum = sum;
        f.tok[tid].rscale = rs;
        s_rs[tid] = rs;
    }
    for (int e = tid; e < 256; e += nthr) s_cnt[e] = 0;
    __syncthreads();

    // 2. logits (fixed-order sum of the K-slice partials), sigmoid, score key
    if (tid < 256) {
        for (int t = 0; t < T; ++t) {
            unsigned long long key = 0ull;  // padding experts: below every real key
            float sig = 0.f;
            if (tid < E) {
                float a[32];
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    a[i] = i < f.S ? ld_agent(&f.part[((size_t)i * T + t) * Epad + tid]) : 0.f;
                float l = 0.f;
#pragma unroll
                for (int i = 0; i < 32; ++i) l += a[i];
                l *= s_rs[t];
                sig = 1.0f / (1.0f + expf(-l));
                const float c = sig + bias_e;
                key = ((unsigned long long)ord_float(c) << 32) | (uint32_t)(0xFFFFu - tid);
            }
            s_key[t][tid] = key;
            s_sig[t][tid] = sig;
        }
    }
    __syncthreads();

    // 3. ranks: experts with rank < K are chosen, in rank order
    if (tid < E) {
        for (int t = 0; t < T; ++t) {
            const unsigned long long mine = s_key[t][tid];
            int rank = 0;
            for (int e = 0; e < Epad; e += 2) {
                const ulonglong2 kk = *(const ulonglong2*)&s_key[t][e];
                rank += (kk.x > mine) + (kk.y > mine);
            }
            if (rank < K) s_ids[t * K + rank] = tid;
        }
    }
    __syncthreads();
    // weights: renormalised over the chosen experts, summed in rank order
    if (tid < T * K) {
        const int t = tid / K;
        float ssum = 0.f;
        for (int k = 0; k < K; ++k) ssum += s_sig[t][s_ids[t * K + k]];
        const float sg = s_sig[t][s_ids[tid]];
        f.ids[tid] = s_ids[tid];
        f.wts[tid] = f.norm_topk ? f.routed_scale * (sg / (ssum + 1e-20f)) : f.routed_scale * sg;
    }

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
            Group g;
            g.base = slot_e >= 0 ? f.pool + (size_t)slot_e * f.slot_bytes : nullptr;
            g.cnt = s_cnt[tid];
            g.off = s_off[tid];
            g.kind = 0;
            g.expert = tid;
            f.groups[f.n_shared + idx] = g;
            if (slot_e < 0) {
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
// Workgroup (b, q) = expert block b (64 experts, one per lane) and RW
// consecutive K-slices of 64 input columns (one per wavefront, 16 float4
// chunks, all loads in flight at once), reduced in LDS in a fixed order.
// Wavefronts of expert block 0 also form the token sums of their 64
// columns (a group of the affine format) and the sums of squares.
// Partials go to f.part / f.tpart (one per workgroup row q); the last
// workgroup to arrive runs router_tail.
// ---------------------------------------------------------------------------

template <int NT>
__global__ void __launch_bounds__(512) k_router_small(Fwd f, const float* __restrict__ X)
{
    __shared__ float red[8][NT][64];
    __shared__ float sred[8][NT][2];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int RW = blockDim.x >> 6;
    const int b = blockIdx.x, s = blockIdx.y * RW + w;
    const int H = f.H, T = f.T, CH = H / 4;
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc((const float4*)f.wr + ((size_t)b * CH + (size_t)s * 16) * 64, 16 * 1024);
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const uint4 q = bload16(rw, (uint32_t)lane * 16 + (u & 3) * 1024, (u >> 2) * 4096);
        v[u] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                           __uint_as_float(q.w));
    }
    if (b == 0) {
        // token sums and sums of squares of this 64-column span; the span
        // staged as fp16 for the expert GEMVs
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < T) {
                const float xv = X[(size_t)j * H + s * 64 + lane];
                const float gs = wave_sum(xv), ss = wave_sum(xv * xv);
                stage_span64(xv, lane, (uint16_t*)(f.xq + (size_t)j * (H / 8) + s * 8),
                             f.xsc + (size_t)j * (H / 64) + s);
                if (lane == 0) {
                    sred[w][j][0] = gs;
                    sred[w][j][1] = ss;
                }
            }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        float acc = 0.f;
        if (j < T) {
            cf32* xs = as_const(X + (size_t)j * H + s * 64);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                acc = fmaf(v[u].x, xs[4 * u + 0], acc);
                acc = fmaf(v[u].y, xs[4 * u + 1], acc);
                acc = fmaf(v[u].z, xs[4 * u + 2], acc);
                acc = fmaf(v[u].w, xs[4 * u + 3], acc);
            }
        }
        red[w][j][lane] = acc;
    }
    __syncthreads();
    for (int j = w; j < T; j += RW) {
        float acc = 0.f;
        for (int v2 = 0; v2 < RW; ++v2) acc += red[v2][j][lane];
        st_agent(&f.part[((size_t)blockIdx.y * T + j) * f.Epad + b * 64 + lane], acc);
    }
    if (b == 0 && w == 0 && lane < T) {
        float gs = 0.f, ss = 0.f;
        for (int v2 = 0; v2 < RW; ++v2) {
            gs += sred[v2][lane][0];
            ss += sred[v2][lane][1];
        }
        st_agent(&f.tpart[((size_t)blockIdx.y * T + lane) * 2 + 0], gs);
        st_agent(&f.tpart[((size_t)blockIdx.y * T + lane) * 2 + 1], ss);
    }

    if (!arrive_block(&f.counters[0], gridDim.x * gridDim.y)) return;
    router_tail<NT>(f);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_router_small(const Fwd& f, hipStream_t st)
{
    const int slices = f.H / 64, rw = slices % 8 == 0 ? 8 : 4;
    const dim3 grid(f.Epad / 64, slices / rw), block(rw * 64);
    if (f.T <= 1) hipLaunchKernelGGL(k_router_small<1>, grid, block, 0, st, f, f.x);
    else if (f.T <= 2) hipLaunchKernelGGL(k_router_small<2>, grid, block, 0, st, f, f.x);
    else if (f.T <= 4) hipLaunchKernelGGL(k_router_small<4>, grid, block, 0, st, f, f.x);
    else if (f.T <= 8) hipLaunchKernelGGL(k_router_small<8>, grid, block, 0, st, f, f.x);
    else hipLaunchKernelGGL(k_router_small<16>, grid, block, 0, st, f, f.x);
    return hipGetLastError();
}

}  // namespace moe
