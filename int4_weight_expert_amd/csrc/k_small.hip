// k_small.hip -- the decode-size router (few tokens): split-K router GEMV
// with the token statistics, then (in the last workgroup to finish) sigmoid,
// correction bias, top-k by ranks, renormalised weights and the
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

// The score c of a selection key (ord_float(c) << 32 | id bits), exactly.
__device__ __forceinline__ float key_score(unsigned long long key)
{
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// ---------------------------------------------------------------------------
// Router tail (one workgroup of 256 threads, one per expert): token
// statistics, sigmoid, bias, top-K per token, weights, bucketing into expert
// groups, slot resolution.  Runs in the last router workgroup to arrive
// (T <= 8).
// Selection: the score key of expert e is (score, then lower id) packed in
// 64 bits, so keys are distinct and "greater key" is the pages' strict
// greater-than scan order.  Each wavefront ranks the keys of one block of 64
// experts among themselves; the block's keys of rank < K are candidates, and
// the candidates' ranks among all candidates are the global ranks: the
// experts of rank < K are the choice, in rank order.
// ---------------------------------------------------------------------------

constexpr int RT_THREADS = 256;

// Partial layouts (written by the router workgroups with agent-scope stores):
// one token: the logit partials of expert e, slice row i at part[e * Sp + i]
// (the tail's thread e reads its row contiguously); several tokens:
// part[(i * T + t) * Epad + e] (a block's last workgroup sums them, lanes =
// experts, into the logits at part_logits(), [t][Epad]).  Statistics (sum,
// sum of squares) of token t at tpart[t * S2p + 2 i + {0, 1}].  Sp, S2p are
// rounded up to whole 16-byte vectors.
__device__ __forceinline__ int router_sp(int T, int S) { return (T * S + 3) & ~3; }
__device__ __forceinline__ int router_s2p(int S) { return (2 * S + 3) & ~3; }
// past the largest partial region, S * 8 * Epad floats (the buffer holds
// (H / 64) * 8 * Epad = 4 S * 8 * Epad)
__device__ __forceinline__ float* part_logits(const Fwd& f) { return f.part + (size_t)f.S * 8 * f.Epad; }

// 16-byte agent-coherent (sc1) buffer load
__device__ __forceinline__ float4 bload16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 16);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                       __uint_as_float(v.w));
}

// Fixed-order sum of n (<= 64) consecutive partials starting at float index
// `at` of resource r (lane-private offset voff); all loads issued first.
__device__ __forceinline__ void load64(__amdgpu_buffer_rsrc_t r, uint32_t voff, int at, int n,
                                       float (&a)[64])
{
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const float4 v = 4 * q < n ? bload16_agent(r, voff, (uint32_t)(at + 4 * q) * 4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        a[4 * q + 0] = 4 * q + 0 < n ? v.x : 0.f;  // padding floats are never written
        a[4 * q + 1] = 4 * q + 1 < n ? v.y : 0.f;
        a[4 * q + 2] = 4 * q + 2 < n ? v.z : 0.f;
        a[4 * q + 3] = 4 * q + 3 < n ? v.w : 0.f;
    }
}

// PRE (one token): the expert's logit and the token's sum of squares come
// from the caller (which also wrote the token's statistics) instead of the
// partial buffers.
template <int NT, bool PRE = false>
__device__ void router_tail(const Fwd& f, float bias_e, int slot_e, float pre_l = 0.f,
                            float pre_ss = 0.f)
{
    __shared__ unsigned long long s_key[NT][256];
    __shared__ unsigned long long s_cand[NT][32];
    __shared__ float s_sig[NT][256];
    __shared__ float s_rs[NT];
    __shared__ int s_ids[NT * 8];
    __shared__ int s_cnt[256];
    __shared__ int s_off[257];
    __shared__ int s_act[256];
    __shared__ int s_nact;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = f.T, H = f.H, E = f.E, K = f.K, Epad = f.Epad, S = f.S;
    const int Sp = router_sp(T, S), S2p = router_s2p(S);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(f.part, (uint32_t)(Epad * Sp * 4));
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(f.tpart, (uint32_t)(T * S2p * 4));
    // 1. token statistics and logits.  T = 1: every thread sums the token's
    //    statistics itself (no barrier); otherwise thread t < T does, via LDS.
    float lsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) lsum[t] = 0.f;
    float rs0 = 1.f;
    // (the loads of a step are issued together, before any of them is used)
    if (NT == 1 && PRE) {
        lsum[0] = pre_l;
        rs0 = f.residual ? 1.0f / sqrtf(pre_ss / (float)H + f.eps) : 1.0f;
    } else if (NT == 1) {
        float a[64], st[64];
        load64(rp, (uint32_t)tid * Sp * 4, 0, S, a);  // S <= 64
        load64(rt, 0, 0, min(2 * S, 64), st);
        float sum = 0.f, ss = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            sum += st[2 * i];
            ss += st[2 * i + 1];
        }
        for (int c0 = 64; c0 < 2 * S; c0 += 64) {  // H > 8192
            load64(rt, 0, c0, 2 * S - c0, st);
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                sum += st[2 * i];
                ss += st[2 * i + 1];
            }
        }
#pragma unroll
        for (int i = 0; i < 64; ++i) lsum[0] += a[i];
        rs0 = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
        if (tid == 0) {
            f.tok[0].xsum = sum;
            f.tok[0].rscale = rs0;
            flag_range(f, ss);
        }
    } else {
        // expert tid's logits (summed per expert block by its last
        // workgroup) and, for thread t < T, token t's statistics; every
        // thread loads (indices clamped), so that no branch separates them
        const float* lg = part_logits(f);
        const int ec = min(tid, Epad - 1);
        float lv[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) lv[t] = ld_agent(&lg[(size_t)min(t, T - 1) * Epad + ec]);
        // token ts = tid / 32 (T <= 8): its 32 threads each sum every 32nd
        // slice's (sum, sum of squares), all loads of a round of 4 slices in
        // flight, then a fixed butterfly over the 32
        const int ts = tid >> 5, sub = tid & 31, tsc = min(ts, T - 1);
        const float* tp = f.tpart + (size_t)tsc * S2p;
        float sum = 0.f, ss = 0.f;
        for (int i0 = 0; i0 < S; i0 += 128) {
            float2 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = min(i0 + sub + 32 * q, S - 1);
                v[q] = make_float2(ld_agent(&tp[2 * i]), ld_agent(&tp[2 * i + 1]));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + sub + 32 * q < S) {
                    sum += v[q].x;
                    ss += v[q].y;
                }
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) {
            sum += __shfl_xor(sum, o);
            ss += __shfl_xor(ss, o);
        }
        if (sub == 0 && ts < T) {
            const float rs = f.residual ? 1.0f / sqrtf(ss / (float)H + f.eps) : 1.0f;
            f.tok[ts].xsum = sum;
            f.tok[ts].rscale = rs;
            s_rs[ts] = rs;
            flag_range(f, ss);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) lsum[t] = (t < T && tid < E) ? lv[t] : 0.f;
    }
    for (int e = tid; e < 256; e += RT_THREADS) s_cnt[e] = 0;
    for (int i = tid; i < T * 32; i += RT_THREADS) s_cand[i >> 5][i & 31] = 0ull;
    if (NT > 1) __syncthreads();

    // 2. scores and keys (keys of all 256 slots are written: padding experts
    //    get 0, below every real key).  Sigmoid: sigma weighs, sigma + bias
    //    selects.  Softmax: the probability over all experts (shifted by the
    //    token's largest logit) weighs and selects.
    float prob[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) prob[t] = 0.f;
    if (f.scoring == MOE_SCORE_SOFTMAX) {
        __shared__ float s_red[NT][RT_THREADS / 64];
        float l[NT], m[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            l[t] = -INFINITY;
            if (t < T && tid < E) l[t] = lsum[t] * (NT == 1 ? rs0 : s_rs[t]);
            const float v = wave_max(l[t]);
            if (lane == 0) s_red[t][w] = v;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            m[t] = s_red[t][0];
#pragma unroll
            for (int i = 1; i < RT_THREADS / 64; ++i) m[t] = fmaxf(m[t], s_red[t][i]);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            prob[t] = (t < T && tid < E) ? expf(l[t] - m[t]) : 0.f;
            const float v = wave_sum(prob[t]);
            if (lane == 0) s_red[t][w] = v;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float z = 0.f;
#pragma unroll
            for (int i = 0; i < RT_THREADS / 64; ++i) z += s_red[t][i];
            prob[t] = prob[t] / z;
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
        if (t < T) {
            unsigned long long key = 0ull;
            float sig = 0.f;
            if (tid < E) {
                float c;
                if (f.scoring == MOE_SCORE_SOFTMAX) {
                    sig = prob[t];
                    c = sig;
                } else {
                    const float rs = NT == 1 ? rs0 : s_rs[t];
                    sig = 1.0f / (1.0f + expf(-(lsum[t] * rs)));
                    c = sig + bias_e;
                }
                key = ((unsigned long long)ord_float(c) << 32) | (uint32_t)(0xFFFFu - tid);
            }
            s_key[t][tid] = key;
            s_sig[t][tid] = sig;
        }
    __syncthreads();

    // 2b. group-limited selection: a group's score is the fp32 sum of its two
    //     largest c; a group is kept when fewer than topk_group groups rank
    //     above it (greater score, or equal score and lower index: the
    //     strictly-greater scan's order); the other groups' keys drop to 0,
    //     below every real key
    if (f.n_group > 1) {
        __shared__ float s_gs[NT][64];
        const int NG = f.n_group, GS = E / NG;
        for (int i = tid; i < T * NG; i += RT_THREADS) {
            const int t = i / NG, g = i - t * NG;
            const unsigned long long* kb = &s_key[t][g * GS];
            float a = -INFINITY, b2 = -INFINITY;
#pragma unroll 8
            for (int e = 0; e < GS; ++e) {
                const float c = key_score(kb[e]);
                b2 = fmaxf(b2, fminf(a, c));
                a = fmaxf(a, c);
            }
            s_gs[t][g] = a + b2;
        }
        __syncthreads();
        if (tid < E) {
            const int g = tid / GS;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                if (t < T) {
                    const float mine = s_gs[t][g];
                    int rank = 0;
                    for (int h = 0; h < NG; ++h) {
                        const float o = s_gs[t][h];
                        rank += (o > mine) || (o == mine && h < g);
                    }
                    if (rank >= f.topk_group) s_key[t][tid] = 0ull;
                }
        }
        __syncthreads();
    }

    // 3a. ranks within each block of 64 experts; rank < K -> candidate (two
    //     (token, block) pairs per pass, so that their LDS reads overlap)
    const int wu = __builtin_amdgcn_readfirstlane(w);
    constexpr int PP = NT > 1 ? 2 : 1;  // one token: one pair per wavefront
    for (int pq = wu; pq < T * 4; pq += PP * (RT_THREADS / 64)) {
        const int pq2 = PP == 2 ? pq + RT_THREADS / 64 : pq;
        const int t = pq >> 2, blk = pq & 3;
        const int t2 = min(pq2, T * 4 - 1) >> 2, blk2 = min(pq2, T * 4 - 1) & 3;
        const unsigned long long* kb = &s_key[t][blk * 64];
        const unsigned long long* kb2 = &s_key[t2][blk2 * 64];
        const unsigned long long mine = kb[lane], mine2 = kb2[lane];
        int rank = 0, rank2 = 0;
#pragma unroll
        for (int e = 0; e < 64; e += 2) {
            const ulonglong2 kk = *(const ulonglong2*)&kb[e];
            rank += (kk.x > mine) + (kk.y > mine);
            if (PP == 2) {
                const ulonglong2 kk2 = *(const ulonglong2*)&kb2[e];
                rank2 += (kk2.x > mine2) + (kk2.y > mine2);
            }
        }
        if (rank < K) s_cand[t][blk * K + rank] = mine;
        if (PP == 2 && pq2 < T * 4 && rank2 < K) s_cand[t2][blk2 * K + rank2] = mine2;
    }
    __syncthreads();
    // 3b. ranks among the 4K candidates: global ranks of the top K
    for (int tc = tid; tc < T * 32; tc += RT_THREADS) {
        const int t = tc >> 5, c = tc & 31;
        const unsigned long long mine = s_cand[t][c];
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 32; j += 2) {
            const ulonglong2 kk = *(const ulonglong2*)&s_cand[t][j];
            rank += (kk.x > mine) + (kk.y > mine);
        }
        if (c < 4 * K && rank < K) s_ids[t * K + rank] = (int)(0xFFFFu - (uint32_t)(mine & 0xFFFFu));
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
    if (tid < f.n_shared) {
        Group g;
        g.base = f.shared + (size_t)tid * f.shared_bytes;
        g.cnt = T;
        g.off = tid;
        g.kind = 1;
        g.expert = -1;
        f.groups[tid] = g;
    }

    // 4. bucketing into active expert groups (ascending expert id), each
    //    group's assignments in assignment order
    int cnt_e = 0, off_e = 0, idx_e = -1;
    if (NT == 1) {
        // one token: the K chosen experts are distinct, one assignment each
        if (tid < E) {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < K) {
                    const int e = s_ids[k];
                    off_e += e < tid;
                    if (e == tid) {
                        cnt_e = 1;
                        idx_e = k;  // assignment index
                    }
                }
            if (cnt_e) {
                f.perm[off_e] = idx_e;
                idx_e = off_e;  // group index = rank of the id among the chosen
            }
        }
        if (tid == 0) {
            f.n_active[0] = K;
            f.n_groups[0] = f.n_shared + K;
            f.off[E] = K;
        }
    } else {
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
        // each assignment's place in its group (n = T K <= 64: wavefront 0,
        // the lanes holding the same id found with 8 ballots over its bits)
        if (w == 0) {
            const bool valid = lane < n;
            const int e = valid ? s_ids[lane] : 0;
            unsigned long long same = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) {
                const bool on = (e >> bit) & 1;
                const unsigned long long bb = __ballot(on);
                same &= on ? bb : ~bb;
            }
            const unsigned long long below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
            if (valid) f.perm[s_off[e] + __popcll(same & below)] = lane;
        }
        if (tid < E) {
            cnt_e = s_cnt[tid];
            off_e = s_off[tid];
            idx_e = s_act[tid];
        }
        if (tid == 0) {
            f.n_active[0] = s_nact;
            f.n_groups[0] = f.n_shared + s_nact;
            f.off[E] = s_off[E];
        }
    }
    if (tid < E) {
        f.cnt[tid] = cnt_e;
        f.off[tid] = off_e;
        if (cnt_e > 0) {
            f.active[idx_e] = tid;
            Group g;
            g.base = slot_e >= 0 ? f.pool + (size_t)slot_e * f.slot_bytes : nullptr;
            g.cnt = cnt_e;
            g.off = off_e;
            g.kind = 0;
            g.expert = tid;
            f.groups[f.n_shared + idx_e] = g;
            if (slot_e == -1) {  // missing (a remote expert, -2, is skipped quietly)
                atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
                const int code = f.layer * E + tid;
                atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small-T router: split-K GEMV over the interleaved router weights.
// Workgroup (expert block b of 64, slice row q) has 4 wavefronts, each one of
// 4 consecutive K-slices of 64 input columns (16 float4 chunks, all loads in
// flight at once), reduced in LDS in a fixed order.  Wavefronts of expert
// block j mod nb also form token j's sums and sums of squares of their 64
// columns and stage them as an fp16 span for the expert GEMVs.  Partials go
// to f.part / f.tpart (one row per workgroup row q).  One token: the last
// workgroup to arrive runs router_tail.  Several tokens: the last workgroup
// of each expert block sums that block's partials into logits (slices in
// order), and the last of those runs router_tail.
// ---------------------------------------------------------------------------

template <int NT>
__global__ void __launch_bounds__(RT_THREADS) k_router_small(Fwd f, const float* __restrict__ X)
{
    constexpr int RW = RT_THREADS / 64;
    __shared__ float red[RW][NT][64];
    __shared__ float sred[RW][NT][2];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = blockIdx.x, s = blockIdx.y * RW + w;
    const int H = f.H, T = f.T, CH = H / 4;
    // expert tid's bias and slot, for whichever workgroup runs the tail:
    // loaded first, so that they have arrived long before the last arrival
    float bias_e = 0.f;
    int slot_e = -1;
    if ((int)threadIdx.x < f.E) {
        bias_e = f.bias[threadIdx.x];
        slot_e = f.tbl[threadIdx.x];
    }
    const __amdgpu_buffer_rsrc_t rw =
        make_rsrc((const float4*)f.wr + ((size_t)b * CH + (size_t)s * 16) * 64, 16 * 1024);
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const uint4 q = bload16(rw, (uint32_t)lane * 16 + (u & 3) * 1024, (u >> 2) * 4096);
        v[u] = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                           __uint_as_float(q.w));
    }
    const int nb = gridDim.x;
    // this span of every token, one coalesced load each (several tokens: the
    // dot products read it back from LDS; one token reads it through the
    // scalar cache instead)
    __shared__ float xl[NT > 1 ? RW : 1][NT][64];
    float xa[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
        xa[j] = (j < T && (NT > 1 || j % nb == b)) ? X[(size_t)j * H + s * 64 + lane] : 0.f;
    if (NT > 1) {
#pragma unroll
        for (int j = 0; j < NT; ++j) xl[NT > 1 ? w : 0][j][lane] = xa[j];
    }
    {
        // token sums and sums of squares of this 64-column span; the span
        // staged as fp16 for the expert GEMVs (token j by expert block j mod nb)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < T && j % nb == b) {
                const float xv = xa[j];
                const float gs = wave_sum(xv), ss = wave_sum(xv * xv);
                stage_span64(xv, lane, (uint16_t*)(f.xq + (size_t)j * (H / 8) + s * 8),
                             f.xsc + (size_t)j * (H / 64) + s);
                if (lane == 0) {
                    sred[w][j][0] = gs;
                    sred[w][j][1] = ss;
                }
            }
    }
    if (NT > 1) __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        float acc = 0.f;
        if (j < T) {
            if (NT == 1) {
                cf32* xs = as_const(X + (size_t)j * H + s * 64);
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    acc = fmaf(v[u].x, xs[4 * u + 0], acc);
                    acc = fmaf(v[u].y, xs[4 * u + 1], acc);
                    acc = fmaf(v[u].z, xs[4 * u + 2], acc);
                    acc = fmaf(v[u].w, xs[4 * u + 3], acc);
                }
            } else {
                const float4* x4 = (const float4*)xl[NT > 1 ? w : 0][j];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float4 xq = x4[u];
                    acc = fmaf(v[u].x, xq.x, acc);
                    acc = fmaf(v[u].y, xq.y, acc);
                    acc = fmaf(v[u].z, xq.z, acc);
                    acc = fmaf(v[u].w, xq.w, acc);
                }
            }
        }
        red[w][j][lane] = acc;
    }
    __syncthreads();
    const int S = f.S, Sp = router_sp(T, S), S2p = router_s2p(S);
    for (int j = w; j < T; j += RW) {
        float acc = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < RW; ++v2) acc += red[v2][j][lane];
        const size_t at = NT == 1 ? (size_t)(b * 64 + lane) * Sp + blockIdx.y
                                  : ((size_t)blockIdx.y * T + j) * f.Epad + b * 64 + lane;
        st_agent(&f.part[at], acc);
    }
    if (w == 0 && lane < T && lane % nb == b) {
        float gs = 0.f, ss = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < RW; ++v2) {
            gs += sred[v2][lane][0];
            ss += sred[v2][lane][1];
        }
        st_agent(&f.tpart[(size_t)lane * S2p + 2 * blockIdx.y + 0], gs);
        st_agent(&f.tpart[(size_t)lane * S2p + 2 * blockIdx.y + 1], ss);
    }

    if (NT == 1) {
        if (!arrive_block(&f.counters[0], gridDim.x * gridDim.y)) return;
    } else {
        // the last of the block's workgroups sums its 64 experts' partials
        // (slices in order) into the logits; the last block runs the tail
        if (!arrive_block(&f.counters[1 + b], gridDim.y)) return;
        // (all loads unconditional, indices clamped, so that they issue together)
        const int tq = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        constexpr int NJ = (NT + RW - 1) / RW;  // tokens per wavefront
        float pv[NJ][64];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int j = tq + jj * RW;
            const float* pj = f.part + (size_t)min(j, T - 1) * f.Epad + b * 64 + lane;
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                const float v = ld_agent(pj + (size_t)min(i, S - 1) * T * f.Epad);
                pv[jj][i] = (j < T && i < S) ? v : 0.f;
            }
        }
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int j = tq + jj * RW;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 64; ++i) acc += pv[jj][i];
            if (j < T) st_agent(&part_logits(f)[(size_t)j * f.Epad + b * 64 + lane], acc);
        }
        if (!arrive_block(&f.counters[0], gridDim.x)) return;
    }
    router_tail<NT>(f, bias_e, slot_e);
}

// ---------------------------------------------------------------------------
// Router for 2..8 tokens from the row-major router copy.  Workgroups e < E
// (512 threads) hold expert e's row in registers (thread l: float4 columns
// l, l + 512, ...) and form its logits for all tokens at once (every
// token's loads in flight together, the 8 wavefronts' sums added in
// wavefront order), stored whole (part_logits: no partials, no per-block
// sums).  Workgroups E, E + 1, ... stage x meanwhile: slice u = (token, 8
// spans of 64), wavefront w taking span 8 q' + w, the slice's sum and sum of
// squares into tpart as two of the tail's 4-span slices (added there in
// order).  The last workgroup to arrive runs router_tail (its first 256
// threads), as the split-K router's does.
// ---------------------------------------------------------------------------

constexpr int R8_THREADS = 512;

template <int NT, int Q>  // Q float4 loads per thread per row (H <= 2048 Q)
__global__ void __launch_bounds__(R8_THREADS) k_router8(Fwd f)
{
    constexpr int RW = R8_THREADS / 64;
    __shared__ float s_red[RW][NT];
    __shared__ float s_st[RW][2];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int e = blockIdx.x, H = f.H, H4 = H / 4, T = f.T, E = f.E, Epad = f.Epad;
    float bias_e = 0.f;
    int slot_e = -1;
    if (tid < E) {
        bias_e = f.bias[tid];
        slot_e = f.tbl[tid];
    }
    if (e < E) {
        const float4* wr = (const float4*)(f.wr_rows + (size_t)e * H);
        float4 wv[Q], xv[NT][Q];
#pragma unroll
        for (int k = 0; k < Q; ++k) {
            const int c = tid + R8_THREADS * k;
            wv[k] = c < H4 ? wr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float4* xr = (const float4*)(f.x + (size_t)min(j, T - 1) * H);
#pragma unroll
            for (int k = 0; k < Q; ++k) xv[j][k] = xr[min(tid + R8_THREADS * k, H4 - 1)];
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < Q; ++k)
                if (tid + R8_THREADS * k < H4) {
                    a = fmaf(wv[k].x, xv[j][k].x, a);
                    a = fmaf(wv[k].y, xv[j][k].y, a);
                    a = fmaf(wv[k].z, xv[j][k].z, a);
                    a = fmaf(wv[k].w, xv[j][k].w, a);
                }
            a = wave_sum(a);
            if (lane == 0) s_red[w][j] = a;
        }
        __syncthreads();
        if (tid < T) {
            float l = 0.f;
#pragma unroll
            for (int v = 0; v < RW; ++v) l += s_red[v][tid];
            st_agent(&part_logits(f)[(size_t)tid * Epad + e], l);
        }
    } else {
        // x staged as fp16 spans; per slice of 8 spans the sums of spans
        // 8 q' .. 8 q' + 3 and 8 q' + 4 .. 8 q' + 7 (the tail's 4-span slices
        // 2 q' and 2 q' + 1)
        const int S = f.S, S2p = router_s2p(S), S8 = S / 2;
        for (int u = e - E; u < T * S8; u += gridDim.x - E) {
            const int t = u / S8, q = u - t * S8, sp = 8 * q + w;
            const float xv = f.x[(size_t)t * H + sp * 64 + lane];
            const float gs = wave_sum(xv), ss = wave_sum(xv * xv);
            stage_span64(xv, lane, (uint16_t*)(f.xq + (size_t)t * (H / 8) + sp * 8),
                         f.xsc + (size_t)t * (H / 64) + sp);
            if (lane == 0) {
                s_st[w][0] = gs;
                s_st[w][1] = ss;
            }
            __syncthreads();
            if (tid < 4) {
                const int hh = tid >> 1, c = tid & 1;  // half hh of the slice, sum or squares
                const float v = (s_st[4 * hh + 0][c] + s_st[4 * hh + 1][c]) +
                                (s_st[4 * hh + 2][c] + s_st[4 * hh + 3][c]);
                st_agent(&f.tpart[(size_t)t * S2p + 2 * (2 * q + hh) + c], v);
            }
            __syncthreads();
        }
    }
    if (!arrive_block_h(f.rt_cnt, gridDim.x)) return;
    if (tid >= RT_THREADS) return;  // the tail is written for RT_THREADS threads
    router_tail<NT>(f, bias_e, slot_e);
}

// ---------------------------------------------------------------------------
// One-token router, logits only: workgroup e computes expert e's whole raw
// logit x . Wr[e] from the row-major copy of the router weights (4
// wavefronts, each a quarter of the H inputs, all loads in flight at once,
// reduced in LDS in wavefront order) and stores it (part[4 e]); workgroup 0
// also forms the token's sum and sum of squares (tpart, and the RMSNorm
// factor), workgroup e stages x spans e, e + E, ... as fp16 for the expert
// kernels.  The selection (sigmoid, bias, top-K, weights) runs either in
// the one-token gate/up kernel, after this launch (SEL 0), or in this
// launch's workgroup 0, once the other workgroups' tagged logits are in:
// the plain sigmoid top-K (SEL 1, router1_select) or the general tail with
// softmax scoring and group-limited selection (SEL 2, router_tail).
// ---------------------------------------------------------------------------

// bounded wait of the selecting workgroup (polls of the tagged logits,
// each after a short sleep): far beyond any launch's duration
constexpr uint32_t RT_SPIN_MAX = 1u << 18;

// The one-token selection in the router's workgroup 0 (sigmoid scoring, one
// group, E <= 256): the same steps and arithmetic as the gate/up kernel's
// selection.  Workgroup e stores expert e's logit with this call's tag in
// one 64-bit word (rt_tag[e], a single store, agent scope); thread e here
// polls word e until it carries the tag (the tag is one more than the last
// selection's, rt_epoch, so a word from an earlier call never matches), up
// to RT_SPIN_MAX rounds (then it flags STATUS_WAIT and goes on).  rs_lds
// holds the token's RMSNorm factor, which this workgroup's thread 0 formed
// (read after the polls' barriers).  Writes ids,
// weights, perm and the routed groups' descriptors (missing experts
// flagged), so that the gate/up kernel reads its expert's slot from its
// group, and then the tag as the last selection's.  Every workgroup is
// resident at once (one per expert, a few per CU), so the wait ends.
// Thread e < E of workgroup 0: expert e's logit once its word carries the
// tag (the polls end together: a barrier per round).
__device__ float poll_logit(const Fwd& f, uint32_t tag)
{
    const int tid = threadIdx.x;
    uint64_t tv = 0;
    int ok = tid >= f.E;
    for (uint32_t n = 0;; ++n) {
        if (!ok) {
            tv = __hip_atomic_load(&f.rt_tag[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = (uint32_t)(tv >> 32) == tag;
        }
        if (__syncthreads_and(ok)) break;
        if (n == RT_SPIN_MAX) {
            if (tid == 0) atomicOr(&f.status[0], (uint32_t)STATUS_WAIT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return tid < f.E ? __uint_as_float((uint32_t)tv) : 0.f;
}

__device__ void router1_select(const Fwd& f, uint32_t tag, const float* rs_lds)
{
    __shared__ unsigned long long s_key[256];
    __shared__ unsigned long long s_cand[32];
    __shared__ float s_sig[256];
    __shared__ int s_slot[256];
    __shared__ int s_ids[8];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, E = f.E, K = f.K, ns = f.n_shared;
    const float bias = tid < E ? f.bias[tid] : 0.f;
    const int slot = tid < E ? f.tbl[tid] : -1;
    const float l = poll_logit(f, tag);
    const float rs = *rs_lds;
    unsigned long long key = 0ull;
    float sig = 0.f;
    if (tid < E) {
        sig = 1.0f / (1.0f + expf(-(l * rs)));
        key = ((unsigned long long)ord_float(sig + bias) << 32) | (uint32_t)(0xFFFFu - tid);
    }
    s_key[tid] = key;
    s_sig[tid] = sig;
    s_slot[tid] = slot;
    if (tid < 32) s_cand[tid] = 0ull;
    __syncthreads();
    {
        const unsigned long long* kb = &s_key[w * 64];
        const unsigned long long mine = kb[lane];
        int rank = 0;
#pragma unroll
        for (int e = 0; e < 64; e += 2) {
            const ulonglong2 kk = *(const ulonglong2*)&kb[e];
            rank += (kk.x > mine) + (kk.y > mine);
        }
        if (rank < K) s_cand[w * K + rank] = mine;
    }
    __syncthreads();
    if (tid < 4 * K) {
        const unsigned long long mine = s_cand[tid];
        int rank = 0;
        for (int j = 0; j < 4 * K; ++j) rank += s_cand[j] > mine;
        if (rank < K) s_ids[rank] = (int)(0xFFFFu - (uint32_t)(mine & 0xFFFFu));
    }
    __syncthreads();
    if (tid < K) {
        float sum = 0.f;
        for (int k = 0; k < K; ++k) sum += s_sig[s_ids[k]];
        const int ek = s_ids[tid], sk = s_slot[ek];
        const float sg = s_sig[ek];
        f.ids[tid] = ek;
        f.wts[tid] = f.norm_topk ? f.routed_scale * (sg / (sum + 1e-20f)) : f.routed_scale * sg;
        f.perm[tid] = tid;
        Group g;
        g.base = sk >= 0 ? f.pool + (size_t)sk * f.slot_bytes : nullptr;
        g.cnt = 1;
        g.off = tid;
        g.kind = 0;
        g.expert = ek;
        f.groups[ns + tid] = g;
        if (sk == -1) {  // missing (a remote expert, -2, is skipped quietly)
            atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
            const int code = f.layer * f.E + ek;
            atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
        }
    }
    if (tid == 0) f.rt_epoch[0] = tag;
}

template <int Q, int SEL>  // Q: float4 loads per lane and wavefront (H = 1024 Q)
__global__ void __launch_bounds__(RT_THREADS) k_router1(Fwd f, const float* __restrict__ X)
{
    constexpr int NW = RT_THREADS / 64;
    __shared__ float s_red[NW][3];
    __shared__ float s_rs, s_ss;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int e = blockIdx.x, H = f.H;
    // SEL 1, 2: this call's tag for the logits
    const uint32_t tag = SEL != 0 ? f.rt_epoch[0] + 1u : 0u;
    const float4* wr = (const float4*)(f.wr_rows + (size_t)e * H) + (size_t)w * (H / 16);
    const float4* x4 = (const float4*)X + (size_t)w * (H / 16);
    float4 a[Q], v[Q];
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        a[k] = wr[k * 64 + lane];
        v[k] = x4[k * 64 + lane];
    }
    // x spans e, e + E, ... as fp16 for the expert kernels (wavefront 0)
    if (w == 0)
        for (int sp = e; sp < H / 64; sp += gridDim.x) {
            const float xv = X[sp * 64 + lane];
            stage_span64(xv, lane, (uint16_t*)(f.xq + (size_t)sp * 8), f.xsc + sp);
        }
    float acc = 0.f, sum = 0.f, ss = 0.f;
#pragma unroll
    for (int k = 0; k < Q; ++k) {
        acc = fmaf(a[k].x, v[k].x, acc);
        acc = fmaf(a[k].y, v[k].y, acc);
        acc = fmaf(a[k].z, v[k].z, acc);
        acc = fmaf(a[k].w, v[k].w, acc);
    }
    acc = wave_sum(acc);
    if (e == 0) {  // the token's statistics, once
#pragma unroll
        for (int k = 0; k < Q; ++k) {
            sum += (v[k].x + v[k].y) + (v[k].z + v[k].w);
            ss = fmaf(v[k].x, v[k].x, ss);
            ss = fmaf(v[k].y, v[k].y, ss);
            ss = fmaf(v[k].z, v[k].z, ss);
            ss = fmaf(v[k].w, v[k].w, ss);
        }
        sum = wave_sum(sum);
        ss = wave_sum(ss);
    }
    if (lane == 0) {
        s_red[w][0] = acc;
        s_red[w][1] = sum;
        s_red[w][2] = ss;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float l = 0.f, gs = 0.f, sq = 0.f;
#pragma unroll
        for (int v2 = 0; v2 < NW; ++v2) {
            l += s_red[v2][0];
            gs += s_red[v2][1];
            sq += s_red[v2][2];
        }
        if (SEL != 0)
            __hip_atomic_store(&f.rt_tag[e], ((uint64_t)tag << 32) | __float_as_uint(l),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            st_agent(&f.part[(size_t)e * 4], l);  // one slice per expert (row stride 4)
        if (e == 0) {                             // one slice of token statistics
            st_agent(&f.tpart[0], gs);
            st_agent(&f.tpart[1], sq);
            const float rs = f.residual ? 1.0f / sqrtf(sq / (float)H + f.eps) : 1.0f;
            f.tok[0].xsum = gs;
            f.tok[0].rscale = rs;
            s_rs = rs;
            s_ss = sq;
            flag_range(f, sq);
        }
    }
    // the descriptors that do not depend on the selection (which the
    // gate/up kernel makes)
    if (e == 0 && (int)threadIdx.x < f.n_shared) {
        Group g;
        g.base = f.shared + (size_t)threadIdx.x * f.shared_bytes;
        g.cnt = 1;
        g.off = threadIdx.x;
        g.kind = 1;
        g.expert = -1;
        f.groups[threadIdx.x] = g;
    }
    if (e == 0 && threadIdx.x == 0) f.n_groups[0] = f.n_shared + f.K;
    if (SEL == 1 && e == 0) router1_select(f, tag, &s_rs);
    if (SEL == 2 && e == 0) {
        // the general tail in workgroup 0 once every tagged logit is in
        const int tid = threadIdx.x;
        const float bias_e = tid < f.E ? f.bias[tid] : 0.f;
        const int slot_e = tid < f.E ? f.tbl[tid] : -1;
        const float l = poll_logit(f, tag);  // (s_ss: read after its barriers)
        router_tail<1, true>(f, bias_e, slot_e, l, s_ss);
        if (tid == 0) f.rt_epoch[0] = tag;
    }
}

bool router1_ok(const Fwd& f)
{
    return f.T == 1 && f.wr_rows != nullptr && f.H % 1024 == 0 && f.H / 1024 <= 8;
}

template <int SEL>
static hipError_t router1_go(const Fwd& f, hipStream_t st)
{
    const dim3 grid((unsigned)f.E), block(RT_THREADS);
    switch (f.H / 1024) {
    case 1: return launch_k(k_router1<1, SEL>, grid, block, 0, st, f, f.x);
    case 2: return launch_k(k_router1<2, SEL>, grid, block, 0, st, f, f.x);
    case 3: return launch_k(k_router1<3, SEL>, grid, block, 0, st, f, f.x);
    case 4: return launch_k(k_router1<4, SEL>, grid, block, 0, st, f, f.x);
    case 5: return launch_k(k_router1<5, SEL>, grid, block, 0, st, f, f.x);
    case 6: return launch_k(k_router1<6, SEL>, grid, block, 0, st, f, f.x);
    case 7: return launch_k(k_router1<7, SEL>, grid, block, 0, st, f, f.x);
    default: return launch_k(k_router1<8, SEL>, grid, block, 0, st, f, f.x);
    }
}

hipError_t launch_router1(const Fwd& f, hipStream_t st)
{
    return f.sel_in_router == 2 ? router1_go<2>(f, st)
                                : f.sel_in_router ? router1_go<1>(f, st) : router1_go<0>(f, st);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

int router_small_slices(int H) { return (H / 64) / (RT_THREADS / 64); }

template <int NT>
static hipError_t router8_go(const Fwd& f, hipStream_t st)
{
    // experts, then staging workgroups: a slice of 8 spans each, up to 256
    const int stage = std::min(f.T * (f.S / 2), 256);
    const dim3 grid((unsigned)(f.E + stage)), block(R8_THREADS);
    switch ((f.H + 2047) / 2048) {
    case 1: return launch_k(k_router8<NT, 1>, grid, block, 0, st, f);
    case 2: return launch_k(k_router8<NT, 2>, grid, block, 0, st, f);
    case 3: return launch_k(k_router8<NT, 3>, grid, block, 0, st, f);
    default: return launch_k(k_router8<NT, 4>, grid, block, 0, st, f);
    }
}

hipError_t launch_router_small(const Fwd& f, hipStream_t st)
{
    if (f.T >= 2 && f.wr_rows != nullptr && f.H <= 8192 && f.H % 512 == 0)  // the row router
        return f.T <= 2 ? router8_go<2>(f, st) : f.T <= 4 ? router8_go<4>(f, st) : router8_go<8>(f, st);
    const dim3 grid(f.Epad / 64, router_small_slices(f.H)), block(RT_THREADS);
    if (f.T <= 1) return launch_k(k_router_small<1>, grid, block, 0, st, f, f.x);
    if (f.T <= 2) return launch_k(k_router_small<2>, grid, block, 0, st, f, f.x);
    if (f.T <= 4) return launch_k(k_router_small<4>, grid, block, 0, st, f, f.x);
    return launch_k(k_router_small<8>, grid, block, 0, st, f, f.x);
}

}  // namespace moe
