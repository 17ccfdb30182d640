// k_tok1.hip -- the one-token expert kernels: gate/up with SiLU*up, and down
// with the weighted combine, each in one launch and without partial sums
// leaving a workgroup.
//
// What is computed, cited by page title and section:
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11: each chosen
//     expert is SwiGLU (gate/up -> silu(g)*u -> down) and its output is added
//     with its routing weight; §04 siluf(x) = x/(1+exp(-x)).
//   GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6b-6d: 6144 -> 2048 ->
//     6144 experts, the shared expert always active, output = routed sum +
//     shared.
//   Edge0 write-up (magicnetworld.com) §三: affine int4 with group size 64.
//
// Work decomposition.  A workgroup owns 8 consecutive output rows of one
// matrix and reduces them completely, so no k-slice partials and no
// finalize or combine launch are needed; there are enough such workgroups
// (GLM shape: 9 x 256 for gate/up, 9 x 192 for down, a few per CU) to spread
// the stream over every CU evenly.  The 8 rows are one 8-row group of the
// slot layout, whose codes are one contiguous run per matrix (128 bytes per
// 32-input chunk), so a workgroup streams contiguous memory; a wavefront
// load, lane (row r of 8, span lane j of 8), covers 8 rows x 8 chunks.  Each step a lane takes two consecutive chunks (one span of
// 64 inputs, whose staged activation scale and sum it folds in itself).
// The lanes of one row are summed with a fixed butterfly, the wavefronts in
// LDS in wavefront order: results are bitwise reproducible.
//
// Gate/up: workgroup (expert group, 8 rows of I), W wavefronts each taking
// H / W inputs; x comes from the router's fp16 staging (spans of 64) through
// LDS; h = silu(g rs) (u rs) goes out in fp32.  Down: workgroup (8 rows of
// H), one wavefront per expert slot (shared experts, then the routed ones in
// rank order), each over all I inputs of its expert; the wavefront stages its
// expert's h as fp16 spans in LDS first (power-of-two scale per span); the
// slots are weighted and added in slot order (+ x for the residual form).
// That suits small layers; on large ones each workgroup would read all
// slots' h, so there the down workgroup is (expert group, 32 rows of H),
// one wavefront per 8-row group over all I inputs with the group's h staged
// once, and the last of a 64-row block's workgroups sums the slots.
//
// Roofline: HBM (the expert codes; the rest is a few hundred KB).
#include <algorithm>

#include "k_common.h"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t dwv(const uint4& v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

__device__ __forceinline__ float dot4(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                      const uint4& xv, float acc)
{
    acc = dot2(p0, xv.x, acc);
    acc = dot2(p1, xv.y, acc);
    acc = dot2(p2, xv.z, acc);
    acc = dot2(p3, xv.w, acc);
    return acc;
}

// 32 codes (one 16-byte piece of a row) against the chunk's 4 activation quads.
__device__ __forceinline__ float dot_chunk(const uint4& w, const uint4* xq, uint32_t mv, float acc)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t p0, p1, p2, p3;
        nib_pairs(dwv(w, d), mv, p0, p1, p2, p3);
        acc = dot4(p0, p1, p2, p3, xq[d], acc);
    }
    return acc;
}

__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// A span's accumulator folded into the running sum: row format (codes
// stored c + 8): sum c x = a/16 - 72 S; affine (w = sc q + mn): sum w x =
// sc a/16 + (mn - 64 sc) S; then the span's 2^-k.
template <int FMT>
__device__ __forceinline__ float fold_span(float tot, float a, float2 span, uint32_t pair)
{
    float v;
    if (FMT == MOE_W_INT4_ROW) {
        v = fmaf(a, 0.0625f, -72.f * span.y);
    } else {
        const float sc = bf_lo(pair), mn = bf_hi(pair);
        v = fmaf(sc * 0.0625f, a, (mn - 64.f * sc) * span.y);
    }
    return fmaf(v, span.x, tot);
}

// Sum over the 8 lanes of a row (lanes r, r+8, ..., r+56), fixed order.
__device__ __forceinline__ float row_sum8(float v)
{
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

__device__ __forceinline__ uint32_t h2pack(_Float16 lo, _Float16 hi)
{
    h2_t v;
    v.x = lo;
    v.y = hi;
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace

// ---------------------------------------------------------------------------
// One-token selection inside a 256-thread workgroup (sigmoid scoring, one
// group): thread e scores expert e from its raw logit (the router's dot
// product) times the token's RMSNorm factor: sigma, c = sigma + bias, key =
// (c, then lower id) in 64 bits, so distinct keys order as the pages'
// strict greater-than scan.  Wavefront w ranks block w of 64 experts; the
// block's keys of rank < K are candidates, and ranks among the 4K
// candidates give the top K in rank order.  Weights: sigma of the chosen
// experts, renormalised (+1e-20) and scaled, summed in rank order.  The
// same steps and arithmetic as the router tail.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t ordf1(float c)
{
    const uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct Sel1 {
    unsigned long long key[256];
    unsigned long long cand[32];
    float sig[256];
    int slot[256];
    int ids[8];
    float wts[8];
};

// Returns with s.ids / s.wts / s.slot valid for every thread of the block.
__device__ void select1(const Fwd& f, Sel1& s)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, E = f.E, K = f.K;
    const float l = tid < E ? f.part[(size_t)tid * 4] : 0.f;
    const float bias = tid < E ? f.bias[tid] : 0.f;
    const int slot = tid < E ? f.tbl[tid] : -1;
    const float ss = f.tpart[1];
    const float rs = f.residual ? 1.0f / sqrtf(ss / (float)f.H + f.eps) : 1.0f;
    unsigned long long key = 0ull;
    float sig = 0.f;
    if (tid < E) {
        sig = 1.0f / (1.0f + expf(-(l * rs)));
        key = ((unsigned long long)ordf1(sig + bias) << 32) | (uint32_t)(0xFFFFu - tid);
    }
    s.key[tid] = key;
    s.sig[tid] = sig;
    s.slot[tid] = slot;
    if (tid < 32) s.cand[tid] = 0ull;  // blocks with fewer than K real experts leave slots unset
    __syncthreads();
    {
        const unsigned long long* kb = &s.key[w * 64];
        const unsigned long long mine = kb[lane];
        int rank = 0;
#pragma unroll
        for (int e = 0; e < 64; e += 2) {
            const ulonglong2 kk = *(const ulonglong2*)&kb[e];
            rank += (kk.x > mine) + (kk.y > mine);
        }
        if (rank < K) s.cand[w * K + rank] = mine;
    }
    __syncthreads();
    if (tid < 4 * K) {
        const unsigned long long mine = s.cand[tid];
        int rank = 0;
        for (int j = 0; j < 4 * K; ++j) rank += s.cand[j] > mine;
        if (rank < K) s.ids[rank] = (int)(0xFFFFu - (uint32_t)(mine & 0xFFFFu));
    }
    __syncthreads();
    if (tid < K) {
        float sum = 0.f;
        for (int k = 0; k < K; ++k) sum += s.sig[s.ids[k]];
        const float sg = s.sig[s.ids[tid]];
        s.wts[tid] = f.norm_topk ? f.routed_scale * (sg / (sum + 1e-20f)) : f.routed_scale * sg;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// gate/up, one token: workgroup (group gi, 8-row block sb of I), W waves each
// taking H / W inputs in NST steps of 16 chunks, every load issued at once
// ---------------------------------------------------------------------------

template <int FMT, int W, int NST, bool SEL>
__global__ void __launch_bounds__(64 * W) k_gu8(Fwd f)
{
    extern __shared__ uint4 lds4[];
    __shared__ float s_red[W][16];
    const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
    const int H = f.H, I = f.I, C = H / 32, G = H / 64, NSB = I / 8;
    // workgroup -> (8-row group sb of I, expert group gi)
    const int sb = blockIdx.x % NSB, gi = blockIdx.x / NSB;
    int t = 0, r;
    const uint8_t* base;
    if (SEL) {
        // the router left raw logits (small layers; large ones select in the
        // router's last workgroup and take the other branch).  Group ns + k
        // is the expert of rank k; every routed workgroup selects for itself
        // (same steps, same result), and the first (group ns, row group 0)
        // also writes the selection out for the later kernels.
        const int ns = f.n_shared;
        if (gi < ns) {
            base = f.shared + (size_t)gi * f.shared_bytes;
            r = f.K + gi;
        } else {
            __shared__ Sel1 sel;
            __shared__ uint64_t s_base;
            const int k = gi - ns;
            r = k;
            select1(f, sel);
            if (k == 0 && sb == 0 && (int)threadIdx.x < f.K) {
                const int kk = threadIdx.x, ek = sel.ids[kk], sk = sel.slot[ek];
                f.ids[kk] = ek;
                f.wts[kk] = sel.wts[kk];
                f.perm[kk] = kk;
                Group g;
                g.base = sk >= 0 ? f.pool + (size_t)sk * f.slot_bytes : nullptr;
                g.cnt = 1;
                g.off = kk;
                g.kind = 0;
                g.expert = ek;
                f.groups[ns + kk] = g;
                if (sk == -1) {  // missing (a remote expert, -2, is skipped quietly)
                    atomicOr(&f.status[0], (uint32_t)STATUS_NOT_RESIDENT);
                    const int code = f.layer * f.E + ek;
                    atomicOr(&f.status[1 + code / 32], 1u << (code % 32));
                }
            }
            if (threadIdx.x == 0) {
                const int slot = sel.slot[sel.ids[k]];
                s_base = (uint64_t)(uintptr_t)(slot >= 0 ? f.pool + (size_t)slot * f.slot_bytes : nullptr);
            }
            __syncthreads();
            base = (const uint8_t*)(uintptr_t)s_base;
        }
        base = (const uint8_t*)(uintptr_t)(((uint64_t)(uint32_t)uni((int)(uint32_t)(uintptr_t)base)) |
                                           ((uint64_t)(uint32_t)uni((int)(uint32_t)((uintptr_t)base >> 32)) << 32));
    } else {
        if (gi >= uni(f.n_groups[0])) return;
        const Group grp = uni_group(f.groups, gi);
        tok_rows(f, f.perm, grp, 0, t, r);
        base = grp.base;
    }
    const int rr = lane & 7, j = lane >> 3;
    constexpr int CW = 16 * NST, NSP = CW / 2;  // chunks and spans of the wave
    const int c0 = w * CW;
    const uint8_t* anchor = (const uint8_t*)f.x;  // any valid address (empty resources)
    // the workgroup's 8 rows are one 8-row group of the slot layout: C * 128
    // contiguous bytes per matrix, 128 per chunk
    const uint32_t mbytes = base ? (uint32_t)C * 128 : 0u;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(base ? base + (size_t)sb * C * 128 : anchor, mbytes);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base ? base + (size_t)I * H / 2 + (size_t)sb * C * 128 : anchor, mbytes);
    const uint32_t voff = (uint32_t)rr * 16 + (uint32_t)(2 * j) * 128;
    uint4 A[2 * NST], B[2 * NST];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t so = (uint32_t)(c0 + st * 16 + h) * 128;
            A[2 * st + h] = bload16(rg, voff, so);
            B[2 * st + h] = bload16(ru, voff, so);
        }
    const uint8_t* tab = base ? base + (size_t)3 * H * I / 2 : anchor;
    uint32_t PA[NST], PB[NST];
    if (FMT != MOE_W_INT4_ROW) {
        const uint32_t tb = base ? (uint32_t)G * 32 : 0u;
        const __amdgpu_buffer_rsrc_t rtg = make_rsrc(tab + (size_t)sb * G * 32, tb);
        const __amdgpu_buffer_rsrc_t rtu = make_rsrc(tab + (size_t)I * G * 4 + (size_t)sb * G * 32, tb);
        const uint32_t toff = (uint32_t)rr * 4 + (uint32_t)j * 32;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const uint32_t so = (uint32_t)(c0 / 2 + st * 8) * 32;
            PA[st] = bload4(rtg, toff, so);
            PB[st] = bload4(rtu, toff, so);
        }
    }
    float sg = 1.f, su = 1.f;
    const int row = sb * 8 + rr;
    if (FMT == MOE_W_INT4_ROW && base != nullptr && threadIdx.x < 8) {
        sg = ((const float*)tab)[row];
        su = ((const float*)tab)[I + row];
    }
    // the wave's x spans into LDS (fp16 pair order, then (2^-k, sum) per span)
    uint4* xq = lds4 + (size_t)w * (NSP * 8 + (NSP + 1) / 2);
    float2* xs = (float2*)(xq + NSP * 8);
    {
        const uint4* gq = f.xq + (size_t)t * (H / 8) + (size_t)c0 * 4;
#pragma unroll
        for (int i = 0; i < NST; ++i) xq[lane + 64 * i] = gq[lane + 64 * i];  // NSP * 8 = 64 NST
        if (lane < NSP) xs[lane] = f.xsc[(size_t)t * (H / 64) + c0 / 2 + lane];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): LDS stores done
    __builtin_amdgcn_wave_barrier();
    const uint32_t mv = magic_vgpr();
    float Gt = 0.f, Ut = 0.f;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int sp = st * 8 + j;
        const uint4* xv = xq + sp * 8;
        float ag = dot_chunk(A[2 * st], xv, mv, 0.f), au = dot_chunk(B[2 * st], xv, mv, 0.f);
        ag = dot_chunk(A[2 * st + 1], xv + 4, mv, ag);
        au = dot_chunk(B[2 * st + 1], xv + 4, mv, au);
        const float2 span = xs[sp];
        Gt = fold_span<FMT>(Gt, ag, span, FMT == MOE_W_INT4_ROW ? 0u : PA[st]);
        Ut = fold_span<FMT>(Ut, au, span, FMT == MOE_W_INT4_ROW ? 0u : PB[st]);
    }
    Gt = row_sum8(Gt);
    Ut = row_sum8(Ut);
    if (lane < 8) {
        s_red[w][lane] = Gt;
        s_red[w][8 + lane] = Ut;
    }
    __syncthreads();
    if (threadIdx.x < 8) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < W; ++v) {
            g += s_red[v][threadIdx.x];
            u += s_red[v][8 + threadIdx.x];
        }
        const float rs = f.tok[t].rscale;
        g = g * sg * rs;
        u = u * su * rs;
        f.hf[(size_t)r * I + row] = g / (1.0f + expf(-g)) * u;
    }
}

// ---------------------------------------------------------------------------
// down + combine, one token: workgroup (8-row block ob of H), one wave per
// expert slot e (shared experts first, then the routed ones in rank order),
// PD steps of 16 chunks in flight
// ---------------------------------------------------------------------------

constexpr int D8_NE = 9;  // expert slots at most

template <int FMT, int PD>
__global__ void __launch_bounds__(64 * D8_NE) k_dn8(Fwd f)
{
    extern __shared__ uint4 lds4[];
    __shared__ float s_y[D8_NE][8];
    __shared__ float s_w[D8_NE];
    const int lane = threadIdx.x & 63, e = uni((int)(threadIdx.x >> 6));
    const int H = f.H, I = f.I, C = I / 32, NP = I / 64, K = f.K, ns = f.n_shared, NST = C / 16;
    const int ob = blockIdx.x, rr = lane & 7, j = lane >> 3;
    // this slot's h row (T = 1): routed rank k is row k, shared expert s row K + s
    const int hrow = e < ns ? K + e : e - ns;
    // its h first (lane c: chunk c of 32 inputs, I <= 2048), so that the
    // loads are in flight while the slot's expert is looked up
    const float4* hr = (const float4*)(f.hf + (size_t)hrow * I);
    float4 hv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) hv[q] = hr[(size_t)min(lane, C - 1) * 8 + q];
    // group g's slot: shared group s -> slot s; routed group ns + i holds the
    // expert of rank perm[i] (T = 1)
    const int ng = ns + K;
    const Group* gp = f.groups + min(lane, ng - 1);
    const uint64_t gbase = (uint64_t)(uintptr_t)gp->base;
    const int pv = lane >= ns && lane < ng ? f.perm[lane - ns] : -1;
    const float wv = e >= ns ? f.wts[e - ns] : 1.f;
    const int slot = lane < ns ? lane : (lane < ng ? ns + pv : -1);
    const unsigned long long m = __ballot(slot == e);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    const uint64_t bsel = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)gbase, src) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(gbase >> 32), src) << 32);
    const uint8_t* base = m ? (const uint8_t*)(uintptr_t)bsel : nullptr;
    const uint8_t* anchor = (const uint8_t*)f.x;
    // the workgroup's 8 rows are one 8-row group of the slot layout (C * 128
    // contiguous bytes, 128 per chunk; 32 bytes of affine pairs per input group)
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(base ? base + (size_t)I * H + (size_t)ob * C * 128 : anchor,
                  base ? (uint32_t)C * 128 : 0u);
    const uint32_t voff = (uint32_t)rr * 16 + (uint32_t)(2 * j) * 128;
    const uint8_t* tab = base ? base + (size_t)3 * H * I / 2 : anchor;
    const __amdgpu_buffer_rsrc_t rt =
        make_rsrc(tab + (size_t)2 * I * (H / 64) * 4 + (size_t)ob * NP * 32,
                  (FMT != MOE_W_INT4_ROW && base) ? (uint32_t)NP * 32 : 0u);
    const uint32_t toff = (uint32_t)rr * 4 + (uint32_t)j * 32;
    uint4 D[2 * PD];
    uint32_t P[PD];
#pragma unroll
    for (int k = 0; k < PD; ++k) {
        D[2 * k] = bload16(rd, voff, (uint32_t)(k * 16) * 128);
        D[2 * k + 1] = bload16(rd, voff, (uint32_t)(k * 16 + 1) * 128);
        if (FMT != MOE_W_INT4_ROW) P[k] = bload4(rt, toff, (uint32_t)(k * 8) * 32);
    }
    const int row = ob * 8 + rr;
    float sd = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr && lane < 8) sd = ((const float*)tab)[2 * I + row];
    if (lane == 0) s_w[e] = wv;

    // stage the slot's h as fp16 spans: lane c takes chunk c (32 inputs),
    // the two lanes of a span agree on its power-of-two scale
    uint4* hq = lds4 + (size_t)e * (C * 4 + (NP + 1) / 2);
    float2* hs = (float2*)(hq + C * 4);
    {
        const int c = lane;  // I <= 2048: one chunk per lane
        float mx = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(hv[q].x), fabsf(hv[q].y)),
                                 fmaxf(fabsf(hv[q].z), fabsf(hv[q].w))));
        mx = fmaxf(mx, __shfl_xor(mx, 1));  // the span's other chunk
        int ex;
        frexpf(mx, &ex);
        ex = max(ex, -100);
        const float sc = ldexpf(1.0f, 14 - ex);
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // quad q = inputs 8q..8q+7 of the chunk: hv[2q] (0..3), hv[2q+1] (4..7)
            const float4 lo = hv[2 * q], hi = hv[2 * q + 1];
            const _Float16 a0 = (_Float16)(lo.x * sc), a1 = (_Float16)(lo.y * sc);
            const _Float16 a2 = (_Float16)(lo.z * sc), a3 = (_Float16)(lo.w * sc);
            const _Float16 a4 = (_Float16)(hi.x * sc), a5 = (_Float16)(hi.y * sc);
            const _Float16 a6 = (_Float16)(hi.z * sc), a7 = (_Float16)(hi.w * sc);
            if (c < C)
                hq[c * 4 + q] = make_uint4(h2pack(a0, a4), h2pack(a1, a5), h2pack(a2, a6),
                                           h2pack(a3, a7));
            sum += (((float)a0 + (float)a1) + ((float)a2 + (float)a3)) +
                   (((float)a4 + (float)a5) + ((float)a6 + (float)a7));
        }
        sum += __shfl_xor(sum, 1);
        if (c < C && !(c & 1)) hs[c >> 1] = make_float2(ldexpf(1.0f, ex - 14), sum);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
    const uint32_t mv = magic_vgpr();
    float Yt = 0.f;
#pragma unroll 1
    for (int st0 = 0; st0 < NST; st0 += PD) {
#pragma unroll
        for (int k = 0; k < PD; ++k) {
            const int sp = (st0 + k) * 8 + j;
            const uint4* xv = hq + sp * 8;
            const uint4 d0 = D[2 * k], d1 = D[2 * k + 1];
            const uint32_t pv2 = P[k];
            const uint32_t so = (uint32_t)((st0 + k + PD) * 16) * 128;
            D[2 * k] = bload16(rd, voff, so);
            D[2 * k + 1] = bload16(rd, voff, so + 128);
            if (FMT != MOE_W_INT4_ROW) P[k] = bload4(rt, toff, (uint32_t)((st0 + k + PD) * 8) * 32);
            float a = dot_chunk(d0, xv, mv, 0.f);
            a = dot_chunk(d1, xv + 4, mv, a);
            Yt = fold_span<FMT>(Yt, a, hs[sp], FMT == MOE_W_INT4_ROW ? 0u : pv2);
        }
    }
    Yt = row_sum8(Yt);
    if (lane < 8) s_y[e][lane] = base ? Yt * sd : 0.f;
    __syncthreads();
    if (threadIdx.x < 8) {
        float o = 0.f;
        for (int v = 0; v < ng; ++v) {
            const float y = s_y[v][threadIdx.x];
            o = v < ns ? o + y : fmaf(s_w[v], y, o);
        }
        const int oi = ob * 8 + threadIdx.x;
        if (f.residual) o = f.x[oi] + o;
        f.out[oi] = o;
    }
}

// ---------------------------------------------------------------------------
// down + combine, one token, large layers: workgroup (expert group gi, 8W
// rows of H), wave v the 8-row group of its rows over all I inputs (NST steps
// of 16 chunks, every load issued at once, one contiguous run of the slot
// layout per wave and 8W * I/2 bytes per workgroup); the group's h is staged
// once per workgroup as fp16 spans.  Each workgroup writes its rows' results;
// the last of the 64-row block's workgroups to arrive sums them (shared
// experts, then the routed ones in rank order) and writes the block's
// outputs (+ x for the residual form).
// ---------------------------------------------------------------------------

template <int FMT, int W, int NST>
__global__ void __launch_bounds__(64 * W) k_dnb(Fwd f)
{
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x & 63, w = uni((int)(threadIdx.x >> 6));
    const int H = f.H, I = f.I, C = I / 32, NP = I / 64, NB = H / 64, PB = 8 / W;
    // workgroup -> (part hb of 64-row block b, expert group gi)
    const int hb = blockIdx.x % PB, b = (blockIdx.x / PB) % NB, gi = blockIdx.x / (PB * NB);
    const int ng = uni(f.n_groups[0]);
    if (gi >= ng) return;
    const Group grp = uni_group(f.groups, gi);
    int t = 0, r = 0;
    tok_rows(f, f.perm, grp, 0, t, r);
    const uint8_t* base = grp.base;
    const uint8_t* anchor = (const uint8_t*)f.x;  // any valid address (empty resources)
    const int sb = b * 8 + hb * W + w, rr = lane & 7, j = lane >> 3;
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(base ? base + (size_t)I * H + (size_t)sb * C * 128 : anchor,
                  base ? (uint32_t)C * 128 : 0u);
    const uint32_t voff = (uint32_t)rr * 16 + (uint32_t)(2 * j) * 128;
    const uint8_t* tab = base ? base + (size_t)3 * H * I / 2 : anchor;
    const __amdgpu_buffer_rsrc_t rt =
        make_rsrc(tab + (size_t)2 * I * (H / 64) * 4 + (size_t)sb * NP * 32,
                  (FMT != MOE_W_INT4_ROW && base) ? (uint32_t)NP * 32 : 0u);
    const uint32_t toff = (uint32_t)rr * 4 + (uint32_t)j * 32;
    uint4 D[2 * NST];
    uint32_t P[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        D[2 * st] = bload16(rd, voff, (uint32_t)(st * 16) * 128);
        D[2 * st + 1] = bload16(rd, voff, (uint32_t)(st * 16 + 1) * 128);
        P[st] = FMT != MOE_W_INT4_ROW ? bload4(rt, toff, (uint32_t)(st * 8) * 32) : 0u;
    }
    const int row = sb * 8 + rr;
    float sd = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr && lane < 8) sd = ((const float*)tab)[2 * I + row];

    // the group's h as fp16 spans: thread g takes inputs 8g .. 8g+7, the 8
    // threads of a span agree on its power-of-two scale and sum its values
    uint4* hq = lds4;
    float2* hs = (float2*)(hq + C * 4);
    {
        const float4* hr = (const float4*)(f.hf + (size_t)r * I);
        const int n8 = I / 8;  // a multiple of 64: whole wavefronts in or out
        for (int g = threadIdx.x; g - lane < n8; g += 64 * W) {
            const float4 lo = hr[2 * g], hi = hr[2 * g + 1];
            float mx = fmaxf(fmaxf(fmaxf(fabsf(lo.x), fabsf(lo.y)), fmaxf(fabsf(lo.z), fabsf(lo.w))),
                             fmaxf(fmaxf(fabsf(hi.x), fabsf(hi.y)), fmaxf(fabsf(hi.z), fabsf(hi.w))));
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            mx = fmaxf(mx, __shfl_xor(mx, 4));
            int ex;
            frexpf(mx, &ex);
            ex = max(ex, -100);
            const float sc = ldexpf(1.0f, 14 - ex);
            const _Float16 a0 = (_Float16)(lo.x * sc), a1 = (_Float16)(lo.y * sc);
            const _Float16 a2 = (_Float16)(lo.z * sc), a3 = (_Float16)(lo.w * sc);
            const _Float16 a4 = (_Float16)(hi.x * sc), a5 = (_Float16)(hi.y * sc);
            const _Float16 a6 = (_Float16)(hi.z * sc), a7 = (_Float16)(hi.w * sc);
            hq[g] = make_uint4(h2pack(a0, a4), h2pack(a1, a5), h2pack(a2, a6), h2pack(a3, a7));
            float sum = (((float)a0 + (float)a1) + ((float)a2 + (float)a3)) +
                        (((float)a4 + (float)a5) + ((float)a6 + (float)a7));
            sum += __shfl_xor(sum, 1);
            sum += __shfl_xor(sum, 2);
            sum += __shfl_xor(sum, 4);
            if ((g & 7) == 0) hs[g >> 3] = make_float2(ldexpf(1.0f, ex - 14), sum);
        }
    }
    __syncthreads();
    const uint32_t mv = magic_vgpr();
    float Yt = 0.f;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        const int sp = st * 8 + j;
        const uint4* xv = hq + sp * 8;
        float a = dot_chunk(D[2 * st], xv, mv, 0.f);
        a = dot_chunk(D[2 * st + 1], xv + 4, mv, a);
        Yt = fold_span<FMT>(Yt, a, hs[sp], P[st]);
    }
    Yt = row_sum8(Yt);
    if (lane < 8) st_agent(f.ypart + (size_t)r * H + row, base ? Yt * sd : 0.f);
    if (!arrive_block(f.dn_cnt + (size_t)b * 64, (uint32_t)(ng * PB))) return;
    if (w != 0) return;
    // one token: routed rank k is h row k, shared expert s row K + s
    const int K = f.K, ns = f.n_shared, d = b * 64 + lane;
    float v[D8_NE];
#pragma unroll
    for (int e = 0; e < D8_NE; ++e) {
        const int re = e < ns ? K + e : e - ns;
        v[e] = e < ng ? ld_agent(f.ypart + (size_t)re * H + d) : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < D8_NE; ++e)
        if (e < ng) m = e < ns ? m + v[e] : fmaf(f.wts[e - ns], v[e], m);
    if (f.residual) m = f.x[d] + m;
    f.out[d] = m;
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

namespace {

// waves per gate/up workgroup (each takes H / W inputs) and its steps of 16
// chunks (all in flight at once)
bool gu8_shape(int H, int& W, int& nst)
{
    if (H % 512) return false;
    const int C = H / 32;
    W = std::min(4, C / 16);
    if (C % (16 * W)) return false;
    nst = C / (16 * W);
    return nst >= 1 && nst <= 4;
}

size_t gu8_lds(int W, int nst) { return (size_t)W * (nst * 64 + (nst * 8 + 1) / 2) * 16; }

size_t dn8_lds(int I, int ne) { return (size_t)ne * ((I / 32) * 4 + (I / 64 + 1) / 2) * 16; }

int tok1_pd(int steps) { return steps % 2 == 0 ? 2 : 1; }

template <typename Kern>
hipError_t lds_attr(Kern kern, size_t lds)
{
    if (lds <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds);
}

template <int FMT, int W, int NST>
hipError_t gu8_go(const Fwd& f, hipStream_t st)
{
    const unsigned wgs = (unsigned)((f.n_shared + f.K) * (f.I / 8));
    const size_t lds = gu8_lds(W, NST);
    if (W == 4 && f.sel_in_gateup) {
        const hipError_t e = lds_attr(k_gu8<FMT, 4, NST, true>, lds);
        if (e != hipSuccess) return e;
        return launch_k(k_gu8<FMT, 4, NST, true>, dim3(wgs), dim3(256), lds, st, f);
    }
    const hipError_t e = lds_attr(k_gu8<FMT, W, NST, false>, lds);
    if (e != hipSuccess) return e;
    return launch_k(k_gu8<FMT, W, NST, false>, dim3(wgs), dim3(64 * W), lds, st, f);
}

template <int FMT, int W>
hipError_t gu8_nst(const Fwd& f, hipStream_t st, int nst)
{
    switch (nst) {
    case 1: return gu8_go<FMT, W, 1>(f, st);
    case 2: return gu8_go<FMT, W, 2>(f, st);
    case 3: return gu8_go<FMT, W, 3>(f, st);
    default: return gu8_go<FMT, W, 4>(f, st);
    }
}

template <int FMT>
hipError_t gu8_fmt(const Fwd& f, hipStream_t st)
{
    int W = 0, nst = 0;
    gu8_shape(f.H, W, nst);
    switch (W) {
    case 1: return gu8_nst<FMT, 1>(f, st, nst);
    case 2: return gu8_nst<FMT, 2>(f, st, nst);
    case 3: return gu8_nst<FMT, 3>(f, st, nst);
    default: return gu8_nst<FMT, 4>(f, st, nst);
    }
}

template <int FMT, int PD>
hipError_t dn8_go(const Fwd& f, hipStream_t st)
{
    const int ne = f.n_shared + f.K;
    const size_t lds = dn8_lds(f.I, ne);
    const hipError_t e = lds_attr(k_dn8<FMT, PD>, lds);
    if (e != hipSuccess) return e;
    return launch_k(k_dn8<FMT, PD>, dim3((unsigned)(f.H / 8)), dim3(64 * ne), lds, st, f);
}

// waves per block-down workgroup (8 rows each; 8 / DNB_W workgroups per
// 64-row block)
constexpr int DNB_W = 4;

size_t dnb_lds(int I) { return (size_t)(I / 8) * 16 + (size_t)(I / 64) * 8; }

template <int FMT, int NST>
hipError_t dnb_go(const Fwd& f, hipStream_t st)
{
    const unsigned wgs = (unsigned)((f.n_shared + f.K) * (f.H / 64) * (8 / DNB_W));
    return launch_k(k_dnb<FMT, DNB_W, NST>, dim3(wgs), dim3(64 * DNB_W), dnb_lds(f.I), st, f);
}

template <int FMT>
hipError_t dnb_fmt(const Fwd& f, hipStream_t st)
{
    switch (f.I / 512) {
    case 1: return dnb_go<FMT, 1>(f, st);
    case 2: return dnb_go<FMT, 2>(f, st);
    case 3: return dnb_go<FMT, 3>(f, st);
    default: return dnb_go<FMT, 4>(f, st);
    }
}

template <int FMT>
hipError_t dn8_fmt(const Fwd& f, hipStream_t st)
{
    // at most 2 steps in flight: the slot's h staging holds registers too
    if (tok1_pd(f.I / 512) == 2) return dn8_go<FMT, 2>(f, st);
    return dn8_go<FMT, 1>(f, st);
}

}  // namespace

// Shapes the one-token gate/up kernel covers: H a multiple of 512 up to
// 8192, I a multiple of 512, int4 shared experts, the token's x within the
// LDS of a workgroup.
bool tok1_ok(const Fwd& f)
{
    int W = 0, nst = 0;
    return f.T == 1 && !shared_int8(f) && gu8_shape(f.H, W, nst) && f.I % 512 == 0 &&
           f.hf != nullptr && gu8_lds(W, nst) <= (size_t)f.lds_max;
}

// The one-token down + combine kernel: I up to 2048 (one h chunk per lane),
// at most 9 expert slots, and small down projections (at most 16 MiB of
// codes per token): every workgroup reads the slots' whole h, which a large
// layer pays for in L2 traffic, so there the down GEMV units (64 rows each,
// h in k-slices) and the combine kernel run instead.
bool tok1_down_ok(const Fwd& f)
{
    const int ne = f.n_shared + f.K;
    return tok1_ok(f) && f.I <= 2048 && ne <= D8_NE && (size_t)ne * f.H * f.I / 2 <= ((size_t)16 << 20) &&
           dn8_lds(f.I, ne) <= (size_t)f.lds_max;
}

// The block down + combine kernel: I up to 2048 (all of a wave's codes in
// flight at once), at most 9 expert slots, the block arrival counters.
bool tok1_dnb_ok(const Fwd& f)
{
    return tok1_ok(f) && f.I <= 2048 && f.n_shared + f.K <= D8_NE && f.dn_cnt != nullptr;
}

// The selection can move into the gate/up kernel (256-thread workgroups,
// one thread per expert) for the plain sigmoid top-K.
bool tok1_sel_ok(const Fwd& f)
{
    int W = 0, nst = 0;
    return tok1_ok(f) && gu8_shape(f.H, W, nst) && W == 4 && f.E <= 256 &&
           f.scoring == MOE_SCORE_SIGMOID && f.n_group == 1;
}

// Where the one-token selection runs: on large layers (more than 512
// gate/up workgroups) in the router's last workgroup, behind an arrival;
// on small ones in every routed gate/up workgroup (the arrival and the
// extra launch tail would cost more than the redundant selections).
bool tok1_sel_in_router(const Fwd& f) { return (f.n_shared + f.K) * (f.I / 8) > 512; }

hipError_t launch_tok1_gateup(const Fwd& f, hipStream_t st)
{
    return f.fmt == MOE_W_INT4_ROW ? gu8_fmt<MOE_W_INT4_ROW>(f, st)
                                   : gu8_fmt<MOE_W_INT4_AFFINE_G64>(f, st);
}

hipError_t launch_tok1_down_blocks(const Fwd& f, hipStream_t st)
{
    return f.fmt == MOE_W_INT4_ROW ? dnb_fmt<MOE_W_INT4_ROW>(f, st)
                                   : dnb_fmt<MOE_W_INT4_AFFINE_G64>(f, st);
}

hipError_t launch_tok1_down(const Fwd& f, hipStream_t st)
{
    return f.fmt == MOE_W_INT4_ROW ? dn8_fmt<MOE_W_INT4_ROW>(f, st)
                                   : dn8_fmt<MOE_W_INT4_AFFINE_G64>(f, st);
}

}  // namespace moe
