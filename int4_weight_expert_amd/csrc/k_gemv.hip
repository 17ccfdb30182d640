// k_gemv.hip -- the int4 expert GEMVs of the decode-size forward, as
// persistent kernels over a work queue.
//
// What is computed, cited by page title and section:
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11: each chosen
//     expert is SwiGLU on the rows routed to it (gate/up -> silu(g)*u ->
//     down) and its output is added with its routing weight; the batch's
//     experts are read once each; §04 siluf(x) = x/(1+exp(-x)).
//   GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6b-6d: 6144 -> 2048 ->
//     6144 experts, the shared expert always active, output = routed sum +
//     shared.
//   Edge0 write-up (magicnetworld.com) §三: affine int4 with group size 64.
//
// Work decomposition.  A unit is (expert group g, 64-row block b, k-slice q):
// one wavefront -- a workgroup of its own -- streams the slice's 16-byte
// chunks of those 64 rows (lane = row, 1 KiB coalesced buffer loads, see the
// slot layout) for every token of the group, two batches of loads in flight.
// Thousands of small workgroups let the hardware dispatcher keep every SIMD
// equally busy whatever the routing.  Partial sums go to a buffer indexed by
// the unit and the last unit of a (group, row block) -- or of a row block,
// for the down projection -- reduces them in a fixed order: results are
// bitwise reproducible.
//
// Arithmetic per weight: one AND per 4 codes, one v_cvt_f32_ubyteN per code,
// one v_fmac_f32 per code and token.  Row-format codes are stored code + 8;
// the unit subtracts 8 * (sum of its activations) once.  Activations of the
// slice are staged in the wavefront's own LDS area and read with
// wave-uniform (broadcast) ds_read_b128.
#include "k_common.h"

namespace moe {

constexpr int SUB = 16;  // chunks staged in LDS at a time
constexpr int UG = 4;    // chunks per batch of gate/up loads (x2 matrices)
constexpr int UD = 8;    // chunks per batch of down loads

__device__ __forceinline__ void lds_wave_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// Unit index -> (group, row block, k-slice).  Units of one k-slice and row
// block are adjacent across groups so that a (group, row block)'s slices are
// spread over the launch.
__device__ __forceinline__ void unit_coords(int u, int n_groups_max, int NB, int& gi, int& b,
                                            int& q)
{
    gi = u % n_groups_max;
    const int rest = u / n_groups_max;
    b = rest % NB;
    q = rest / NB;
}

// One batch of U chunks in flight per wavefront (the other resident
// wavefronts of the SIMD hide the latency); the first batch is issued before
// the activations are staged.  (Written out with macros: the buffers must
// stay in registers.)
#define GU_LOAD(BG, BU, I_)                                                        \
    _Pragma("unroll") for (int k_ = 0; k_ < UG; ++k_)                               \
    {                                                                              \
        BG[k_] = bload16(rg, voff + k_ * 1024, (sc0 + (I_) * UG) * 1024);           \
        BU[k_] = bload16(ru, voff + k_ * 1024, (sc0 + (I_) * UG) * 1024);           \
    }
#define GU_USE(BG, BU, I_)                                                         \
    _Pragma("unroll") for (int j_ = 0; j_ < NT; ++j_) if (j_ < nj)                 \
    {                                                                              \
        _Pragma("unroll") for (int k_ = 0; k_ < UG; ++k_)                           \
        {                                                                          \
            const float* xp_ = xl + j_ * SUB * 32 + ((I_) * UG + k_) * 32;          \
            dot32(BG[k_], xp_, ge[j_], go[j_]);                                    \
            dot32(BU[k_], xp_, ue[j_], uo[j_]);                                    \
        }                                                                          \
    }
#define DN_LOAD(BD, I_)                                                            \
    _Pragma("unroll") for (int k_ = 0; k_ < UD; ++k_)                               \
        BD[k_] = bload16(rd, voff + k_ * 1024, (sc0 + (I_) * UD) * 1024);
#define DN_USE(BD, I_)                                                             \
    _Pragma("unroll") for (int j_ = 0; j_ < NT; ++j_) if (j_ < nj)                 \
    {                                                                              \
        _Pragma("unroll") for (int k_ = 0; k_ < UD; ++k_)                           \
        {                                                                          \
            dot32(BD[k_], hl + j_ * SUB * 32 + ((I_) * UD + k_) * 32, ye[j_], yo[j_]); \
        }                                                                          \
    }

// ---------------------------------------------------------------------------
// gate/up: h[r][row] = silu(sg[row] * (Wg x)_row * rs) * (su[row] * (Wu x)_row * rs)
// ---------------------------------------------------------------------------

template <int FMT, int NT>
__global__ void __launch_bounds__(64, 4)
    k_gu(Fwd f, const float* __restrict__ X, const Group* __restrict__ GR,
         const int32_t* __restrict__ P, const TokStat* __restrict__ TS,
         const int32_t* __restrict__ NG, float* __restrict__ Hout, int n_groups_max)
{
    __shared__ float xl[NT * SUB * 32];
    const int lane = threadIdx.x;
    const int H = f.H, I = f.I, C = H / 32, G = H / 64, NB = I / 64;
    const int KS = f.gu_ks, CPU = f.gu_cpu;
    int gi, b, q;
    unit_coords(blockIdx.x, n_groups_max, NB, gi, b, q);
    if (gi >= NG[0]) return;
    const Group grp = GR[gi];
    const int row = b * 64 + lane, c0 = q * CPU;
    const uint8_t* base = grp.base;
    const uint32_t voff = (uint32_t)lane * 16;
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc(base + ((size_t)b * C + c0) * 1024, (uint32_t)CPU * 1024);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base + (size_t)I * H / 2 + ((size_t)b * C + c0) * 1024, (uint32_t)CPU * 1024);
    float sgr = 1.f, sur = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr) {
        const float* sc = (const float*)(base + (size_t)3 * H * I / 2);
        sgr = sc[row];
        sur = sc[I + row];
    }
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int tt[NT], rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            tt[j] = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, P, grp, p0 + j, tt[j], rr[j]);
        }
        float ge[NT], go[NT], ue[NT], uo[NT], xs[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) ge[j] = go[j] = ue[j] = uo[j] = xs[j] = 0.f;
        if (base != nullptr) {
            for (int sc0 = 0; sc0 < CPU; sc0 += SUB) {
                const int ns = min(SUB, CPU - sc0);
                auto stage = [&]() {
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        if (j < nj) {
                            const float4* src =
                                (const float4*)(X + (size_t)tt[j] * H + (size_t)(c0 + sc0) * 32);
                            for (int i = lane; i < ns * 8; i += 64) {
                                const float4 v = src[i];
                                ((float4*)(xl + j * SUB * 32))[i] = v;
                                xs[j] += (v.x + v.y) + (v.z + v.w);
                            }
                        }
                    lds_wave_sync();
                };
                if (FMT == MOE_W_INT4_ROW) {
                    const int nbt = ns / UG;
                    uint4 ag[UG], au[UG];
                    if (nbt > 0) {
                        GU_LOAD(ag, au, 0)
                    }
                    stage();  // overlaps the first batch's loads
                    for (int i = 0; i < nbt; ++i) {
                        if (i > 0) {
                            GU_LOAD(ag, au, i)
                        }
                        GU_USE(ag, au, i)
                    }
                    for (int c = nbt * UG; c < ns; ++c) {
                        const uint4 vg = bload16(rg, voff, (sc0 + c) * 1024);
                        const uint4 vu = bload16(ru, voff, (sc0 + c) * 1024);
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            if (j < nj) {
                                const float* xp = xl + j * SUB * 32 + c * 32;
                                dot32(vg, xp, ge[j], go[j]);
                                dot32(vu, xp, ue[j], uo[j]);
                            }
                    }
                } else {
                    // affine: groups of 64 inputs (2 chunks), (scale, min) per row and group
                    stage();
                    const uint32_t* ag = (const uint32_t*)(base + (size_t)3 * H * I / 2) +
                                         (size_t)b * G * 64 + lane;
                    const uint32_t* au = ag + (size_t)I * G;
                    for (int c = 0; c < ns; c += 2) {
                        const int gq = (c0 + sc0 + c) / 2;
                        const uint4 g0 = bload16(rg, voff, (sc0 + c) * 1024);
                        const uint4 g1 = bload16(rg, voff + 1024, (sc0 + c) * 1024);
                        const uint4 u0 = bload16(ru, voff, (sc0 + c) * 1024);
                        const uint4 u1 = bload16(ru, voff + 1024, (sc0 + c) * 1024);
                        const uint32_t pg = ag[(size_t)gq * 64], pu = au[(size_t)gq * 64];
                        const float scg = __uint_as_float(pg << 16);
                        const float mng = __uint_as_float(pg & 0xFFFF0000u);
                        const float scu = __uint_as_float(pu << 16);
                        const float mnu = __uint_as_float(pu & 0xFFFF0000u);
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            if (j < nj) {
                                const float* xp = xl + j * SUB * 32 + c * 32;
                                const float sx = wave_sum(xp[lane]);
                                float ae = 0.f, ao = 0.f, be = 0.f, bo = 0.f;
                                dot32(g0, xp, ae, ao);
                                dot32(g1, xp + 32, ae, ao);
                                dot32(u0, xp, be, bo);
                                dot32(u1, xp + 32, be, bo);
                                ge[j] = fmaf(scg, fmaf(ao, 0.0625f, ae), fmaf(mng, sx, ge[j]));
                                ue[j] = fmaf(scu, fmaf(bo, 0.0625f, be), fmaf(mnu, sx, ue[j]));
                            }
                    }
                }
                lds_wave_sync();
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                float gp = ge[j], up = ue[j];
                if (FMT == MOE_W_INT4_ROW) {
                    const float x8 = 8.0f * wave_sum(xs[j]);
                    gp = (fmaf(go[j], 0.0625f, ge[j]) - x8) * sgr;
                    up = (fmaf(uo[j], 0.0625f, ue[j]) - x8) * sur;
                }
                if (KS == 1) {
                    const float rs = TS[tt[j]].rscale;
                    const float gg = gp * rs, uu = up * rs;
                    Hout[(size_t)rr[j] * I + row] = gg / (1.0f + expf(-gg)) * uu;
                } else {
                    float* pp = f.gu_part + (((size_t)rr[j] * NB + b) * KS + q) * 128;
                    st_agent(pp + lane, gp);
                    st_agent(pp + 64 + lane, up);
                }
            }
    }
    if (KS > 1 && arrive_wave(&f.gu_ctr[gi * NB + b], KS)) {
        for (int j = 0; j < grp.cnt; ++j) {
            int t, r;
            tok_rows(f, P, grp, j, t, r);
            const float* pp = f.gu_part + ((size_t)r * NB + b) * KS * 128;
            float gg = 0.f, uu = 0.f;
            for (int q0 = 0; q0 < KS; q0 += 8) {
                float a[8], c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a[i] = q0 + i < KS ? ld_agent(pp + (q0 + i) * 128 + lane) : 0.f;
                    c[i] = q0 + i < KS ? ld_agent(pp + (q0 + i) * 128 + 64 + lane) : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    gg += a[i];
                    uu += c[i];
                }
            }
            const float rs = TS[t].rscale;
            gg *= rs;
            uu *= rs;
            Hout[(size_t)r * I + row] = gg / (1.0f + expf(-gg)) * uu;
        }
    }
}

// ---------------------------------------------------------------------------
// down: partial y[r][row] over k-slices; the last unit of a row block sums
// them and combines: out[t] = (x[t] +) sum_s y_shared_s + sum_k w_tk y_tk.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float sum_slices(const float* pp, int KS, int lane)
{
    float s = 0.f;
    for (int q0 = 0; q0 < KS; q0 += 8) {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = q0 + i < KS ? ld_agent(pp + (q0 + i) * 64 + lane) : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) s += a[i];
    }
    return s;
}

template <int FMT, int NT>
__global__ void __launch_bounds__(64, 4)
    k_dn(Fwd f, const Group* __restrict__ GR, const int32_t* __restrict__ P,
         const float* __restrict__ Hin, const int32_t* __restrict__ NG, int n_groups_max,
         int fused_combine)
{
    __shared__ float hl[NT * SUB * 32];
    const int lane = threadIdx.x;
    const int H = f.H, I = f.I, C = I / 32, GI = I / 64, NB = H / 64;
    const int KS = f.dn_ks, CPU = f.dn_cpu;
    int gi, b, q;
    unit_coords(blockIdx.x, n_groups_max, NB, gi, b, q);
    const int n_groups = NG[0];
    if (gi >= n_groups) return;
    const Group grp = GR[gi];
    const int row = b * 64 + lane, c0 = q * CPU;
    const uint8_t* base = grp.base;
    const uint32_t voff = (uint32_t)lane * 16;
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(base + (size_t)I * H + ((size_t)b * C + c0) * 1024, (uint32_t)CPU * 1024);
    float sdr = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr)
        sdr = ((const float*)(base + (size_t)3 * H * I / 2))[2 * I + row];
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int t = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, P, grp, p0 + j, t, rr[j]);
        }
        float ye[NT], yo[NT], hs[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) ye[j] = yo[j] = hs[j] = 0.f;
        if (base != nullptr) {
            for (int sc0 = 0; sc0 < CPU; sc0 += SUB) {
                const int ns = min(SUB, CPU - sc0);
                auto stage = [&]() {
#pragma unroll
                    for (int j = 0; j < NT; ++j)
                        if (j < nj) {
                            const float4* src =
                                (const float4*)(Hin + (size_t)rr[j] * I + (size_t)(c0 + sc0) * 32);
                            for (int i = lane; i < ns * 8; i += 64) {
                                const float4 v = src[i];
                                ((float4*)(hl + j * SUB * 32))[i] = v;
                                hs[j] += (v.x + v.y) + (v.z + v.w);
                            }
                        }
                    lds_wave_sync();
                };
                if (FMT == MOE_W_INT4_ROW) {
                    const int nbt = ns / UD;
                    uint4 ad4[UD];
                    if (nbt > 0) {
                        DN_LOAD(ad4, 0)
                    }
                    stage();  // overlaps the first batch's loads
                    for (int i = 0; i < nbt; ++i) {
                        if (i > 0) {
                            DN_LOAD(ad4, i)
                        }
                        DN_USE(ad4, i)
                    }
                    for (int c = nbt * UD; c < ns; ++c) {
                        const uint4 vd = bload16(rd, voff, (sc0 + c) * 1024);
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            if (j < nj) dot32(vd, hl + j * SUB * 32 + c * 32, ye[j], yo[j]);
                    }
                } else {
                    stage();
                    const uint32_t* ad = (const uint32_t*)(base + (size_t)3 * H * I / 2) +
                                         (size_t)2 * I * (H / 64) + (size_t)b * GI * 64 + lane;
                    for (int c = 0; c < ns; c += 2) {
                        const int gq = (c0 + sc0 + c) / 2;
                        const uint4 d0 = bload16(rd, voff, (sc0 + c) * 1024);
                        const uint4 d1 = bload16(rd, voff + 1024, (sc0 + c) * 1024);
                        const uint32_t pd = ad[(size_t)gq * 64];
                        const float sc = __uint_as_float(pd << 16);
                        const float mn = __uint_as_float(pd & 0xFFFF0000u);
#pragma unroll
                        for (int j = 0; j < NT; ++j)
                            if (j < nj) {
                                const float* hp = hl + j * SUB * 32 + c * 32;
                                const float sh = wave_sum(hp[lane]);
                                float ae = 0.f, ao = 0.f;
                                dot32(d0, hp, ae, ao);
                                dot32(d1, hp + 32, ae, ao);
                                ye[j] = fmaf(sc, fmaf(ao, 0.0625f, ae), fmaf(mn, sh, ye[j]));
                            }
                    }
                }
                lds_wave_sync();
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                float yp = ye[j];
                if (FMT == MOE_W_INT4_ROW)
                    yp = (fmaf(yo[j], 0.0625f, ye[j]) - 8.0f * wave_sum(hs[j])) * sdr;
                st_agent(f.dn_part + (((size_t)rr[j] * NB + b) * KS + q) * 64 + lane, yp);
            }
    }
    if (fused_combine && arrive_wave(&f.dn_ctr[b], (uint32_t)(n_groups * KS))) {
        const int T = f.T, K = f.K;
        for (int t = 0; t < T; ++t) {
            float m = 0.f;
            for (int s = 0; s < f.n_shared; ++s) {
                const int r = T * K + s * T + t;
                m += sum_slices(f.dn_part + ((size_t)r * NB + b) * KS * 64, KS, lane);
            }
            for (int k = 0; k < K; ++k) {
                const int r = t * K + k;
                m = fmaf(f.wts[r], sum_slices(f.dn_part + ((size_t)r * NB + b) * KS * 64, KS, lane),
                         m);
            }
            if (f.residual) m = f.x[(size_t)t * H + row] + m;
            f.out[(size_t)t * H + row] = m;
        }
    }
}

// Stand-alone combine for token counts where the fused one would be a long
// serial tail: one thread per output element, same fixed order.
__global__ void __launch_bounds__(256) k_combine(Fwd f)
{
    const int H = f.H, NB = H / 64, KS = f.dn_ks, T = f.T, K = f.K;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * H) return;
    const int t = (int)(idx / H), d = (int)(idx - (int64_t)t * H);
    const int b = d >> 6, lane = d & 63;
    float m = 0.f;
    for (int s = 0; s < f.n_shared; ++s) {
        const float* pp = f.dn_part + ((size_t)(T * K + s * T + t) * NB + b) * KS * 64 + lane;
        float y = 0.f;
        for (int q = 0; q < KS; ++q) y += pp[q * 64];
        m += y;
    }
    for (int k = 0; k < K; ++k) {
        const float* pp = f.dn_part + ((size_t)(t * K + k) * NB + b) * KS * 64 + lane;
        float y = 0.f;
        for (int q = 0; q < KS; ++q) y += pp[q * 64];
        m = fmaf(f.wts[t * K + k], y, m);
    }
    if (f.residual) m = f.x[idx] + m;
    f.out[idx] = m;
}

// ---------------------------------------------------------------------------
// launch: one wavefront-sized workgroup per unit
// ---------------------------------------------------------------------------

static int tokens_per_pass(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : 4; }

static int max_groups(const Fwd& f) { return f.n_shared + std::min(f.E, f.T * f.K); }

template <int FMT, int NT>
static hipError_t gu_launch(const Fwd& f, hipStream_t st)
{
    const int mg = max_groups(f);
    const unsigned grid = (unsigned)(mg * (f.I / 64) * f.gu_ks);
    hipLaunchKernelGGL((k_gu<FMT, NT>), dim3(grid), dim3(64), 0, st, f, f.x, f.groups, f.perm,
                       f.tok, f.n_groups, f.h, mg);
    return hipGetLastError();
}

template <int FMT, int NT>
static hipError_t dn_launch(const Fwd& f, hipStream_t st)
{
    const int mg = max_groups(f);
    const unsigned grid = (unsigned)(mg * (f.H / 64) * f.dn_ks);
    const int fused = f.T * (f.K + f.n_shared) * f.dn_ks <= 64;
    hipLaunchKernelGGL((k_dn<FMT, NT>), dim3(grid), dim3(64), 0, st, f, f.groups, f.perm, f.h,
                       f.n_groups, mg, fused);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && !fused) {
        const int64_t n = (int64_t)f.T * f.H;
        hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, f);
        e = hipGetLastError();
    }
    return e;
}

template <int FMT>
static hipError_t gu_dispatch(const Fwd& f, hipStream_t st)
{
    switch (tokens_per_pass(f.T)) {
    case 1: return gu_launch<FMT, 1>(f, st);
    case 2: return gu_launch<FMT, 2>(f, st);
    default: return gu_launch<FMT, 4>(f, st);
    }
}

template <int FMT>
static hipError_t dn_dispatch(const Fwd& f, hipStream_t st)
{
    switch (tokens_per_pass(f.T)) {
    case 1: return dn_launch<FMT, 1>(f, st);
    case 2: return dn_launch<FMT, 2>(f, st);
    default: return dn_launch<FMT, 4>(f, st);
    }
}

hipError_t launch_gateup_gemv(const Fwd& f, hipStream_t st)
{
    if (f.fmt == MOE_W_INT4_ROW) return gu_dispatch<MOE_W_INT4_ROW>(f, st);
    return gu_dispatch<MOE_W_INT4_AFFINE_G64>(f, st);
}

hipError_t launch_down_gemv(const Fwd& f, hipStream_t st)
{
    if (f.fmt == MOE_W_INT4_ROW) return dn_dispatch<MOE_W_INT4_ROW>(f, st);
    return dn_dispatch<MOE_W_INT4_AFFINE_G64>(f, st);
}

}  // namespace moe
