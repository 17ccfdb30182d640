// k_midt.hip -- the expert FFN for a few tokens (9 .. the grouped GEMM's
// threshold), row format, on the matrix cores.
//
// What is computed, cited by page title and section:
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11: each chosen
//     expert is SwiGLU on the rows routed to it (gate/up -> silu(g)*u ->
//     down), its output added with its routing weight; the batch's experts
//     are read once each; §15: verification runs a batch of 1 + g tokens.
//   GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6b-6d: the shared
//     expert always active, output = routed sum + shared.
//
// Why matrix cores here: the per-token GEMV spends 4 v_dot2 per 8 codes and
// token on top of the dequantisation, so with more tokens per expert it
// becomes bound by the vector ALU, not by HBM.  Here the codes are
// dequantised once (fp16 1024 + 16 n as in the GEMVs, formed in plain code:
// see nib_pairs_mfma) and the tokens ride in the N dimension of
// v_mfma_f32_16x16x32_f16 (16 tokens per pass over the codes).  Up to 8
// tokens the GEMVs measured as fast (their dot products are then cheap).
//
// Work decomposition: the GEMVs' unit (expert group, 64-row block, k-slice),
// one wavefront, streaming its slice in steps of 4 chunks (128 inputs) with
// a one-step rolling prefetch.  Lane l = (i = l % 16, g = l / 16): for
// row-group s (rows 16 s .. 16 s + 15 of the block) the lane loads the
// 16-byte piece of row 16 s + i in chunk 4 step + g (the slot layout keeps
// each 8-row group's pieces of a chunk in 128 contiguous bytes), and as the B
// operand the staged activations of token i of the pass in the same chunk
// (64 contiguous bytes).  Dword j of the piece (8 codes) with quad j of the
// activations is the lane's K-group of MFMA (s, j): K = 32 inputs per MFMA,
// in the activations' pair order on both sides.
//
// Activations are staged per token row (one power-of-two scale per row, as
// for the grouped GEMM), so one accumulator runs over the whole slice; the
// slice's activation sum per token, needed for the offset-binary correction
// (sum c x = acc / 16 - 72 sum x), comes from one more MFMA per K step with
// an all-ones A operand.  Partial sums of the k-slices go to the GEMVs'
// buffers and are reduced in a fixed order (the h finalize below, the
// combine kernel), so results are bitwise reproducible.
#include <algorithm>

#include "k_common.h"

namespace moe {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MT_N = 16;    // tokens per pass (the MFMA's N)
constexpr int MT_STEP = 4;  // chunks per rolling step

__device__ __forceinline__ uint32_t dwq(const uint4& v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

__device__ __forceinline__ half8 as_h8(const uint4& v) { return __builtin_bit_cast(half8, v); }

// Dword j of a 16-byte code piece as the fp16 A operand (1024 + 16 n, pair order).
__device__ __forceinline__ half8 codes_h8(const uint4& w, int j, uint32_t mv)
{
    uint32_t p0, p1, p2, p3;
    nib_pairs_mfma(dwq(w, j), mv, p0, p1, p2, p3);
    return as_h8(make_uint4(p0, p1, p2, p3));
}

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Token and h row of entry j of a group (per lane; tok_rows' layout: routed
// rows t K + k in token order, shared expert s rows T K + s T + t).
__device__ __forceinline__ void lane_rows(const Fwd& f, const Group& g, int j, int& t, int& r)
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

}  // namespace

// ---------------------------------------------------------------------------
// gate/up unit: (Wg x, Wu x) of one k-slice for up to 16 tokens per pass,
// times the row scales -> gpart[r][b][q][2][64] (unreduced; the h rows
// kernel sums the slices).  One step of codes and activations in flight
// (gate and up together already hold 196 VGPRs).
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(64) k_gum(Fwd f)
{
    __shared__ float s_sc[2][64];
    const int lane = threadIdx.x, i = lane & 15, g = lane >> 4;
    const int KS = f.gu_ks, H = f.H, I = f.I, NB = I / 64, C = H / 32;
    const int q = blockIdx.x % KS, b = (blockIdx.x / KS) % NB, gi = blockIdx.x / (KS * NB);
    if (gi >= uni(f.n_groups[0])) return;
    const Group grp = uni_group(f.groups, gi);
    const int CPU = C / KS, c0 = q * CPU, nst = CPU / MT_STEP;
    const uint8_t* base = grp.base;
    const uint8_t* anchor = (const uint8_t*)f.x;  // any valid address (empty resources)
    const uint32_t mbytes = base ? (uint32_t)C * 1024 : 0u;
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(base ? base + (size_t)b * C * 1024 : anchor, mbytes);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base ? base + (size_t)I * H / 2 + (size_t)b * C * 1024 : anchor, mbytes);
    // the block's row scales, in registers until the first epilogue puts
    // them in LDS (each lane then needs 16 rows of them)
    const float* tab = (const float*)(base ? base + (size_t)3 * H * I / 2 : anchor);
    const float sgl = base ? tab[b * 64 + lane] : 0.f, sul = base ? tab[I + b * 64 + lane] : 0.f;
    const half8 ones = as_h8(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
    const uint32_t mv = f.magic;
    // row-group s: row 16 s + i of chunk 4 step + g
    uint32_t voff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) voff[s] = blk_off(16 * s + i, C, c0 + g);
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += MT_N) {
        const int nj = min(MT_N, grp.cnt - p0);
        int tt, rr;
        lane_rows(f, grp, p0 + min(i, nj - 1), tt, rr);
        const uint4* xr = f.xq + (size_t)tt * (H / 8) + (size_t)(c0 + g) * 4;
        f32x4 dg[4], du[4], ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) dg[s] = du[s] = ds;
        if (base) {
            uint4 A[4], B[4], X[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                A[s] = bload16(rg, voff[s], 0);
                B[s] = bload16(ru, voff[s], 0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) X[j] = xr[j];
            // the last step's loads re-read its own activations and read
            // zeros past the slice (codes)
#pragma unroll 1
            for (int st = 0; st < nst; ++st) {
                uint4 a[4], bb[4], x[4];
                const int sn = st + 1;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    a[s] = A[s];
                    bb[s] = B[s];
                    A[s] = bload16(rg, voff[s], (uint32_t)(sn * MT_STEP) * 128);
                    B[s] = bload16(ru, voff[s], (uint32_t)(sn * MT_STEP) * 128);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = X[j];
                    X[j] = xr[min(sn, nst - 1) * MT_STEP * 4 + j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half8 xb = as_h8(x[j]);
                    ds = mfma16(ones, xb, ds);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        dg[s] = mfma16(codes_h8(a[s], j, mv), xb, dg[s]);
                        du[s] = mfma16(codes_h8(bb[s], j, mv), xb, du[s]);
                    }
                }
            }
        }
        if (p0 == 0) {
            s_sc[0][lane] = sgl;
            s_sc[1][lane] = sul;
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wavefront's LDS writes done
            __builtin_amdgcn_wave_barrier();
        }
        // D entry (lane, e): row 16 s + 4 g + e, token i of the pass
        if (i < nj) {
            const float sx = f.xrow[tt].x, corr = -72.f * ds[0];
            float* o = f.gpart + (((size_t)rr * NB + b) * KS + q) * 128;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r0 = 16 * s + 4 * g;
                float4 vg, vu;
                vg.x = fmaf(dg[s][0], 0.0625f, corr) * sx * s_sc[0][r0];
                vg.y = fmaf(dg[s][1], 0.0625f, corr) * sx * s_sc[0][r0 + 1];
                vg.z = fmaf(dg[s][2], 0.0625f, corr) * sx * s_sc[0][r0 + 2];
                vg.w = fmaf(dg[s][3], 0.0625f, corr) * sx * s_sc[0][r0 + 3];
                vu.x = fmaf(du[s][0], 0.0625f, corr) * sx * s_sc[1][r0];
                vu.y = fmaf(du[s][1], 0.0625f, corr) * sx * s_sc[1][r0 + 1];
                vu.z = fmaf(du[s][2], 0.0625f, corr) * sx * s_sc[1][r0 + 2];
                vu.w = fmaf(du[s][3], 0.0625f, corr) * sx * s_sc[1][r0 + 3];
                if (!base) vg = vu = make_float4(0.f, 0.f, 0.f, 0.f);
                *(float4*)(o + r0) = vg;
                *(float4*)(o + 64 + r0) = vu;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// down unit: (Wd h) of one k-slice for up to 16 tokens per pass, times the
// row scale -> ypart[r][b][q][64] (the combine sums slices and experts)
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(64) k_dnm(Fwd f)
{
    __shared__ float s_sc[64];
    const int lane = threadIdx.x, i = lane & 15, g = lane >> 4;
    const int KS = f.dn_ks, H = f.H, I = f.I, NB = H / 64, C = I / 32;
    const int q = blockIdx.x % KS, b = (blockIdx.x / KS) % NB, gi = blockIdx.x / (KS * NB);
    if (gi >= uni(f.n_groups[0])) return;
    const Group grp = uni_group(f.groups, gi);
    const int CPU = C / KS, c0 = q * CPU, nst = CPU / MT_STEP;
    const uint8_t* base = grp.base;
    const uint8_t* anchor = (const uint8_t*)f.x;
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(base ? base + (size_t)I * H + (size_t)b * C * 1024 : anchor,
                  base ? (uint32_t)C * 1024 : 0u);
    const float sdl =
        base ? ((const float*)(base + (size_t)3 * H * I / 2))[2 * I + b * 64 + lane] : 0.f;
    const half8 ones = as_h8(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u));
    const uint32_t mv = f.magic;
    uint32_t voff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) voff[s] = blk_off(16 * s + i, C, c0 + g);
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += MT_N) {
        const int nj = min(MT_N, grp.cnt - p0);
        int tt, rr;
        lane_rows(f, grp, p0 + min(i, nj - 1), tt, rr);
        const uint4* hr = f.hq + (size_t)rr * (I / 8) + (size_t)(c0 + g) * 4;
        f32x4 dy[4], ds = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) dy[s] = ds;
        if (base) {
            uint4 D[4], X[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) D[s] = bload16(rd, voff[s], 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) X[j] = hr[j];
#pragma unroll 1
            for (int st = 0; st < nst; ++st) {
                uint4 w[4], x[4];
                const int sn = st + 1;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    w[s] = D[s];
                    D[s] = bload16(rd, voff[s], (uint32_t)(sn * MT_STEP) * 128);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = X[j];
                    X[j] = hr[min(sn, nst - 1) * MT_STEP * 4 + j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half8 xb = as_h8(x[j]);
                    ds = mfma16(ones, xb, ds);
#pragma unroll
                    for (int s = 0; s < 4; ++s) dy[s] = mfma16(codes_h8(w[s], j, mv), xb, dy[s]);
                }
            }
        }
        if (p0 == 0) {
            s_sc[lane] = sdl;
            __builtin_amdgcn_s_waitcnt(0xC07F);
            __builtin_amdgcn_wave_barrier();
        }
        if (i < nj) {
            const float sx = f.hrow[rr].x, corr = -72.f * ds[0];
            float* o = f.ypart + (((size_t)rr * NB + b) * KS + q) * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r0 = 16 * s + 4 * g;
                float4 v;
                v.x = fmaf(dy[s][0], 0.0625f, corr) * sx * s_sc[r0];
                v.y = fmaf(dy[s][1], 0.0625f, corr) * sx * s_sc[r0 + 1];
                v.z = fmaf(dy[s][2], 0.0625f, corr) * sx * s_sc[r0 + 2];
                v.w = fmaf(dy[s][3], 0.0625f, corr) * sx * s_sc[r0 + 3];
                if (!base) v = make_float4(0.f, 0.f, 0.f, 0.f);
                *(float4*)(o + r0) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// h rows: a workgroup per row r of h.  Wavefront w takes the 64-row blocks
// w, w + 4, ...: it sums each block's k-slices in slice order (all slices'
// loads in flight together), h = silu(g rs) (u rs) (rs: the token's RMSNorm
// factor) into LDS; then wavefront 0 stages the whole row as fp16 with one
// power-of-two scale (pair order, (2^-k, sum)) for the down units.
// ---------------------------------------------------------------------------

constexpr int HR_MAXKS = 16;

template <int NG>
__global__ void __launch_bounds__(256) k_hrows(Fwd f)
{
    extern __shared__ float4 hl4[];
    float* hl = (float*)hl4;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, r = blockIdx.x;
    const int KS = f.gu_ks, I = f.I, NB = I / 64, TK = f.T * f.K;
    const int t = r < TK ? r / f.K : (r - TK) % f.T;
    const float rs = f.tok[t].rscale;
    const float* gp = f.gpart + (size_t)r * NB * KS * 128;
#pragma unroll 1
    for (int b = w; b < NB; b += 4) {
        float gv[HR_MAXKS], uv[HR_MAXKS];
#pragma unroll
        for (int q = 0; q < HR_MAXKS; ++q) {
            const int qc = min(q, KS - 1);
            gv[q] = gp[((size_t)b * KS + qc) * 128 + lane];
            uv[q] = gp[((size_t)b * KS + qc) * 128 + 64 + lane];
        }
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int q = 0; q < HR_MAXKS; ++q)
            if (q < KS) {
                gs += gv[q];
                us += uv[q];
            }
        const float gg = gs * rs, uu = us * rs;
        hl[b * 64 + lane] = gg / (1.0f + expf(-gg)) * uu;
    }
    __syncthreads();
    if (w == 0) {
        float sum, ss;
        stage_row<NG>(hl, I, lane, f.hq + (size_t)r * (I / 8), f.hrow + r, sum, ss);
    }
}

// ---------------------------------------------------------------------------
// plan and launch
// ---------------------------------------------------------------------------

namespace {

// k-slices: each slice a whole number of 4-chunk steps; the smallest count
// that gives about 3,072 units over every possible group, within the
// partial buffer (longer units measured faster than short ones here: a
// few-token batch activates about half the groups).
int midt_ks(int chunks, int blocks, int max_ks, size_t part_need_per_ks, size_t part_bytes)
{
    static const int cand[] = {1, 2, 3, 4, 6, 8, 12, 16};
    int best = 1;
    for (int ks : cand) {
        if (ks > max_ks) break;
        if (chunks % ks != 0 || (chunks / ks) % MT_STEP != 0) continue;
        if (ks > 1 && part_need_per_ks * ks > part_bytes) break;
        best = ks;
        if ((int64_t)blocks * ks >= 3072) break;
    }
    return best;
}

}  // namespace

// The few-token matrix-core path: row format, at least 2 tokens, no int8
// shared expert (its GEMV branch stays), rows short enough for one-pass row
// staging (H, I <= 8192), and the row-staging buffers present.
bool midt_ok(const Fwd& f)
{
    return f.T >= MIDT_MIN_T && f.fmt == MOE_W_INT4_ROW && !shared_int8(f) && f.H <= 8192 &&
           f.I <= 8192 && f.xrow != nullptr && f.hrow != nullptr;
}

void midt_plan(Fwd& f, size_t gpart_bytes, size_t ypart_bytes)
{
    const int max_groups = f.n_shared + std::min(f.E, f.T * f.K);
    const size_t rows = (size_t)f.T * (f.K + f.n_shared);
    f.gu_ks = midt_ks(f.H / 32, max_groups * (f.I / 64), 16, rows * f.I * 2 * 4, gpart_bytes);
    f.dn_ks = midt_ks(f.I / 32, max_groups * (f.H / 64), 4, rows * f.H * 4, ypart_bytes);
}

hipError_t launch_midt_gateup(const Fwd& f, hipStream_t st)
{
    const int max_groups = f.n_shared + std::min(f.E, f.T * f.K);
    const unsigned units = (unsigned)(max_groups * (f.I / 64) * f.gu_ks);
    return launch_k(k_gum, dim3(units), dim3(64), 0, st, f);
}

hipError_t launch_midt_hrows(const Fwd& f, hipStream_t st)
{
    const unsigned rows = (unsigned)(f.T * (f.K + f.n_shared));
    const int ng = (f.I + 511) / 512;
    const size_t lds = (size_t)f.I * 4;
    auto go = [&](auto kern) {
        if (lds > 65536) {
            const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
        }
        return launch_k(kern, dim3(rows), dim3(256), lds, st, f);
    };
    if (ng <= 1) return go(k_hrows<1>);
    if (ng <= 2) return go(k_hrows<2>);
    if (ng <= 4) return go(k_hrows<4>);
    if (ng <= 8) return go(k_hrows<8>);
    if (ng <= 12) return go(k_hrows<12>);
    return go(k_hrows<16>);
}

hipError_t launch_midt_down(const Fwd& f, hipStream_t st)
{
    const int max_groups = f.n_shared + std::min(f.E, f.T * f.K);
    const unsigned units = (unsigned)(max_groups * (f.H / 64) * f.dn_ks);
    return launch_k(k_dnm, dim3(units), dim3(64), 0, st, f);
}

}  // namespace moe
