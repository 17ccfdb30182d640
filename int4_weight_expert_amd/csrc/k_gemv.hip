// k_gemv.hip -- the int4 expert GEMVs of the decode-size forward.
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
// Work decomposition.  A unit is (expert group g, 64-row block b, k-slice q)
// and is one wavefront, a workgroup of its own, so the hardware dispatcher
// spreads the weight stream evenly over every SIMD whatever the routing.
// The unit streams its slice's 16-byte chunks of the 64 rows (lane = row,
// 1 KiB coalesced buffer loads, see the slot layout) with a rolling
// prefetch: each chunk register is refilled with the chunk one step ahead
// as soon as it is consumed.  The slice's activations (fp16 spans staged by
// the router or by the gate/up finalize) are copied into the wavefront's
// LDS once per pass and read with wave-uniform (broadcast) ds_read_b128.
// Partial sums of the k-slices go to a small buffer; a finalize kernel
// (gate/up: h = silu(g) * u, staged as fp16 spans for the down projection)
// or the combine kernel (down: weighted sum over experts, residual) reduces
// them in a fixed order, so results are bitwise reproducible.  With a single
// k-slice the unit writes its result directly.
//
// Arithmetic per 8 codes and token: 3 shifts, 4 bit-field inserts (codes ->
// fp16 1024 + 16 n, shared by the tokens of a pass) and 4 v_dot2_f32_f16;
// per span of 64 inputs the fp32 sum is corrected with the span's stored
// activation sum and rescaled (see k_common.h).
#include "k_common.h"

namespace moe {

constexpr int UG = 2;  // chunks per rolling step, gate/up (x2 matrices)
constexpr int UD = 4;  // chunks per rolling step, down

__device__ __forceinline__ void lds_wave_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int d)
{
    return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// One dword of codes (8 inputs) against activation pair quad xv.
__device__ __forceinline__ float dot_dword(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                           const uint4& xv, float acc)
{
    acc = dot2(p0, xv.x, acc);
    acc = dot2(p1, xv.y, acc);
    acc = dot2(p2, xv.z, acc);
    acc = dot2(p3, xv.w, acc);
    return acc;
}

// Chunk ck of the slice (4 dwords, 32 codes) of one matrix against the
// tokens of the pass; xq = LDS activations [NT][CPU*4] uint4.
template <int NT>
__device__ __forceinline__ void chunk1(const uint4& w, const uint4* xq, int cpu4, int ck, int nj,
                                       uint32_t mv, float (&acc)[NT])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t p0, p1, p2, p3;
        nib_pairs(dw(w, d), mv, p0, p1, p2, p3);
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) acc[j] = dot_dword(p0, p1, p2, p3, xq[j * cpu4 + ck * 4 + d], acc[j]);
    }
}

// Same for two matrices sharing the activations (gate and up).
template <int NT>
__device__ __forceinline__ void chunk2(const uint4& wa, const uint4& wb, const uint4* xq,
                                       int cpu4, int ck, int nj, uint32_t mv, float (&aa)[NT],
                                       float (&ab)[NT])
{
    if (NT == 1) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
            nib_pairs(dw(wa, d), mv, a0, a1, a2, a3);
            nib_pairs(dw(wb, d), mv, b0, b1, b2, b3);
            const uint4 xv = xq[ck * 4 + d];
            aa[0] = dot_dword(a0, a1, a2, a3, xv, aa[0]);
            ab[0] = dot_dword(b0, b1, b2, b3, xv, ab[0]);
        }
        return;
    }
    // several tokens: the chunk's codes dequantised once, then per token its
    // four activation vectors read together (one LDS wait per token and chunk;
    // the down projection's single matrix does better with the per-dword order)
    uint32_t pa[16], pb[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        nib_pairs(dw(wa, d), mv, pa[4 * d], pa[4 * d + 1], pa[4 * d + 2], pa[4 * d + 3]);
        nib_pairs(dw(wb, d), mv, pb[4 * d], pb[4 * d + 1], pb[4 * d + 2], pb[4 * d + 3]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
        if (j < nj) {
            const uint4* xj = xq + j * cpu4 + ck * 4;
            const uint4 x0 = xj[0], x1 = xj[1], x2 = xj[2], x3 = xj[3];
            float a = aa[j], bb = ab[j];
            a = dot_dword(pa[0], pa[1], pa[2], pa[3], x0, a);
            bb = dot_dword(pb[0], pb[1], pb[2], pb[3], x0, bb);
            a = dot_dword(pa[4], pa[5], pa[6], pa[7], x1, a);
            bb = dot_dword(pb[4], pb[5], pb[6], pb[7], x1, bb);
            a = dot_dword(pa[8], pa[9], pa[10], pa[11], x2, a);
            bb = dot_dword(pb[8], pb[9], pb[10], pb[11], x2, bb);
            aa[j] = dot_dword(pa[12], pa[13], pa[14], pa[15], x3, a);
            ab[j] = dot_dword(pb[12], pb[13], pb[14], pb[15], x3, bb);
        }
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// End of a span of 64 inputs: fold the span accumulator `a` into `tot`.
// Row format (codes stored c + 8): sum c x = a/16 - 72 S.  Affine (w = sc q
// + mn): sum w x = sc a/16 + (mn - 64 sc) S.  Then rescale by the span's 2^-k.
template <int FMT>
__device__ __forceinline__ float fold(float tot, float a, float2 span, uint32_t affine_pair)
{
    float v;
    if (FMT == MOE_W_INT4_ROW) {
        v = fmaf(a, 0.0625f, -72.f * span.y);
    } else {
        const float sc = bf16_lo(affine_pair), mn = bf16_hi(affine_pair);
        v = fmaf(sc * 0.0625f, a, (mn - 64.f * sc) * span.y);
    }
    return fmaf(v, span.x, tot);
}

// Copies the slice's staged activations of the pass's tokens into LDS:
// xq [NT][CPU*4] uint4 then xs [NT][CPU/2] float2.  BATCH: for slices of
// up to 16 chunks, every token's loads first, then the stores (the int8
// units, which hold more codes in flight, keep the loop form: the batch
// would push them past 128 VGPRs).
template <int NT, bool BATCH = true>
__device__ __forceinline__ void copy_slice(const uint4* __restrict__ gq,
                                           const float2* __restrict__ gs, const int (&src)[NT],
                                           int nj, int row_q, int row_s, int c0, int CPU,
                                           int lane, uint4* xq, float2* xs)
{
    if (BATCH && CPU <= 16) {
        // one vector and one span scale per lane and token: every token's
        // loads issue together (indices clamped, absent tokens read token 0),
        // then the stores
        const int i = min(lane, CPU * 4 - 1), k = min(lane, CPU / 2 - 1);
        uint4 vq[NT];
        float2 vs[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int sj = j < nj ? src[j] : src[0];
            vq[j] = gq[(size_t)sj * row_q + (size_t)c0 * 4 + i];
            vs[j] = gs[(size_t)sj * row_s + c0 / 2 + k];
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                if (lane < CPU * 4) xq[j * CPU * 4 + lane] = vq[j];
                if (lane < CPU / 2) xs[j * (CPU / 2) + lane] = vs[j];
            }
        lds_wave_sync();
        return;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
        if (j < nj) {
            const uint4* sq = gq + (size_t)src[j] * row_q + (size_t)c0 * 4;
            const float2* ss = gs + (size_t)src[j] * row_s + c0 / 2;
            for (int i = lane; i < CPU * 4; i += 64) xq[j * CPU * 4 + i] = sq[i];
            for (int i = lane; i < CPU / 2; i += 64) xs[j * (CPU / 2) + i] = ss[i];
        }
    lds_wave_sync();
}

// The slice's h of one row from fp32 (the one-token gate/up kernel's
// output) into LDS as fp16 spans, as the gate/up finalize stages it: per span
// of 64 inputs a power of two that puts its largest magnitude in [2^13,
// 2^14), pair order, (2^-k, sum of the fp16 values).  Lane g takes inputs
// 8g..8g+7 of the slice; a span's 8 lanes agree on its scale.
__device__ __forceinline__ void stage_slice_f32(const float* __restrict__ hrow, int c0, int CPU,
                                                int lane, uint4* xq, float2* xs)
{
    const int n8 = CPU * 4;
    const float4* h4 = (const float4*)(hrow + (size_t)c0 * 32);
    for (int g0 = 0; g0 < n8; g0 += 64) {
        const int g = g0 + lane, gc = min(g, n8 - 1);
        const float4 a = h4[2 * gc], b = h4[2 * gc + 1];
        float m = fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                        fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
        m = fmaxf(m, __shfl_xor(m, 1));
        m = fmaxf(m, __shfl_xor(m, 2));
        m = fmaxf(m, __shfl_xor(m, 4));
        int e;
        frexpf(m, &e);
        e = max(e, -100);
        const float sc = ldexpf(1.0f, 14 - e);
        const _Float16 h0 = (_Float16)(a.x * sc), h1 = (_Float16)(a.y * sc);
        const _Float16 h2 = (_Float16)(a.z * sc), h3 = (_Float16)(a.w * sc);
        const _Float16 h4v = (_Float16)(b.x * sc), h5 = (_Float16)(b.y * sc);
        const _Float16 h6 = (_Float16)(b.z * sc), h7 = (_Float16)(b.w * sc);
        float t = (((float)h0 + (float)h1) + ((float)h2 + (float)h3)) +
                  (((float)h4v + (float)h5) + ((float)h6 + (float)h7));
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        if (g < n8) {
            xq[g] = make_uint4(pack_h2(h0, h4v), pack_h2(h1, h5), pack_h2(h2, h6), pack_h2(h3, h7));
            if ((g & 7) == 0) xs[g >> 3] = make_float2(ldexpf(1.0f, e - 14), t);
        }
    }
    lds_wave_sync();
}

__device__ __forceinline__ void unit_coords(int u, int KS, int NB, int& q, int& b, int& gi)
{
    q = u % KS;
    b = (u / KS) % NB;
    gi = u / (KS * NB);
}

// ---------------------------------------------------------------------------
// Per-row int8 shared experts ("惊呆了！…" §05 quantize_rows with bits = 8,
// the dense precision of the converted model, §06-07).  The slot holds each
// matrix [O][In] as 64-row blocks of 16-input chunks, ((b * In/16 + c) * 64 +
// lane) * 16, codes offset binary (q + 128).  A unit is the int4 kernels'
// unit (group, 64-row block, k-slice, with the same k-slice count and the
// same partial layout), taken as a branch of the int4 GEMV launch for groups
// 0 .. n_shared - 1, so the finalize and the combine are shared.  A code
// byte n becomes the fp16 1024 + n (v_perm_b32 then an OR), in the staged
// activations' pair order; per span of 64 inputs sum q x = acc - 1152 S.
// ---------------------------------------------------------------------------

// Bytes i and 4 + i of an 8-byte group as the fp16 pair (1024 + b_i, 1024 + b_{4+i}).
__device__ __forceinline__ uint32_t byte_pair(uint32_t lo, uint32_t hi, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
}

// One 16-input chunk (4 dwords of codes) against activation quads 2c, 2c+1.
__device__ __forceinline__ float dot_chunk8(const uint4& w, const uint4& x0, const uint4& x1,
                                            float acc)
{
    acc = dot_dword(byte_pair(w.x, w.y, 0x0C040C00u), byte_pair(w.x, w.y, 0x0C050C01u),
                    byte_pair(w.x, w.y, 0x0C060C02u), byte_pair(w.x, w.y, 0x0C070C03u), x0, acc);
    acc = dot_dword(byte_pair(w.z, w.w, 0x0C040C00u), byte_pair(w.z, w.w, 0x0C050C01u),
                    byte_pair(w.z, w.w, 0x0C060C02u), byte_pair(w.z, w.w, 0x0C070C03u), x1, acc);
    return acc;
}

__device__ __forceinline__ float fold8(float tot, float a, float2 span)
{
    return fmaf(a - 1152.f * span.y, span.x, tot);
}

template <int NT>
__device__ __forceinline__ void gu8_unit(const Fwd& f, int q, int b, int gi, uint4* lds4)
{
    const int lane = threadIdx.x;
    const int KS = f.gu_ks, H = f.H, I = f.I, NB = I / 64;
    const int CPU4 = H / 32 / KS;               // the int4 slice: its activations
    const int C8 = H / 16, CPU8 = 2 * CPU4;     // 16-input chunks of the row and of the slice
    const Group grp = uni_group(f.groups, gi);
    const int c0 = q * CPU8, row = b * 64 + lane, nsp = CPU8 / 4;
    uint4* xq = lds4;
    float2* xs = (float2*)(lds4 + NT * CPU4 * 4);
    const uint8_t* base = grp.base;
    const uint32_t voff = (uint32_t)lane * 16;
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc(base + ((size_t)b * C8 + c0) * 1024, (uint32_t)CPU8 * 1024);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base + (size_t)I * H + ((size_t)b * C8 + c0) * 1024, (uint32_t)CPU8 * 1024);
    const float* tab = (const float*)(base + (size_t)3 * H * I);
    const float sgr = tab[row], sur = tab[I + row];
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int tt[NT], rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            tt[j] = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, f.perm, grp, p0 + j, tt[j], rr[j]);
        }
        float Gt[NT], Ut[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) Gt[j] = Ut[j] = 0.f;
        uint4 A[4], B[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            A[k] = bload16(rg, voff + k * 1024, 0);
            B[k] = bload16(ru, voff + k * 1024, 0);
        }
        copy_slice<NT, false>(f.xq, f.xsc, tt, nj, H / 8, H / 64, q * CPU4, CPU4, lane, xq, xs);
#pragma unroll 1
        for (int sp = 0; sp < nsp; ++sp) {
            float ag[NT], au[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) ag[j] = au[j] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 wa = A[k], wb = B[k];
                // the same chunk of the next span (a load past the slice returns zeros)
                A[k] = bload16(rg, voff + k * 1024, (uint32_t)(sp + 1) * 4096);
                B[k] = bload16(ru, voff + k * 1024, (uint32_t)(sp + 1) * 4096);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
                        const uint4* xj = xq + j * CPU4 * 4 + sp * 8 + 2 * k;
                        ag[j] = dot_chunk8(wa, xj[0], xj[1], ag[j]);
                        au[j] = dot_chunk8(wb, xj[0], xj[1], au[j]);
                    }
            }
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (j < nj) {
                    const float2 span = xs[j * (CPU4 / 2) + sp];
                    Gt[j] = fold8(Gt[j], ag[j], span);
                    Ut[j] = fold8(Ut[j], au[j], span);
                }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                const float g = Gt[j] * sgr, u = Ut[j] * sur;
                if (KS == 1) {
                    const float rs = f.tok[tt[j]].rscale;
                    const float gg = g * rs, uu = u * rs;
                    stage_span64(gg / (1.0f + expf(-gg)) * uu, lane,
                                 (uint16_t*)(f.hq + (size_t)rr[j] * (I / 8) + b * 8),
                                 f.hsc + (size_t)rr[j] * (I / 64) + b);
                } else {
                    float* o = f.gpart + (((size_t)rr[j] * NB + b) * KS + q) * 128;
                    o[lane] = g;
                    o[64 + lane] = u;
                }
            }
        lds_wave_sync();
    }
}

template <int NT>
__device__ __forceinline__ void dn8_unit(const Fwd& f, int q, int b, int gi, uint4* lds4)
{
    const int lane = threadIdx.x;
    const int KS = f.dn_ks, H = f.H, I = f.I, NB = H / 64;
    const int CPU4 = I / 32 / KS, C8 = I / 16, CPU8 = 2 * CPU4;
    const Group grp = uni_group(f.groups, gi);
    const int c0 = q * CPU8, row = b * 64 + lane, nsp = CPU8 / 4;
    uint4* xq = lds4;
    float2* xs = (float2*)(lds4 + NT * CPU4 * 4);
    const uint8_t* base = grp.base;
    const uint32_t voff = (uint32_t)lane * 16;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(
        base + (size_t)2 * I * H + ((size_t)b * C8 + c0) * 1024, (uint32_t)CPU8 * 1024);
    const float sdr = ((const float*)(base + (size_t)3 * H * I))[2 * I + row];
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int t = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, f.perm, grp, p0 + j, t, rr[j]);
        }
        float Yt[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) Yt[j] = 0.f;
        uint4 D[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) D[k] = bload16(rd, voff + k * 1024, 0);
        copy_slice<NT, false>(f.hq, f.hsc, rr, nj, I / 8, I / 64, q * CPU4, CPU4, lane, xq, xs);
#pragma unroll 1
        for (int sp = 0; sp < nsp; ++sp) {
            float a[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) a[j] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 wd = D[k];
                D[k] = bload16(rd, voff + k * 1024, (uint32_t)(sp + 1) * 4096);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    if (j < nj) {
                        const uint4* xj = xq + j * CPU4 * 4 + sp * 8 + 2 * k;
                        a[j] = dot_chunk8(wd, xj[0], xj[1], a[j]);
                    }
            }
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (j < nj) Yt[j] = fold8(Yt[j], a[j], xs[j * (CPU4 / 2) + sp]);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) f.ypart[(((size_t)rr[j] * NB + b) * KS + q) * 64 + lane] = Yt[j] * sdr;
        lds_wave_sync();
    }
}

// ---------------------------------------------------------------------------
// gate/up unit: partial (sg (Wg x)_row, su (Wu x)_row) of one k-slice for the
// group's tokens -> gpart[r][b][q][2][64]; with one k-slice, h directly.
// ---------------------------------------------------------------------------

template <int FMT, int NT, bool S8>
__global__ void __launch_bounds__(64) k_gu(Fwd f)
{
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x;
    const int KS = f.gu_ks, H = f.H, I = f.I, NB = I / 64, C = H / 32, G = H / 64;
    int q, b, gi;
    unit_coords(blockIdx.x, KS, NB, q, b, gi);
    if (gi >= uni(f.n_groups[0])) return;
    if (S8 && gi < f.n_shared) {  // int8 shared expert (groups 0 .. n_shared - 1)
        gu8_unit<NT>(f, q, b, gi, lds4);
        return;
    }
    const Group grp = uni_group(f.groups, gi);
    const int CPU = C / KS, c0 = q * CPU, row = b * 64 + lane;
    uint4* xq = lds4;
    float2* xs = (float2*)(lds4 + NT * CPU * 4);
    const uint8_t* base = grp.base;
    // the lane's row in the block: its piece of chunk c0 + j at voff + 128 j
    const uint32_t voff = blk_off(lane, C, c0), toff = tab_off(lane, G, 0);
    const uint32_t mv = magic_vgpr();
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(base + (size_t)b * C * 1024, (uint32_t)C * 1024);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base + (size_t)I * H / 2 + (size_t)b * C * 1024, (uint32_t)C * 1024);
    // row format: fp32 row scales after the codes; affine: (scale, min) bf16
    // pair per row and 64-input group, in 8-row groups per matrix
    const uint8_t* tab = base + (size_t)3 * H * I / 2;
    const __amdgpu_buffer_rsrc_t rtg = make_rsrc(tab + (size_t)b * G * 256, (uint32_t)G * 256);
    const __amdgpu_buffer_rsrc_t rtu =
        make_rsrc(tab + ((size_t)I * G + (size_t)b * G * 64) * 4, (uint32_t)G * 256);
    float sgr = 1.f, sur = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr) {
        sgr = ((const float*)tab)[row];
        sur = ((const float*)tab)[I + row];
    }
    const int nst = CPU / UG;
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int tt[NT], rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            tt[j] = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, f.perm, grp, p0 + j, tt[j], rr[j]);
        }
        float Gt[NT], Ut[NT], ag[NT], au[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) Gt[j] = Ut[j] = ag[j] = au[j] = 0.f;
        if (base != nullptr) {
            uint4 A[UG], B[UG];
            uint32_t PA = 0, PB = 0;
#pragma unroll
            for (int k = 0; k < UG; ++k) {
                A[k] = bload16(rg, voff + k * 128, 0);
                B[k] = bload16(ru, voff + k * 128, 0);
            }
            if (FMT != MOE_W_INT4_ROW) {
                PA = bload4(rtg, toff, (uint32_t)(c0 / 2) * 32);
                PB = bload4(rtu, toff, (uint32_t)(c0 / 2) * 32);
            }
            copy_slice<NT>(f.xq, f.xsc, tt, nj, H / 8, H / 64, c0, CPU, lane, xq, xs);
            // one rolling step = one span (2 chunks); the last step loads nothing
#define GU_STEP(I_, LOAD_)                                                               \
    {                                                                                    \
        const uint32_t pa = PA, pb = PB;                                                 \
        _Pragma("unroll") for (int k = 0; k < UG; ++k)                                    \
        {                                                                                \
            const uint4 wa = A[k], wb = B[k];                                            \
            if (LOAD_) {                                                                 \
                A[k] = bload16(rg, voff + k * 128, ((I_) + 1) * UG * 128);             \
                B[k] = bload16(ru, voff + k * 128, ((I_) + 1) * UG * 128);             \
            }                                                                            \
            chunk2<NT>(wa, wb, xq, CPU * 4, (I_) * UG + k, nj, mv, ag, au);               \
        }                                                                                \
        if (FMT != MOE_W_INT4_ROW && (LOAD_)) {                                          \
            PA = bload4(rtg, toff, (uint32_t)(c0 / 2 + (I_) + 1) * 32);                 \
            PB = bload4(rtu, toff, (uint32_t)(c0 / 2 + (I_) + 1) * 32);                 \
        }                                                                                \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) if (j < nj)                       \
        {                                                                                \
            const float2 sp = xs[j * (CPU / 2) + (I_)];                                  \
            Gt[j] = fold<FMT>(Gt[j], ag[j], sp, pa);                                     \
            Ut[j] = fold<FMT>(Ut[j], au[j], sp, pb);                                     \
            ag[j] = au[j] = 0.f;                                                         \
        }                                                                                \
    }
#pragma unroll 1
            for (int i = 0; i < nst - 1; ++i) GU_STEP(i, true)
            GU_STEP(nst - 1, false)
#undef GU_STEP
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                const float g = Gt[j] * sgr, u = Ut[j] * sur;
                if (KS == 1) {
                    const float rs = f.tok[tt[j]].rscale;
                    const float gg = g * rs, uu = u * rs;
                    stage_span64(gg / (1.0f + expf(-gg)) * uu, lane,
                                 (uint16_t*)(f.hq + (size_t)rr[j] * (I / 8) + b * 8),
                                 f.hsc + (size_t)rr[j] * (I / 64) + b);
                } else {
                    float* o = f.gpart + (((size_t)rr[j] * NB + b) * KS + q) * 128;
                    o[lane] = g;
                    o[64 + lane] = u;
                }
            }
        lds_wave_sync();
    }
}

// One workgroup per (group, 64-row block), for layers with few of them (each
// then gets a CU of its own): wavefront q streams k-slice q exactly as a
// k_gu unit does, the slices' (sg Wg x, su Wu x) meet in LDS and are summed
// in slice order (the finalize kernel's order, so h is bit-identical), and
// token j's h is staged by wavefront j mod KS.  No partials leave the
// workgroup and no finalize kernel follows.
__host__ __device__ constexpr int gemv_wave_lds_u4(int CPU, int nt) { return (nt * CPU * 68 + 15) / 16; }

template <int FMT, int NT>
__global__ void __launch_bounds__(1024) k_gu_wg(Fwd f)
{
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x & 63, q = uni((int)(threadIdx.x >> 6));
    const int KS = f.gu_ks, H = f.H, I = f.I, NB = I / 64, C = H / 32, G = H / 64;
    const int b = blockIdx.x % NB, gi = blockIdx.x / NB;
    if (gi >= uni(f.n_groups[0])) return;
    const Group grp = uni_group(f.groups, gi);
    const int CPU = C / KS, c0 = q * CPU, row = b * 64 + lane;
    const int wl = gemv_wave_lds_u4(CPU, NT);
    uint4* xq = lds4 + q * wl;
    float2* xs = (float2*)(xq + NT * CPU * 4);
    float* red = (float*)(lds4 + KS * wl);  // [KS][NT][2][64]
    const uint8_t* base = grp.base;
    // the lane's row in the block: its piece of chunk c0 + j at voff + 128 j
    const uint32_t voff = blk_off(lane, C, c0), toff = tab_off(lane, G, 0);
    const uint32_t mv = magic_vgpr();
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(base + (size_t)b * C * 1024, (uint32_t)C * 1024);
    const __amdgpu_buffer_rsrc_t ru =
        make_rsrc(base + (size_t)I * H / 2 + (size_t)b * C * 1024, (uint32_t)C * 1024);
    // row format: fp32 row scales after the codes; affine: (scale, min) bf16
    // pair per row and 64-input group, in 8-row groups per matrix
    const uint8_t* tab = base + (size_t)3 * H * I / 2;
    const __amdgpu_buffer_rsrc_t rtg = make_rsrc(tab + (size_t)b * G * 256, (uint32_t)G * 256);
    const __amdgpu_buffer_rsrc_t rtu =
        make_rsrc(tab + ((size_t)I * G + (size_t)b * G * 64) * 4, (uint32_t)G * 256);
    float sgr = 1.f, sur = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr) {
        sgr = ((const float*)tab)[row];
        sur = ((const float*)tab)[I + row];
    }
    const int nst = CPU / UG;
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int tt[NT], rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            tt[j] = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, f.perm, grp, p0 + j, tt[j], rr[j]);
        }
        float Gt[NT], Ut[NT], ag[NT], au[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) Gt[j] = Ut[j] = ag[j] = au[j] = 0.f;
        if (base != nullptr) {
            uint4 A[UG], B[UG];
            uint32_t PA = 0, PB = 0;
#pragma unroll
            for (int k = 0; k < UG; ++k) {
                A[k] = bload16(rg, voff + k * 128, 0);
                B[k] = bload16(ru, voff + k * 128, 0);
            }
            if (FMT != MOE_W_INT4_ROW) {
                PA = bload4(rtg, toff, (uint32_t)(c0 / 2) * 32);
                PB = bload4(rtu, toff, (uint32_t)(c0 / 2) * 32);
            }
            copy_slice<NT>(f.xq, f.xsc, tt, nj, H / 8, H / 64, c0, CPU, lane, xq, xs);
            // one rolling step = one span (2 chunks); the last step loads nothing
#define GU_STEP(I_, LOAD_)                                                               \
    {                                                                                    \
        const uint32_t pa = PA, pb = PB;                                                 \
        _Pragma("unroll") for (int k = 0; k < UG; ++k)                                    \
        {                                                                                \
            const uint4 wa = A[k], wb = B[k];                                            \
            if (LOAD_) {                                                                 \
                A[k] = bload16(rg, voff + k * 128, ((I_) + 1) * UG * 128);             \
                B[k] = bload16(ru, voff + k * 128, ((I_) + 1) * UG * 128);             \
            }                                                                            \
            chunk2<NT>(wa, wb, xq, CPU * 4, (I_) * UG + k, nj, mv, ag, au);               \
        }                                                                                \
        if (FMT != MOE_W_INT4_ROW && (LOAD_)) {                                          \
            PA = bload4(rtg, toff, (uint32_t)(c0 / 2 + (I_) + 1) * 32);                 \
            PB = bload4(rtu, toff, (uint32_t)(c0 / 2 + (I_) + 1) * 32);                 \
        }                                                                                \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) if (j < nj)                       \
        {                                                                                \
            const float2 sp = xs[j * (CPU / 2) + (I_)];                                  \
            Gt[j] = fold<FMT>(Gt[j], ag[j], sp, pa);                                     \
            Ut[j] = fold<FMT>(Ut[j], au[j], sp, pb);                                     \
            ag[j] = au[j] = 0.f;                                                         \
        }                                                                                \
    }
#pragma unroll 1
            for (int i = 0; i < nst - 1; ++i) GU_STEP(i, true)
            GU_STEP(nst - 1, false)
#undef GU_STEP
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                red[(q * NT + j) * 128 + lane] = Gt[j] * sgr;
                red[(q * NT + j) * 128 + 64 + lane] = Ut[j] * sur;
            }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj && j % KS == q) {
                float g = 0.f, u = 0.f;
                for (int s2 = 0; s2 < KS; ++s2) {
                    g += red[(s2 * NT + j) * 128 + lane];
                    u += red[(s2 * NT + j) * 128 + 64 + lane];
                }
                const float rs = f.tok[tt[j]].rscale;
                g *= rs;
                u *= rs;
                stage_span64(g / (1.0f + expf(-g)) * u, lane,
                             (uint16_t*)(f.hq + (size_t)rr[j] * (I / 8) + b * 8),
                             f.hsc + (size_t)rr[j] * (I / 64) + b);
            }
        __syncthreads();
    }
}

// gate/up finalize: one wavefront per (row r, block b): fixed-order sum of
// the k-slices, h = silu(g rs) * (u rs), staged as an fp16 span.
__global__ void __launch_bounds__(256) k_gu_fin(Fwd f, int n_rows)
{
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int NB = f.I / 64, KS = f.gu_ks;
    if (w >= n_rows * NB) return;
    const int r = w / NB, b = w - r * NB;
    const float* p = f.gpart + ((size_t)r * NB + b) * KS * 128;
    // all loads unconditional (slice index clamped), so that they issue
    // together; the slices past KS are then zeroed
    float gv[16], uv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int vc = min(v, KS - 1);
        gv[v] = p[vc * 128 + lane];
        uv[v] = p[vc * 128 + 64 + lane];
    }
#pragma unroll
    for (int v = 0; v < 16; ++v)
        if (v >= KS) gv[v] = uv[v] = 0.f;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        g += gv[v];
        u += uv[v];
    }
    const int TK = f.T * f.K;
    const int t = r < TK ? r / f.K : (r - TK) % f.T;
    const float rs = f.tok[t].rscale;
    g *= rs;
    u *= rs;
    stage_span64(g / (1.0f + expf(-g)) * u, lane, (uint16_t*)(f.hq + (size_t)r * (f.I / 8) + b * 8),
                 f.hsc + (size_t)r * (f.I / 64) + b);
}

// ---------------------------------------------------------------------------
// down unit: partial sd (Wd h_r)_row of one k-slice -> ypart[r][b][q][64].
// CMB (one token): the partials go out agent-coherent and each unit arrives
// on its output block's counter; the unit that completes a block (every
// group's every k-slice) sums it as the combine kernel would (shared experts,
// then the routed ones in rank order, each the sum of its k-slices in order)
// and writes the block's outputs, so no combine launch follows.
// ---------------------------------------------------------------------------

template <int FMT, int NT, bool S8, bool HF = false, bool CMB = false>
__global__ void __launch_bounds__(64) k_dn(Fwd f)
{
    extern __shared__ uint4 lds4[];
    const int lane = threadIdx.x;
    const int KS = f.dn_ks, H = f.H, I = f.I, NB = H / 64, C = I / 32, GI = I / 64;
    int q, b, gi;
    unit_coords(blockIdx.x, KS, NB, q, b, gi);
    if (gi >= uni(f.n_groups[0])) return;
    if (S8 && gi < f.n_shared) {
        dn8_unit<NT>(f, q, b, gi, lds4);
        return;
    }
    const Group grp = uni_group(f.groups, gi);
    const int CPU = C / KS, c0 = q * CPU, row = b * 64 + lane;
    uint4* xq = lds4;
    float2* xs = (float2*)(lds4 + NT * CPU * 4);
    const uint8_t* base = grp.base;
    // the lane's row in the block: its piece of chunk c0 + j at voff + 128 j
    const uint32_t voff = blk_off(lane, C, c0), toff = tab_off(lane, GI, 0);
    const uint32_t mv = magic_vgpr();
    const __amdgpu_buffer_rsrc_t rd =
        make_rsrc(base + (size_t)I * H + (size_t)b * C * 1024, (uint32_t)C * 1024);
    const uint8_t* tab = base + (size_t)3 * H * I / 2;
    const __amdgpu_buffer_rsrc_t rtd = make_rsrc(
        tab + ((size_t)2 * I * (H / 64) + (size_t)b * GI * 64) * 4, (uint32_t)GI * 256);
    float sdr = 1.f;
    if (FMT == MOE_W_INT4_ROW && base != nullptr) sdr = ((const float*)tab)[2 * I + row];
    const int nst = CPU / UD;
#pragma unroll 1
    for (int p0 = 0; p0 < grp.cnt; p0 += NT) {
        const int nj = min(NT, grp.cnt - p0);
        int rr[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            int t = 0;
            rr[j] = 0;
            if (j < nj) tok_rows(f, f.perm, grp, p0 + j, t, rr[j]);
        }
        float Yt[NT], a0[NT], a1[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) Yt[j] = a0[j] = a1[j] = 0.f;
        if (base != nullptr) {
            uint4 D[UD];
            uint32_t P0 = 0, P1 = 0;
#pragma unroll
            for (int k = 0; k < UD; ++k) D[k] = bload16(rd, voff + k * 128, 0);
            if (FMT != MOE_W_INT4_ROW) {
                P0 = bload4(rtd, toff, (uint32_t)(c0 / 2) * 32);
                P1 = bload4(rtd, toff, (uint32_t)(c0 / 2 + 1) * 32);
            }
            if (HF)  // one token, h in fp32 from the one-token gate/up kernel
                stage_slice_f32(f.hf + (size_t)rr[0] * I, c0, CPU, lane, xq, xs);
            else
                copy_slice<NT>(f.hq, f.hsc, rr, nj, I / 8, I / 64, c0, CPU, lane, xq, xs);
            // one rolling step = two spans (4 chunks); the last step loads nothing
#define DN_STEP(I_, LOAD_)                                                               \
    {                                                                                    \
        const uint32_t p0v = P0, p1v = P1;                                               \
        _Pragma("unroll") for (int k = 0; k < UD; ++k)                                    \
        {                                                                                \
            const uint4 wd = D[k];                                                       \
            if (LOAD_) D[k] = bload16(rd, voff + k * 128, ((I_) + 1) * UD * 128);      \
            if (k < 2) chunk1<NT>(wd, xq, CPU * 4, (I_) * UD + k, nj, mv, a0);            \
            else chunk1<NT>(wd, xq, CPU * 4, (I_) * UD + k, nj, mv, a1);                  \
        }                                                                                \
        if (FMT != MOE_W_INT4_ROW && (LOAD_)) {                                          \
            P0 = bload4(rtd, toff, (uint32_t)(c0 / 2 + 2 * (I_) + 2) * 32);             \
            P1 = bload4(rtd, toff, (uint32_t)(c0 / 2 + 2 * (I_) + 3) * 32);             \
        }                                                                                \
        _Pragma("unroll") for (int j = 0; j < NT; ++j) if (j < nj)                       \
        {                                                                                \
            Yt[j] = fold<FMT>(Yt[j], a0[j], xs[j * (CPU / 2) + 2 * (I_)], p0v);          \
            Yt[j] = fold<FMT>(Yt[j], a1[j], xs[j * (CPU / 2) + 2 * (I_) + 1], p1v);      \
            a0[j] = a1[j] = 0.f;                                                         \
        }                                                                                \
    }
#pragma unroll 1
            for (int i = 0; i < nst - 1; ++i) DN_STEP(i, true)
            DN_STEP(nst - 1, false)
#undef DN_STEP
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (j < nj) {
                float* yp = f.ypart + (((size_t)rr[j] * NB + b) * KS + q) * 64 + lane;
                if (CMB)
                    st_agent(yp, Yt[j] * sdr);
                else
                    *yp = Yt[j] * sdr;
            }
        lds_wave_sync();
    }
    if constexpr (CMB) {
        // one token (T = 1): routed rank k is row k, shared expert s row K + s
        if (!arrive_wave(f.dn_cnt + (size_t)b * 64, (uint32_t)(uni(f.n_groups[0]) * KS))) return;
        const int K = f.K, ns = f.n_shared;
        float v[9][4];
#pragma unroll
        for (int e = 0; e < 9; ++e) {
            int r = -1;
            if (e < ns) r = K + e;
            else if (e - ns < K) r = e - ns;
            const float* p = f.ypart + ((size_t)(r < 0 ? 0 : r) * NB + b) * KS * 64 + lane;
#pragma unroll
            for (int s = 0; s < 4; ++s) v[e][s] = ld_agent(p + min(s, KS - 1) * 64);
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (r < 0 || s >= KS) v[e][s] = 0.f;
        }
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 9; ++e) {
            const float y = (v[e][0] + v[e][1]) + (v[e][2] + v[e][3]);
            if (e < ns) m += y;
            else if (e - ns < K) m = fmaf(f.wts[e - ns], y, m);
        }
        const int d = b * 64 + lane;
        if (f.residual) m = f.x[d] + m;
        f.out[d] = m;
    }
}

// Combine, one thread per output element, fixed order: shared experts, then
// routed experts in rank order, each the sum of its k-slices in order;
// out = (x +) that sum.
__global__ void __launch_bounds__(256) k_combine(Fwd f)
{
    const int H = f.H, T = f.T, K = f.K, KS = f.dn_ks, NB = H / 64;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * H) return;
    const int t = (int)(idx / H), d = (int)(idx - (int64_t)t * H);
    const int b = d >> 6, lane = d & 63;
    // up to 9 expert rows x 4 k-slices in flight
    float v[9][4];
#pragma unroll
    for (int e = 0; e < 9; ++e) {
        int r = -1;
        if (e < f.n_shared) r = T * K + e * T + t;
        else if (e - f.n_shared < K) r = t * K + (e - f.n_shared);
        const float* p = f.ypart + ((size_t)(r < 0 ? 0 : r) * NB + b) * KS * 64 + lane;
        // unconditional loads (indices clamped), then the absent ones zeroed
#pragma unroll
        for (int s = 0; s < 4; ++s) v[e][s] = p[min(s, KS - 1) * 64];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            if (r < 0 || s >= KS) v[e][s] = 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 9; ++e) {
        const float y = (v[e][0] + v[e][1]) + (v[e][2] + v[e][3]);
        if (e < f.n_shared) m += y;
        else if (e - f.n_shared < K) m = fmaf(f.wts[t * K + (e - f.n_shared)], y, m);
    }
    if (f.residual) m = f.x[idx] + m;
    f.out[idx] = m;
}

// ---------------------------------------------------------------------------
// One token: the down projection and the combine in one kernel.  The output
// rows go to 256 workgroups (one per CU), RG groups of 8 rows each, so that
// every CU streams the same share; a workgroup covers its rows for every
// expert slot (the shared experts, then the routed ones in rank order), so
// the whole reduction of those rows stays inside it: no partial sums leave
// the workgroup and no combine kernel follows.  Wavefront w takes chunk
// group w (8 chunks of 32 inputs) of every (slot, row group): lane = (row r
// of 8, chunk c of 8), one 16-byte code load covering 8 rows x 8 chunks,
// DC_D loads in flight.  The slots' h (fp16 spans, staged by the gate/up
// finalize) is copied to LDS once.  Sums are reduced in LDS in a fixed order
// (chunk, then wavefront), scaled, weighted and added in slot order (+ x).
// ---------------------------------------------------------------------------

constexpr int DC_NE = 9;   // expert slots at most (shared + routed)
constexpr int DC_D = 12;   // code loads in flight per wavefront
constexpr int DC_HL = 5;   // h staging loads per thread at most

// LDS: h [NE][I/8] uint4 + spans [NE][I/64] float2, later reused for the
// partial sums [NCG][NE][RG][64] and the chunk-reduced [NCG][NE][RG][8].
size_t dn2_lds_bytes(int I, int RG)
{
    const int ncg = I / 256;
    const size_t h = (size_t)DC_NE * I * 2 + (size_t)DC_NE * (I / 64) * 8;
    const size_t r = (size_t)ncg * DC_NE * RG * 64 * 4 + (size_t)ncg * DC_NE * RG * 8 * 4;
    return std::max(h, r);
}

template <int FMT, int RG>
__global__ void __launch_bounds__(512) k_dn2(Fwd f)
{
    extern __shared__ uint4 lds4[];
    __shared__ uint64_t s_base[DC_NE];
    __shared__ int s_row[DC_NE];
    __shared__ float s_wt[DC_NE];
    const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
    const int NCG = (int)(blockDim.x >> 6);  // chunk groups = wavefronts
    const int H = f.H, I = f.I, NP = I / 64, C = I / 32;
    const int ne = f.n_shared + f.K;

    // slot table: shared experts first, routed experts in rank order
    if (tid < DC_NE) {
        s_base[tid] = 0ull;
        s_row[tid] = 0;
        s_wt[tid] = 0.f;
    }
    __syncthreads();
    if (tid < uni(f.n_groups[0])) {
        const Group g = f.groups[tid];
        int e, r;
        float wt = 1.f;
        if (g.kind == 1) {
            e = g.off;
            r = f.K + g.off;  // T = 1
        } else {
            r = f.perm[g.off];  // assignment = rank
            e = f.n_shared + r;
            wt = f.wts[r];
        }
        s_base[e] = (uint64_t)(uintptr_t)g.base;
        s_row[e] = r;
        s_wt[e] = wt;
    }
    __syncthreads();

    uint4* hq = lds4;                                // [DC_NE][I/8]
    float2* hs = (float2*)(lds4 + DC_NE * (I / 8));  // [DC_NE][NP]
    // h staging loads first (they return before the code stream)
    const int nh = ne * (I / 8), nsc = ne * NP, nthr = 64 * NCG;
    uint4 hv[DC_HL];
#pragma unroll
    for (int k = 0; k < DC_HL; ++k) {
        const int i = tid + k * nthr;
        const int e = min(i / (I / 8), DC_NE - 1), c = i - e * (I / 8);
        hv[k] = i < nh ? f.hq[(size_t)s_row[e] * (I / 8) + c] : make_uint4(0u, 0u, 0u, 0u);
    }
    float2 sv = make_float2(0.f, 0.f);
    if (tid < nsc) sv = f.hsc[(size_t)s_row[tid / NP] * NP + tid % NP];

    // slot bases (wave-uniform); a slot without an expert (beyond ne, or not
    // resident) gets an empty resource, whose loads return zeros; its sums
    // are never combined
    uint64_t bases[DC_NE];
#pragma unroll
    for (int e = 0; e < DC_NE; ++e) {
        const uint64_t b = e < ne ? s_base[e] : 0ull;
        bases[e] = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b)) |
                   ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32);
    }
    const uint8_t* anchor = (const uint8_t*)f.x;  // any valid address
    const int r8 = lane & 7, c8 = lane >> 3;
    const int chunk = 8 * w + c8;  // this lane's chunk (32 inputs)
    // per slot: one resource over the whole down matrix (codes) and its
    // table; the row group's block and row go into the lane offset
    auto code_rsrc = [&](int e) {
        const uint8_t* b = (const uint8_t*)(uintptr_t)bases[e];
        return make_rsrc(b ? b + (size_t)I * H : anchor, b ? (uint32_t)((size_t)I * H / 2) : 0u);
    };
    auto tab_rsrc = [&](int e) {
        const uint8_t* b = (const uint8_t*)(uintptr_t)bases[e];
        return make_rsrc(b ? b + (size_t)3 * H * I / 2 + (size_t)2 * I * (H / 64) * 4 : anchor,
                         (b && FMT != MOE_W_INT4_ROW) ? (uint32_t)(H / 64) * NP * 256 : 0u);
    };
    uint32_t coff[RG], toff[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int rg = blockIdx.x * RG + g, blk = rg >> 3, row64 = (rg & 7) * 8 + r8;
        coff[g] = (uint32_t)blk * C * 1024 + blk_off(row64, C, chunk);
        toff[g] = (uint32_t)blk * NP * 256 + tab_off(row64, NP, chunk >> 1);
    }
    const uint32_t mv = magic_vgpr();
    constexpr int NS = DC_NE * RG;  // steps (slot e, row group g), e outer
    uint4 R[DC_D];
    uint32_t P[DC_D];
#pragma unroll
    for (int st = 0; st < DC_D; ++st)
        if (st < NS) {
            const int e = st / RG, g = st % RG;
            R[st] = bload16(code_rsrc(e), coff[g], 0);
            P[st] = FMT != MOE_W_INT4_ROW ? bload4(tab_rsrc(e), toff[g], 0) : 0u;
        }
#pragma unroll
    for (int k = 0; k < DC_HL; ++k) {
        const int i = tid + k * nthr;
        if (i < nh) hq[i] = hv[k];
    }
    if (tid < nsc) hs[tid] = sv;
    __syncthreads();

    float Y[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const int e = st / RG;
        const uint4 wv = R[st % DC_D];
        const uint32_t pv = P[st % DC_D];
        const int sn = st + DC_D;
        if (sn < NS) {
            const int en = sn / RG, gn = sn % RG;
            R[st % DC_D] = bload16(code_rsrc(en), coff[gn], 0);
            if (FMT != MOE_W_INT4_ROW) P[st % DC_D] = bload4(tab_rsrc(en), toff[gn], 0);
        }
        // 32 codes of row r8 (of row group g), chunk `chunk`, against the slot's h
        const uint4* xv = hq + e * (I / 8) + chunk * 4;
        float a = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t p0, p1, p2, p3;
            nib_pairs(dw(wv, d), mv, p0, p1, p2, p3);
            a = dot_dword(p0, p1, p2, p3, xv[d], a);
        }
        // the span's correction term once (its even chunk), then 2^-k
        const float2 sp = hs[e * NP + (chunk >> 1)];
        const bool odd = chunk & 1;
        float v;
        if (FMT == MOE_W_INT4_ROW) {
            v = fmaf(a, 0.0625f, odd ? 0.f : -72.f * sp.y);
        } else {
            const float sc = bf16_lo(pv), mn = bf16_hi(pv);
            v = fmaf(sc * 0.0625f, a, odd ? 0.f : (mn - 64.f * sc) * sp.y);
        }
        Y[st] = v * sp.x;
    }
    __syncthreads();  // h is no longer read: its LDS takes the partial sums
    float* red = (float*)lds4;                          // [NCG][NS][64]
    float* red8 = red + (size_t)NCG * NS * 64;          // [NCG][NS][8]
#pragma unroll
    for (int st = 0; st < NS; ++st) red[(w * NS + st) * 64 + lane] = Y[st];
    __syncthreads();
    // sum over the 8 chunks of each wavefront, in chunk order
    for (int i = tid; i < NCG * NS * 8; i += nthr) {
        const int ws = i >> 3, r = i & 7;
        float y = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) y += red[ws * 64 + c * 8 + r];
        red8[i] = y;
    }
    __syncthreads();
    // row (g, r): sum over the wavefronts in order, scale, weight, combine
    if (tid < 8 * RG) {
        const int g = tid >> 3, r = tid & 7;
        const int o = (blockIdx.x * RG + g) * 8 + r;
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < DC_NE; ++e)
            if (e < ne) {
                float y = 0.f;
                for (int v2 = 0; v2 < NCG; ++v2) y += red8[(v2 * NS + e * RG + g) * 8 + r];
                const uint8_t* base = (const uint8_t*)(uintptr_t)s_base[e];
                if (base == nullptr) y = 0.f;  // not resident: no contribution
                else if (FMT == MOE_W_INT4_ROW)
                    y *= ((const float*)(base + (size_t)3 * H * I / 2))[2 * I + o];
                if (e < f.n_shared) m += y;
                else m = fmaf(s_wt[e], y, m);
            }
        if (f.residual) m = f.x[o] + m;
        f.out[o] = m;
    }
}

// Combine of single-slice partials ([rows][H], the grouped GEMM's layout),
// one thread per 4 consecutive outputs of a token: the same fixed order and
// arithmetic per element as combine_one.
__global__ void __launch_bounds__(256) k_combine_rows(Fwd f)
{
    const int H4 = f.H / 4, T = f.T, K = f.K;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * H4) return;
    const int t = (int)(idx / H4), d4 = (int)(idx - (int64_t)t * H4);
    float4 v[9];
#pragma unroll
    for (int e = 0; e < 9; ++e) {
        int r = -1;
        if (e < f.n_shared) r = T * K + e * T + t;
        else if (e - f.n_shared < K) r = t * K + (e - f.n_shared);
        v[e] = r >= 0 ? ((const float4*)(f.ypart + (size_t)r * f.H))[d4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int e = 0; e < 9; ++e) {
        if (e < f.n_shared) {
            m.x += v[e].x;
            m.y += v[e].y;
            m.z += v[e].z;
            m.w += v[e].w;
        } else if (e - f.n_shared < K) {
            const float w = f.wts[t * K + (e - f.n_shared)];
            m.x = fmaf(w, v[e].x, m.x);
            m.y = fmaf(w, v[e].y, m.y);
            m.z = fmaf(w, v[e].z, m.z);
            m.w = fmaf(w, v[e].w, m.w);
        }
    }
    float4* o = (float4*)(f.out + (size_t)t * f.H) + d4;
    if (f.residual) {
        const float4 x = ((const float4*)(f.x + (size_t)t * f.H))[d4];
        m = make_float4(x.x + m.x, x.y + m.y, x.z + m.z, x.w + m.w);
    }
    *o = m;
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

// Tokens per pass over the weights.
static int tokens_per_pass(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : 4; }

static int max_groups(const Fwd& f) { return f.n_shared + std::min(f.E, f.T * f.K); }

size_t gemv_lds_bytes(int chunks_per_slice, int T)
{
    const int nt = tokens_per_pass(T);
    return (size_t)nt * (chunks_per_slice * 4 * 16 + (chunks_per_slice / 2) * 8);
}

int gemv_step_chunks(int which) { return which == 0 ? UG : UD; }

int gemv_max_dn_ks() { return 4; }

// Dynamic LDS above the default 64 KiB needs the kernel's attribute raised
// (once per kernel, before its first launch that needs it).
template <typename Kern>
static hipError_t allow_lds(Kern kern, size_t lds, bool& done)
{
    if (lds <= 65536 || done) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void*)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    done = e == hipSuccess;
    return e;
}

template <int FMT, int NT, bool S8>
static hipError_t gu_launch(const Fwd& f, hipStream_t st)
{
    const int KS = f.gu_ks, CPU = f.H / 32 / KS;
    const unsigned units = (unsigned)(max_groups(f) * (f.I / 64) * KS);
    const size_t lds = gemv_lds_bytes(CPU, f.T);
    static bool big = false;
    hipError_t e0 = allow_lds(k_gu<FMT, NT, S8>, lds, big);
    if (e0 != hipSuccess) return e0;
    return launch_k(k_gu<FMT, NT, S8>, dim3(units), dim3(64), lds, st, f);
}

template <int FMT, int NT, bool S8, bool HF = false, bool CMB = false>
static hipError_t dn_launch(const Fwd& f, hipStream_t st)
{
    const int KS = f.dn_ks, CPU = f.I / 32 / KS;
    const unsigned units = (unsigned)(max_groups(f) * (f.H / 64) * KS);
    const size_t lds = gemv_lds_bytes(CPU, f.T);
    static bool big = false;
    hipError_t e0 = allow_lds(k_dn<FMT, NT, S8, HF, CMB>, lds, big);
    if (e0 != hipSuccess) return e0;
    return launch_k(k_dn<FMT, NT, S8, HF, CMB>, dim3(units), dim3(64), lds, st, f);
}

template <int FMT, bool S8>
static hipError_t gu_dispatch(const Fwd& f, hipStream_t st)
{
    switch (tokens_per_pass(f.T)) {
    case 1: return gu_launch<FMT, 1, S8>(f, st);
    case 2: return gu_launch<FMT, 2, S8>(f, st);
    default: return gu_launch<FMT, 4, S8>(f, st);
    }
}

template <int FMT, bool S8>
static hipError_t dn_dispatch(const Fwd& f, hipStream_t st)
{
    switch (tokens_per_pass(f.T)) {
    case 1: return dn_launch<FMT, 1, S8>(f, st);
    case 2: return dn_launch<FMT, 2, S8>(f, st);
    default: return dn_launch<FMT, 4, S8>(f, st);
    }
}

bool shared_int8(const Fwd& f) { return f.n_shared > 0 && f.shared_fmt == MOE_W_INT8_ROW; }

size_t gemv_wg_lds_bytes(int chunks_per_slice, int T, int ks)
{
    const int nt = tokens_per_pass(T);
    return (size_t)ks * gemv_wave_lds_u4(chunks_per_slice, nt) * 16 + (size_t)ks * nt * 128 * 4;
}

template <int FMT, int NT>
static hipError_t gu_wg_launch(const Fwd& f, hipStream_t st)
{
    const int KS = f.gu_ks, CPU = f.H / 32 / KS;
    const unsigned wgs = (unsigned)(max_groups(f) * (f.I / 64));
    const size_t lds = gemv_wg_lds_bytes(CPU, f.T, KS);
    static bool big = false;
    hipError_t e0 = allow_lds(k_gu_wg<FMT, NT>, lds, big);
    if (e0 != hipSuccess) return e0;
    return launch_k(k_gu_wg<FMT, NT>, dim3(wgs), dim3(64 * KS), lds, st, f);
}

template <int FMT>
static hipError_t gu_wg_dispatch(const Fwd& f, hipStream_t st)
{
    switch (tokens_per_pass(f.T)) {
    case 1: return gu_wg_launch<FMT, 1>(f, st);
    case 2: return gu_wg_launch<FMT, 2>(f, st);
    default: return gu_wg_launch<FMT, 4>(f, st);
    }
}

// With int8 shared experts, their units take the int8 branch inside the same
// launch as the routed experts' units.
hipError_t launch_gateup_gemv(const Fwd& f, hipStream_t st)
{
    if (f.gu_wg)
        return f.fmt == MOE_W_INT4_ROW ? gu_wg_dispatch<MOE_W_INT4_ROW>(f, st)
                                       : gu_wg_dispatch<MOE_W_INT4_AFFINE_G64>(f, st);
    const bool s8 = shared_int8(f);
    if (f.fmt == MOE_W_INT4_ROW)
        return s8 ? gu_dispatch<MOE_W_INT4_ROW, true>(f, st) : gu_dispatch<MOE_W_INT4_ROW, false>(f, st);
    return s8 ? gu_dispatch<MOE_W_INT4_AFFINE_G64, true>(f, st)
              : gu_dispatch<MOE_W_INT4_AFFINE_G64, false>(f, st);
}

hipError_t launch_down_gemv(const Fwd& f, hipStream_t st)
{
    if (f.h_f32 && f.dn_fused)  // one token, the combine in the last unit of each block
        return f.fmt == MOE_W_INT4_ROW ? dn_launch<MOE_W_INT4_ROW, 1, false, true, true>(f, st)
                                       : dn_launch<MOE_W_INT4_AFFINE_G64, 1, false, true, true>(f, st);
    if (f.h_f32)  // one token after the one-token gate/up kernel (int4 shared experts)
        return f.fmt == MOE_W_INT4_ROW ? dn_launch<MOE_W_INT4_ROW, 1, false, true>(f, st)
                                       : dn_launch<MOE_W_INT4_AFFINE_G64, 1, false, true>(f, st);
    const bool s8 = shared_int8(f);
    if (f.fmt == MOE_W_INT4_ROW)
        return s8 ? dn_dispatch<MOE_W_INT4_ROW, true>(f, st) : dn_dispatch<MOE_W_INT4_ROW, false>(f, st);
    return s8 ? dn_dispatch<MOE_W_INT4_AFFINE_G64, true>(f, st)
              : dn_dispatch<MOE_W_INT4_AFFINE_G64, false>(f, st);
}

bool gateup_needs_finalize(const Fwd& f) { return f.gu_ks > 1 && !f.gu_wg; }

hipError_t launch_gateup_finalize(const Fwd& f, hipStream_t st)
{
    const int n_rows = f.T * (f.K + f.n_shared);
    const int waves = n_rows * (f.I / 64);
    return launch_k(k_gu_fin, dim3((waves + 3) / 4), dim3(256), 0, st, f, n_rows);
}

// One-token down + combine: shapes it covers (otherwise the down GEMV and
// the combine kernel run): 256 workgroups of H/256 rows in groups of 8, one
// wavefront per 256 inputs.
static int dn2_rg(const Fwd& f) { return f.H % 2048 == 0 ? f.H / 2048 : 0; }

// Used for small down projections (at most 16 MiB of codes per token),
// where the separate combine launch dominates; the many-unit down GEMV
// streams large ones faster.
bool down_combine1_ok(const Fwd& f)
{
    const int rg = dn2_rg(f), ncg = f.I / 256, ne = f.n_shared + f.K;
    return f.T == 1 && !shared_int8(f) && ne <= DC_NE && (size_t)ne * f.H * f.I / 2 <= ((size_t)16 << 20) && rg >= 1 && rg <= 4 && f.I % 256 == 0 && ncg >= 1 &&
           ncg <= 8 && ne * (f.I / 8) <= DC_HL * 64 * ncg && ne * (f.I / 64) <= 64 * ncg &&
           dn2_lds_bytes(f.I, rg) <= 65536;
}

template <int FMT>
static hipError_t dn2_launch(const Fwd& f, hipStream_t st)
{
    const int rg = dn2_rg(f);
    const dim3 grid(f.H / (8 * rg)), block(64 * (f.I / 256));
    const size_t lds = dn2_lds_bytes(f.I, rg);
    switch (rg) {
    case 1: return launch_k(k_dn2<FMT, 1>, grid, block, lds, st, f);
    case 2: return launch_k(k_dn2<FMT, 2>, grid, block, lds, st, f);
    case 3: return launch_k(k_dn2<FMT, 3>, grid, block, lds, st, f);
    default: return launch_k(k_dn2<FMT, 4>, grid, block, lds, st, f);
    }
}

hipError_t launch_down_combine1(const Fwd& f, hipStream_t st)
{
    if (f.fmt == MOE_W_INT4_ROW) return dn2_launch<MOE_W_INT4_ROW>(f, st);
    return dn2_launch<MOE_W_INT4_AFFINE_G64>(f, st);
}

hipError_t launch_combine(const Fwd& f, hipStream_t st)
{
    if (f.dn_ks == 1 && f.n_shared + f.K <= 9) {
        const int64_t n = (int64_t)f.T * (f.H / 4);
        return launch_k(k_combine_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, f);
    }
    const int64_t n = (int64_t)f.T * f.H;
    return launch_k(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, f);
}

}  // namespace moe
