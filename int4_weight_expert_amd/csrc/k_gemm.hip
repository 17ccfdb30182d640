// k_gemm.hip -- the expert FFN for many tokens as MFMA grouped GEMMs.
//
// What is computed, cited by page title and section:
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11: each chosen
//     expert is SwiGLU on the rows routed to it (gate/up -> silu(g)*u ->
//     down), each expert's weights read once for all of its rows; §04
//     siluf(x) = x/(1+exp(-x)).
//   GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6b-6d: 6144 -> 2048 ->
//     6144 experts plus the always-active shared expert.
// With hundreds of rows per expert the step is a dense contraction, so it
// runs on the matrix cores: per expert group, [rows x H] . [H x I] twice
// (gate and up, SiLU(gate)*up fused into the epilogue), then
// [rows x I] . [I x H] (down).
//
// Operands.  Activations (x, then h) are staged per row as fp16 after an
// exact power-of-two scale 2^k (largest magnitude in [2^13, 2^14)), in the
// pair order of k_common.h (x0 x4 x1 x5 x2 x6 x3 x7 per 8 inputs), with the
// row's (2^-k, sum of its fp16 values).  Codes become fp16 1024 + 16 n in
// registers (3 shifts and 4 bit-field inserts per 8 codes), already in the
// same pair order, so each v_mfma_f32_32x32x16_f16 multiplies matching
// inputs; the epilogue recovers sum c x = acc/16 - 72 S (row format codes
// are stored c + 8) and applies 2^-k and the fp32 row scale.  Accumulation
// is fp32 in the matrix cores.
//
// Tiling.  A work item is (expert group, 128 rows of it, N tile) on a
// workgroup of 8 wavefronts.  Gate/up: the N tile is 256 output rows; each
// wavefront owns 32 of them in both matrices (two 32-column MFMA blocks).
// Down: the N tile is 512 output rows, 64 per wavefront (two blocks).  Wide
// N tiles let one staged activation tile feed many output columns: the
// activations (2 bytes per input) are the larger share of operand traffic.  Each
// wavefront covers the 128 rows as four 32-row blocks: 8 accumulator tiles.
// Per K step of 64 inputs (two 16-byte chunks of int4 codes per output row):
// the activation tile (128 x 64 fp16) is double-buffered in LDS, piece-major
// so the A-operand reads are conflict-free; every wavefront loads its own
// codes straight into registers with one 16-byte load per lane (lanes l and
// l+32 read the step's two chunks of a row, each feeding four MFMAs).
// Activations and codes are fetched 4 steps ahead.  (Per-row int8 codes, a
// shared expert: 32-input steps of two 16-byte chunks.)
#include <type_traits>

#include "k_common.h"

namespace moe {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16 __attribute__((ext_vector_type(16)));

constexpr int GM = 128;    // rows per tile
constexpr int GDEP = 8;    // K steps of activations and codes in flight
constexpr int GW = 8;      // wavefronts per workgroup

enum { GEMM_GU = 0, GEMM_DN = 1 };

// Row j of an expert group: token t and row r (as tok_rows, per lane).
__device__ __forceinline__ void tok_rows_lane(const Fwd& f, const Group& g, int j, int& t, int& r)
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

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(half8, make_uint4(a, b, c, d));
}

// B operand of one 16-input half of a chunk: dword `d` of a row's 16 bytes
__device__ __forceinline__ half8 b_operand(uint32_t dword, uint32_t mv)
{
    uint32_t p0, p1, p2, p3;
    nib_pairs_mfma(dword, mv, p0, p1, p2, p3);
    return as_half8(p0, p1, p2, p3);
}

// Output rows o0, o1 of wavefront w's two B blocks in N tile `ntile`, and
// the byte offsets of their matrices in the expert's slot.
template <int MODE, bool S8 = false>
__device__ __forceinline__ void gemm_out_rows(int ntile, int w, int n, int H, int I, int& o0,
                                              int& o1, size_t& mat0, size_t& mat1)
{
    // int8 matrices take a byte per weight, int4 half a byte
    const size_t msz = S8 ? (size_t)I * H : (size_t)I * H / 2;
    if (MODE == GEMM_GU) {
        o0 = ntile * 256 + 32 * w + n;  // gate and up of the same row
        o1 = o0;
        mat0 = 0;
        mat1 = msz;
    } else {
        o0 = ntile * 512 + 64 * w + n;  // rows n and n + 32 of one block
        o1 = o0 + 32;
        mat0 = mat1 = 2 * msz;
    }
}

// B operand of 8 int8 codes (stored q + 128): bytes i and 4 + i of the
// dword pair as the fp16 pair (1024 + b_i, 1024 + b_{4+i}), the activations'
// pair order
__device__ __forceinline__ half8 b_operand8(uint32_t lo, uint32_t hi)
{
    const uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
    const uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
    const uint32_t p2 = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
    const uint32_t p3 = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
    return as_half8(p0, p1, p2, p3);
}

// The tile's prologue, K loop and epilogue, specialised on the number MB of
// 32-row blocks that hold rows of the group: a partial tile issues only its
// blocks' LDS reads and MFMAs.  Each specialisation is self-contained, so no
// register array lives across the dispatch.  This one: per-row int8 codes
// (a shared expert), K step of 32 inputs = two 16-byte chunks, lane half h
// loading chunk 2 step + h whole.
template <int MODE, int MB>
__device__ __forceinline__ void gemm_tile8(const Fwd& f, uint4 (*As)[8][GM], const int* s_src,
                                          const int* s_out, const float* s_inv,
                                          const float* s_sum, const float* s_rs,
                                          const uint8_t* base, int ntile, int rows)
{
    const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
    const int n = lane & 31, half = lane >> 5;
    const int H = f.H, I = f.I;
    const int K = MODE == GEMM_GU ? H : I;  // reduction length
    const int NC = K / 32;                  // K steps (chunks)
    int o0, o1;
    size_t mat0, mat1;
    gemm_out_rows<MODE, true>(ntile, w, n, H, I, o0, o1, mat0, mat1);
    // fp32 row scales after the three matrices
    const uint8_t* tab = base + (size_t)3 * H * I;

    // weight streams: the wavefront's rows lie in one 64-row block (a
    // wave-uniform resource); the lane's row within it is the offset.  A
    // 16-byte chunk holds 16 int8 codes: a K step of 32 inputs is two chunks
    // (lane half h reads chunk 2 step + h whole).
    const int C = 2 * NC;  // chunks per weight row
    const int blk = MODE == GEMM_GU ? ntile * 4 + (w >> 1) : ntile * 8 + w;
    const __amdgpu_buffer_rsrc_t rw0 =
        make_rsrc(base + mat0 + (size_t)blk * C * 1024, (uint32_t)C * 1024);
    const __amdgpu_buffer_rsrc_t rw1 =
        make_rsrc(base + mat1 + (size_t)blk * C * 1024, (uint32_t)C * 1024);
    const uint32_t v0 = (uint32_t)(o0 & 63) * 16 + half * 1024;
    const uint32_t v1 = (uint32_t)(o1 & 63) * 16 + half * 1024;
    constexpr uint32_t STEP = 2048;  // code bytes per K step and 64-row block

    // activation loader: thread -> row tid & 127, piece tid >> 7 (a
    // wavefront writes 64 consecutive rows of one piece: no bank conflict)
    const int arow = tid & (GM - 1), apc = tid >> 7;
    const int asrc = s_src[arow];
    const uint4* Ag = nullptr;
    if (asrc >= 0)
        Ag = (MODE == GEMM_GU ? f.xq + (size_t)asrc * (H / 8) : f.hq + (size_t)asrc * (I / 8)) +
             apc;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

    float16 acc[4][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        acc[mb][0] = (float16){};
        acc[mb][1] = (float16){};
    }

    // prologue: chunk 0 into LDS buffer 0; activation chunks 1..GDEP-1 and
    // code chunks 0..GDEP-1 in flight.  Activations and codes both run GDEP
    // steps ahead, so that waiting for one (vmcnt counts in issue order)
    // never drains the other early.
    uint4 A0[GDEP];  // activation chunk j in slot j % GDEP
    A0[0] = z4;
    if (Ag) A0[0] = Ag[0];
    As[0][apc][arow] = A0[0];
#pragma unroll
    for (int k = 1; k < GDEP; ++k) {
        A0[k] = z4;
        if (Ag) A0[k] = Ag[k * 4];
    }
    // codes: 16 bytes per lane and step, GDEP steps in flight
    uint4 B0[GDEP], B1[GDEP];
#pragma unroll
    for (int k = 0; k < GDEP; ++k) {
        B0[k] = bload16(rw0, v0 + k * STEP, 0);
        B1[k] = bload16(rw1, v1 + k * STEP, 0);
    }
    __syncthreads();

#pragma unroll 1
    for (int c0 = 0; c0 < NC; c0 += GDEP) {
#pragma unroll
        for (int k = 0; k < GDEP; ++k) {
            const int c = c0 + k;
            // chunk c + 1 (slot (c + 1) % GDEP) into the other LDS buffer (its
            // readers of step c - 1 passed the barrier); slot c % GDEP (chunk
            // c, already in LDS) fetches chunk c + GDEP
            const int s1 = (k + 1) % GDEP;
            if (c + 1 < NC) As[(c + 1) & 1][apc][arow] = A0[s1];
            if (Ag && c + GDEP < NC) A0[k] = Ag[(c + GDEP) * 4];
            // codes of step c; refill the slot with step c + GDEP (a load
            // past the row's last chunk returns zeros)
            const uint4 w0 = B0[k], w1 = B1[k];
            // the K order inside a step is free as long as A and B agree:
            // lane half h takes inputs 16h..16h+7 in the first MFMA and
            // 16h+8..16h+15 in the second (LDS pieces 2h, 2h+1)
            B0[k] = bload16(rw0, v0 + (c + GDEP) * STEP, 0);
            B1[k] = bload16(rw1, v1 + (c + GDEP) * STEP, 0);
            const half8 b00 = b_operand8(w0.x, w0.y), b01 = b_operand8(w0.z, w0.w);
            const half8 b10 = b_operand8(w1.x, w1.y), b11 = b_operand8(w1.z, w1.w);
            const uint4(*Ab)[GM] = As[c & 1];
            half8 a0[4], a1[4];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                a0[mb] = __builtin_bit_cast(half8, Ab[2 * half][32 * mb + n]);
                a1[mb] = __builtin_bit_cast(half8, Ab[2 * half + 1][32 * mb + n]);
            }
            // first 16 inputs for all 8 accumulators, then the next 16: a
            // dependent MFMA follows 7 independent ones
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[mb], b00, acc[mb][0], 0, 0, 0);
                acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0[mb], b10, acc[mb][1], 0, 0, 0);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[mb], b01, acc[mb][0], 0, 0, 0);
                acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1[mb], b11, acc[mb][1], 0, 0, 0);
            }
            __syncthreads();
        }
    }

    // epilogue: lane holds column o of each block, rows (j/4)*8 + half*4 + j%4;
    // int8 (stored q + 128, 1024 + n): sum q x = acc - 1152 S
    constexpr float CA = 1.0f, CB = -1152.f;
    if (MODE == GEMM_GU) {
        const float sg = ((const float*)tab)[o0], su = ((const float*)tab)[I + o0];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = 32 * mb + (j >> 2) * 8 + half * 4 + (j & 3);
                if (i < rows) {
                    const float sc = s_inv[i] * s_rs[i];
                    const float g = fmaf(acc[mb][0][j], CA, CB * s_sum[i]) * sc * sg;
                    const float u = fmaf(acc[mb][1][j], CA, CB * s_sum[i]) * sc * su;
                    f.hbuf[(size_t)s_out[i] * I + o0] = g / (1.0f + expf(-g)) * u;
                }
            }
    } else {
        const float sd0 = ((const float*)tab)[2 * I + o0], sd1 = ((const float*)tab)[2 * I + o1];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = 32 * mb + (j >> 2) * 8 + half * 4 + (j & 3);
                if (i < rows) {
                    const float sc = s_inv[i];
                    float* y = f.ypart + (size_t)s_out[i] * H;
                    y[o0] = fmaf(acc[mb][0][j], CA, CB * s_sum[i]) * sc * sd0;
                    y[o1] = fmaf(acc[mb][1][j], CA, CB * s_sum[i]) * sc * sd1;
                }
            }
    }
}

// int4 codes with a K step of 64 inputs: lane half h loads chunk 2s + h of
// its row whole (one 16-byte load; a wavefront's 32 rows are four 8-row
// groups of the slot layout), and dword d of it (inputs 8d..8d+7 of
// the chunk, pair order) meets LDS piece 4h + d in MFMA round d; the
// activation tile of a step is 128 rows x 64 fp16 (8 pieces), double
// buffered, so a step has 4 rounds of MFMAs behind one barrier.
template <int MODE, int MB>
__device__ __forceinline__ void gemm_tile64(const Fwd& f, uint4 (*As)[8][GM], const int* s_src,
                                            const int* s_out, const float* s_inv,
                                            const float* s_sum, const float* s_rs,
                                            const uint8_t* base, int ntile, int rows)
{
    constexpr int D = GDEP / 2;  // K steps in flight (the same bytes as GDEP 32-input steps)
    const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
    const int n = lane & 31, half = lane >> 5;
    const int H = f.H, I = f.I;
    const int K = MODE == GEMM_GU ? H : I;  // reduction length
    const int NC = K / 32, NS = K / 64;     // chunks, K steps
    int o0, o1;
    size_t mat0, mat1;
    gemm_out_rows<MODE, false>(ntile, w, n, H, I, o0, o1, mat0, mat1);
    const uint8_t* tab = base + (size_t)3 * H * I / 2;  // fp32 row scales
    const uint32_t mv = f.magic;
    const int blk = MODE == GEMM_GU ? ntile * 4 + (w >> 1) : ntile * 8 + w;
    const __amdgpu_buffer_rsrc_t rw0 =
        make_rsrc(base + mat0 + (size_t)blk * NC * 1024, (uint32_t)NC * 1024);
    const __amdgpu_buffer_rsrc_t rw1 =
        make_rsrc(base + mat1 + (size_t)blk * NC * 1024, (uint32_t)NC * 1024);
    // the lane's row in its 64-row block, chunk `half` of the first step
    const uint32_t v0 = blk_off(o0 & 63, NC, half);
    const uint32_t v1 = blk_off(o1 & 63, NC, half);
    constexpr uint32_t STEP = 256;  // code bytes per K step and row (two chunks of an 8-row group)

    // activation loader: thread -> row tid & 127, pieces p and 4 + p of the
    // step (p = tid >> 7: piece p of each of the step's two chunks)
    const int arow = tid & (GM - 1), apc = tid >> 7;
    const int asrc = s_src[arow];
    const uint4* Ag = nullptr;
    if (asrc >= 0)
        Ag = (MODE == GEMM_GU ? f.xq + (size_t)asrc * (H / 8) : f.hq + (size_t)asrc * (I / 8)) +
             apc;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

    float16 acc[4][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        acc[mb][0] = (float16){};
        acc[mb][1] = (float16){};
    }

    uint4 A0[D], A1[D];  // step j's two chunks in slot j % D
    A0[0] = A1[0] = z4;
    if (Ag) {
        A0[0] = Ag[0];
        A1[0] = Ag[4];
    }
    As[0][apc][arow] = A0[0];
    As[0][4 + apc][arow] = A1[0];
#pragma unroll
    for (int k = 1; k < D; ++k) {
        A0[k] = A1[k] = z4;
        if (Ag) {
            A0[k] = Ag[k * 8];
            A1[k] = Ag[k * 8 + 4];
        }
    }
    uint4 B0[D], B1[D];
#pragma unroll
    for (int k = 0; k < D; ++k) {
        B0[k] = bload16(rw0, v0 + k * STEP, 0);
        B1[k] = bload16(rw1, v1 + k * STEP, 0);
    }
    __syncthreads();

#pragma unroll 1
    for (int s0 = 0; s0 < NS; s0 += D) {
#pragma unroll
        for (int k = 0; k < D; ++k) {
            const int s = s0 + k;
            // step s + 1 (slot (s + 1) % D) into the other LDS buffer; slot
            // s % D (step s, already in LDS) fetches step s + D
            const int s1 = (k + 1) % D;
            if (s + 1 < NS) {
                As[(s + 1) & 1][apc][arow] = A0[s1];
                As[(s + 1) & 1][4 + apc][arow] = A1[s1];
            }
            if (Ag && s + D < NS) {
                A0[k] = Ag[(s + D) * 8];
                A1[k] = Ag[(s + D) * 8 + 4];
            }
            // codes of step s; refill with step s + D (past the row's last
            // chunk the loads return zeros)
            const uint4 w0 = B0[k], w1 = B1[k];
            B0[k] = bload16(rw0, v0 + (s + D) * STEP, 0);
            B1[k] = bload16(rw1, v1 + (s + D) * STEP, 0);
            const uint4(*Ab)[GM] = As[s & 1];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const half8 bd0 = b_operand(d == 0 ? w0.x : d == 1 ? w0.y : d == 2 ? w0.z : w0.w, mv);
                const half8 bd1 = b_operand(d == 0 ? w1.x : d == 1 ? w1.y : d == 2 ? w1.z : w1.w, mv);
                half8 a[4];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) a[mb] = __builtin_bit_cast(half8, Ab[4 * half + d][32 * mb + n]);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    acc[mb][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb], bd0, acc[mb][0], 0, 0, 0);
                    acc[mb][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mb], bd1, acc[mb][1], 0, 0, 0);
                }
            }
            __syncthreads();
        }
    }

    // epilogue (int4 stored c + 8, 1024 + 16 n): sum c x = acc/16 - 72 S
    if (MODE == GEMM_GU) {
        const float sg = ((const float*)tab)[o0], su = ((const float*)tab)[I + o0];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = 32 * mb + (j >> 2) * 8 + half * 4 + (j & 3);
                if (i < rows) {
                    const float sc = s_inv[i] * s_rs[i];
                    const float g = fmaf(acc[mb][0][j], 0.0625f, -72.f * s_sum[i]) * sc * sg;
                    const float u = fmaf(acc[mb][1][j], 0.0625f, -72.f * s_sum[i]) * sc * su;
                    f.hbuf[(size_t)s_out[i] * I + o0] = g / (1.0f + expf(-g)) * u;
                }
            }
    } else {
        const float sd0 = ((const float*)tab)[2 * I + o0], sd1 = ((const float*)tab)[2 * I + o1];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int i = 32 * mb + (j >> 2) * 8 + half * 4 + (j & 3);
                if (i < rows) {
                    const float sc = s_inv[i];
                    float* y = f.ypart + (size_t)s_out[i] * H;
                    y[o0] = fmaf(acc[mb][0][j], 0.0625f, -72.f * s_sum[i]) * sc * sd0;
                    y[o1] = fmaf(acc[mb][1][j], 0.0625f, -72.f * s_sum[i]) * sc * sd1;
                }
            }
    }
}

template <int MODE>
__global__ void __launch_bounds__(64 * GW, 1) k_gemm(Fwd f)
{
    __shared__ uint4 As[2][8][GM];  // [buffer][16-byte piece][row]
    __shared__ int s_src[GM], s_out[GM];
    __shared__ float s_inv[GM], s_sum[GM], s_rs[GM];

    // Workgroup -> (tile, N tile), XCD-aware: workgroup p runs on XCD p % 8;
    // tile i goes to XCD i % 8 with its N tiles innermost, so the
    // workgroups sharing a tile's activations run together behind one L2 and
    // every XCD gets an even share of the list's mix of tiles.
    const int n_tiles = uni(f.n_tiles[0]);
    const int NT = gridDim.y;  // N tiles
    const int p = blockIdx.y * gridDim.x + blockIdx.x;
    const int xcd = p & 7, q = p >> 3;
    const int tile = (q / NT) * 8 + xcd;  // tile i on XCD i mod 8
    const int ntile = q % NT;
    if (tile >= n_tiles) return;
    const int2 td = f.tiles[tile];
    const Group grp = uni_group(f.groups, uni(td.x));
    const int m0 = uni(td.y);
    const int rows = min(GM, grp.cnt - m0);
    const int tid = threadIdx.x, lane = tid & 63, w = uni(tid >> 6);
    const int n = lane & 31;
    const int H = f.H, I = f.I;

    // per-row data of the tile
    if (tid < GM) {
        int src = -1, out = -1;
        float inv = 0.f, S = 0.f, rs = 1.f;
        if (tid < rows) {
            int t, r;
            tok_rows_lane(f, grp, m0 + tid, t, r);
            out = r;
            if (MODE == GEMM_GU) {
                src = t;
                const float2 xs = f.xrow[t];
                inv = xs.x;
                S = xs.y;
                rs = f.tok[t].rscale;
            } else {
                src = r;
                const float2 hs = f.hrow[r];
                inv = hs.x;
                S = hs.y;
            }
        }
        s_src[tid] = src;
        s_out[tid] = out;
        s_inv[tid] = inv;
        s_sum[tid] = S;
        s_rs[tid] = rs;
    }
    __syncthreads();

    // output rows of this wavefront's two B blocks
    const uint8_t* base = grp.base;
    if (base == nullptr) {
        // expert not resident: no contribution (the router flagged it)
        int o0, o1;
        size_t mat0, mat1;
        gemm_out_rows<MODE>(ntile, w, n, H, I, o0, o1, mat0, mat1);
        for (int i = 0; i < rows; ++i) {
            if (MODE == GEMM_GU) {
                if (lane < 32) f.hbuf[(size_t)s_out[i] * I + o0] = 0.f;
            } else {
                if (lane < 32) {
                    f.ypart[(size_t)s_out[i] * H + o0] = 0.f;
                    f.ypart[(size_t)s_out[i] * H + o1] = 0.f;
                }
            }
        }
        return;
    }
    if (grp.kind == 1 && f.shared_fmt == MOE_W_INT8_ROW) {
        // per-row int8 shared expert (the same tile, int8 B operands)
        switch ((rows + 31) >> 5) {
        case 1: gemm_tile8<MODE, 1>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
        case 2: gemm_tile8<MODE, 2>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
        case 3: gemm_tile8<MODE, 3>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
        default: gemm_tile8<MODE, 4>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
        }
        return;
    }
    switch ((rows + 31) >> 5) {
    case 1: gemm_tile64<MODE, 1>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
    case 2: gemm_tile64<MODE, 2>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
    case 3: gemm_tile64<MODE, 3>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
    default: gemm_tile64<MODE, 4>(f, As, s_src, s_out, s_inv, s_sum, s_rs, base, ntile, rows); break;
    }
}

// Per-row fp16 staging (one wavefront per row of `len` fp32 values):
// q [rows][len/8] in pair order, s[row] = (2^-k, sum of the fp16 values).
template <int NG>
__global__ void __launch_bounds__(256) k_rowstage(const float* __restrict__ src, int n_rows,
                                                  int len, uint4* __restrict__ q,
                                                  float2* __restrict__ s)
{
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    float sum, ss;
    stage_row<NG>(src + (size_t)r * len, len, lane, q + (size_t)r * (len / 8), s + r, sum, ss);
}

// Inclusive sum over the 512 threads of a workgroup (wavefront scans, then
// the 8 wavefront totals); *total receives the sum of all.
__device__ __forceinline__ int block_scan512(int v, int* s_w, int* total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) s_w[w] = v;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        before += i < w ? s_w[i] : 0;
        all += s_w[i];
    }
    __syncthreads();  // s_w may be rewritten by the next scan
    *total = all;
    return before + v;
}

// Tile list.  Sorted first: every group's full 128-row tiles (groups in
// order), then the partial tiles by descending number of occupied 32-row
// blocks (groups in order within a class).  Full tiles are matrix-core
// heavy and read their codes once per 128 rows; partial tiles read the same
// codes per tile for fewer rows, so a run of them asks more of HBM than it
// can give while the full tiles leave it half idle.  The list therefore
// spreads the full tiles evenly among the partial ones, except for the last
// 32 tiles (one wave of workgroups at 8 N tiles each), which are the
// smallest partial tiles, so that the launch still ends on short work.
// k_gemm runs tile i on XCD i mod 8.
constexpr int TILE_LIST_LDS = 2048;  // tiles reordered in LDS (beyond: sorted order)

__global__ void __launch_bounds__(512) k_tiles(Fwd f)
{
    __shared__ int s_w[8];
    __shared__ int2 s_t[TILE_LIST_LDS];
    const int tid = threadIdx.x;
    const int ng = f.n_groups[0];
    int cnt = 0;
    if (tid < ng) cnt = f.groups[tid].cnt;
    const int nfull = cnt / GM, rem = cnt - nfull * GM;
    const int cls = rem ? (rem + 31) >> 5 : 0;  // occupied blocks of the partial tile
    // the sorted list's length first, to know where it can be built
    int nF, nPart;
    block_scan512(nfull, s_w, &nF);
    block_scan512(rem ? 1 : 0, s_w, &nPart);
    const int L = nF + nPart;
    int2* dst = L <= TILE_LIST_LDS ? s_t : f.tiles;
    int base = 0;
    // pass 0: full tiles; passes 1..4: partial tiles with 4, 3, 2, 1 blocks
    for (int pass = 0; pass < 5; ++pass) {
        const int v = pass == 0 ? nfull : (cls == 5 - pass ? 1 : 0);
        int total;
        const int excl = block_scan512(v, s_w, &total) - v;
        for (int i = 0; i < v; ++i)
            dst[base + excl + i] = make_int2(tid, pass == 0 ? i * GM : nfull * GM);
        base += total;
    }
    if (tid == 0) f.n_tiles[0] = base;
    if (dst == f.tiles) return;
    __syncthreads();
    // position x < M holds full tile c if x = floor(c M / nF), else the next
    // partial tile; positions from M on hold the last `tail` partial tiles
    const int tail = min(nPart, 32), M = L - tail;
    for (int x = tid; x < L; x += 512) {
        int src = x;  // from M on (or with no full tiles): partial tile x - nF
        if (x < M && nF > 0) {
            const int c = (int)(((int64_t)x * nF + M - 1) / M);         // first full tile at or after x
            const int cF = (int)(((int64_t)(x + 1) * nF + M - 1) / M);  // full tiles at positions <= x
            src = (c < nF && (int)((int64_t)c * M / nF) == x) ? c : nF + (x - cF);
        }
        f.tiles[x] = s_t[src];
    }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------

int gemm_max_tiles(int T, int K, int E, int n_shared)
{
    const int64_t routed = (int64_t)T * K;
    return (int)((routed + GM - 1) / GM + std::min<int64_t>(E, routed) +
                 (int64_t)n_shared * ((T + GM - 1) / GM));
}

// the row staging of x happens in the router's token statistics
hipError_t launch_gemm_prep(const Fwd& f, hipStream_t st)
{
    return launch_k(k_tiles, dim3(1), dim3(512), 0, st, f);
}

// grid: (max tiles rounded up to the 8 XCDs) x (N tiles); the kernel maps
// workgroups onto the actual tiles
static dim3 gemm_grid(const Fwd& f, int n_tiles_n)
{
    const int mt = (gemm_max_tiles(f.T, f.K, f.E, f.n_shared) + 7) / 8 * 8;
    return dim3(mt, n_tiles_n);
}

hipError_t launch_gemm_gateup(const Fwd& f, hipStream_t st)
{
    return launch_k(k_gemm<GEMM_GU>, gemm_grid(f, f.I / 256), dim3(64 * GW), 0, st, f);
}

hipError_t launch_gemm_hstage(const Fwd& f, hipStream_t st)
{
    const int rows = f.T * (f.K + f.n_shared);
    const dim3 grid((rows + 3) / 4), block(256);
    const int ng = (f.I + 511) / 512;  // 8-value groups per lane
    auto go = [&](auto kern) {
        return launch_k(kern, grid, block, 0, st, (const float*)f.hbuf, rows, f.I, f.hq, f.hrow);
    };
    if (ng <= 1) return go(k_rowstage<1>);
    if (ng <= 2) return go(k_rowstage<2>);
    if (ng <= 4) return go(k_rowstage<4>);
    if (ng <= 8) return go(k_rowstage<8>);
    if (ng <= 12) return go(k_rowstage<12>);
    return go(k_rowstage<16>);
}

hipError_t launch_gemm_down(const Fwd& f, hipStream_t st)
{
    return launch_k(k_gemm<GEMM_DN>, gemm_grid(f, f.H / 512), dim3(64 * GW), 0, st, f);
}

// Shapes the grouped GEMM tiles exactly: N tiles of 256 (gate/up) and 512
// (down) output rows; rows of at most 8192 values for the one-pass row
// staging (16 groups of 8 per lane).
bool gemm_shape_ok(int H, int I) { return H % 512 == 0 && I % 256 == 0 && H <= 8192 && I <= 8192; }

}  // namespace moe
