/*
 * moe_oracle.c -- plain, slow, single-threaded CPU oracle of the int4-weight
 * MoE FFN step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code.  The GPU library
 * never links, includes or calls it, and it shares no code, header, table or
 * constant generator with the GPU library.
 *
 * Precision: every dot product and sum is accumulated in fp64.  Each named
 * intermediate (router logit, sigmoid score, gate, up, h, expert output,
 * layer output) is rounded to fp32, which is at least as accurate as any
 * fp32 evaluation order.  Decisions that produce integers (quantised codes,
 * expert selection) are taken in fp32, the precision in which the pages make
 * them.
 *
 * Sources (web pages; cited by title and section):
 *   [GLM-C]  "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx): section 04
 *            (basic math: rmsnorm, siluf), 05 (400-line streaming engine:
 *            quantize_rows, moe()), 06 (FP8 to int4: FP8 block-scale decode,
 *            quant_int4, pack_int4, decoded container), 07 (np.rint == lrintf), 11 (MoE routing and
 *            expert execution), 13 (contiguous expert slab, VRAM hot tier).
 *   [FLOW]   GLM-5.2 inference dataflow page (devpress.csdn.net), section
 *            2.3 (MoE FFN: 256 routed + 1 shared) and section 三, Step 6
 *            (6a router, 6b experts, 6c shared expert, 6d merge).
 *   [COLI]   "初始化与权重加载" (colibrì analysis, blog.chen3feng.top):
 *            section 1.1 (Cfg: n_group, topk_group, norm_topk, routed_scale),
 *            1.2 (load_cfg asserts n_group == 1), 2.2 (ESlot).
 *   [EDGE0]  Edge0 write-up (magicnetworld.com, "19.5 GB 的模型装进 24 GB 的机器"):
 *            section 三 (affine int4, group size 64, 1.77 MB per expert),
 *            section 七 (sigmoid-group routing formula with the 1e-20 term).
 *
 * Readings taken where the pages are silent or disagree (each is also listed
 * in the design notes):
 *   - nibbles are two's complement (q & 0xF), even column in the low nibble;
 *     the pages' container stores q+8 (offset binary), which is the same byte
 *     with both nibbles' top bits flipped (byte ^ 0x88);
 *   - codes are clamped to [-7, 7]; with s = amax/7 the code -8 cannot occur;
 *   - rounding is round-half-to-even (rintf), the rounding the pages show to
 *     match numpy's rint;
 *   - chosen weights are renormalised before the routed scale ([EDGE0] §七,
 *     [COLI] §1.1 norm_topk), the [GLM-C] §11 snippet being abbreviated;
 *   - sigmoid(z) = 1/(1+exp(-z)); silu(z) = z/(1+exp(-z)) ([GLM-C] §04);
 *   - affine g64 quantisation: per group of 64 input columns, scale =
 *     bf16((max-min)/15), min = bf16(min), q = clamp(rint((w-min)/scale),0,15);
 *   - the shared expert uses the routed experts' int4 format, weight 1;
 *   - layer chaining normalises the MoE input with a unit-weight RMSNorm
 *     (eps 1e-6, double mean square as in [GLM-C] §04).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_W_INT4_ROW = 1, ORC_W_INT4_AFFINE_G64 = 2, ORC_W_INT8_ROW = 3 };

/* ------------------------------------------------------------------------ */
/* Sizes ([GLM-C] §13 one contiguous g|u|d slab per expert; [EDGE0] §三).    */
/* ------------------------------------------------------------------------ */

int64_t orc_blob_bytes(int fmt, int64_t H, int64_t I)
{
    if (fmt == ORC_W_INT8_ROW) return 3 * H * I + 4 * (I + I + H);
    int64_t packed = I * (H / 2) * 2 + H * (I / 2);
    if (fmt == ORC_W_INT4_ROW) return packed + 4 * (I + I + H);
    if (fmt == ORC_W_INT4_AFFINE_G64) return packed + 4 * (I * (H / 64) * 2 + H * (I / 64));
    return -1;
}

/* ------------------------------------------------------------------------ */
/* bf16 helpers (round to nearest even)                                      */
/* ------------------------------------------------------------------------ */

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float orc_bf16_round(float f) { return bf16_to_f32(f32_to_bf16_rne(f)); }

/* ------------------------------------------------------------------------ */
/* O1: per-row symmetric int4 pack ([GLM-C] §05 quantize_rows, §06 pack_int4) */
/* ------------------------------------------------------------------------ */

/* w [O][I] fp32 row-major -> q [O][(I+1)/2] bytes, s [O] fp32.
 * s = max|w|/7 with a 1e-8 floor; q = rint(w/s) clamped to [-7, 7]; the
 * nibble of column 2j is the low half of byte j, column 2j+1 the high half. */
void orc_pack_int4_row(const float *w, int64_t O, int64_t I, uint8_t *q, float *s)
{
    int64_t rb = (I + 1) / 2;
    for (int64_t o = 0; o < O; ++o) {
        const float *wr = w + o * I;
        float amax = 0.0f;
        for (int64_t i = 0; i < I; ++i) {
            float a = fabsf(wr[i]);
            if (a > amax) amax = a;
        }
        float sc = amax / 7.0f;
        if (sc < 1e-8f) sc = 1e-8f;
        s[o] = sc;
        uint8_t *qr = q + o * rb;
        memset(qr, 0, (size_t)rb);
        for (int64_t i = 0; i < I; ++i) {
            int v = (int)rintf(wr[i] / sc);
            if (v > 7) v = 7;
            if (v < -7) v = -7;
            uint8_t nib = (uint8_t)(v & 0xF);
            if (i & 1) qr[i >> 1] |= (uint8_t)(nib << 4);
            else qr[i >> 1] |= nib;
        }
    }
}

/* Signed code of column i of a packed row. */
static int nib_signed(const uint8_t *row, int64_t i)
{
    int v = (i & 1) ? (row[i >> 1] >> 4) : (row[i >> 1] & 0xF);
    return v >= 8 ? v - 16 : v;
}

static int nib_unsigned(const uint8_t *row, int64_t i)
{
    return (i & 1) ? (row[i >> 1] >> 4) : (row[i >> 1] & 0xF);
}

/* O3 (row): the codes as int8, q [O][(I+1)/2] -> qv [O][I]. */
void orc_unpack_int4_row(const uint8_t *q, int64_t O, int64_t I, int8_t *qv)
{
    int64_t rb = (I + 1) / 2;
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i) qv[o * I + i] = (int8_t)nib_signed(q + o * rb, i);
}

/* O3 (row): dequantised weights w' = q * s in fp64 (exact). */
void orc_dequant_int4_row(const uint8_t *q, const float *s, int64_t O, int64_t I, double *w)
{
    int64_t rb = (I + 1) / 2;
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i)
            w[o * I + i] = (double)nib_signed(q + o * rb, i) * (double)s[o];
}

/* ------------------------------------------------------------------------ */
/* O1b: per-row symmetric int8 ([GLM-C] §05 quantize_rows with bits = 8: the  */
/* streaming engine's expert format, and the dense precision of the           */
/* converted model, §06-07)                                                   */
/* ------------------------------------------------------------------------ */

/* w [O][I] -> q [O][I] int8, s [O]: s = max|w| / 127 floored at 1e-8,
 * q = rint(w / s) clamped to [-128, 127]. */
void orc_pack_int8_row(const float *w, int64_t O, int64_t I, int8_t *q, float *s)
{
    for (int64_t o = 0; o < O; ++o) {
        const float *wr = w + o * I;
        float amax = 0.0f;
        for (int64_t i = 0; i < I; ++i)
            if (fabsf(wr[i]) > amax) amax = fabsf(wr[i]);
        float sc = amax / 127.0f;
        if (sc < 1e-8f) sc = 1e-8f;
        s[o] = sc;
        for (int64_t i = 0; i < I; ++i) {
            int v = (int)rintf(wr[i] / sc);
            if (v > 127) v = 127;
            if (v < -128) v = -128;
            q[o * I + i] = (int8_t)v;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O0: the step before the path, the checkpoint converter ([GLM-C] §06):      */
/* FP8 E4M3 weights with one fp32 inverse scale per 128 x 128 block, or bf16, */
/* decoded to fp32, then packed as O1; and the converter's container, which   */
/* stores code + 8.                                                           */
/* ------------------------------------------------------------------------ */

/* FP8 E4M3 of the "fn" kind the checkpoint's dtype names (float8_e4m3fn):
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
 * subnormal (m/8 * 2^-6); no infinities; S.1111.111 is NaN.  Exact. */
float orc_fp8_e4m3_to_f32(uint8_t b)
{
    int neg = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(neg ? -v : v);
}

/* Block-scale decode: w[o][i] = fp8(q[o][i]) * sinv[o/B][i/B], one fp32
 * multiply, sinv [ceil(O/B)][ceil(I/B)] row-major; the page repeats the
 * scale tensor over each B x B block and crops it to [O, I] (B = 128). */
void orc_dequant_fp8_block(const uint8_t *q, const float *sinv, int64_t O, int64_t I, int64_t B,
                           float *w)
{
    int64_t nbi = (I + B - 1) / B;
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i) {
            float a = orc_fp8_e4m3_to_f32(q[o * I + i]);
            float sc = sinv[(o / B) * nbi + i / B];
            w[o * I + i] = a * sc;
        }
}

/* bf16 -> fp32, exact (the page's .to(float32) of non-FP8 tensors). */
void orc_bf16_to_f32(const uint16_t *b, int64_t n, float *w)
{
    for (int64_t i = 0; i < n; ++i) w[i] = bf16_to_f32(b[i]);
}

/* The converter's own packer, bits = 4: s = amax/7 floored at 1e-8, code =
 * rint(w/s) clamped to [-8, 7], stored offset binary (code + 8), column 2j
 * in the low nibble of byte j.  I even.  q [O][I/2], s [O]. */
void orc_convert_int4_container(const float *w, int64_t O, int64_t I, uint8_t *q, float *s)
{
    for (int64_t o = 0; o < O; ++o) {
        const float *wr = w + o * I;
        float amax = 0.0f;
        for (int64_t i = 0; i < I; ++i)
            if (fabsf(wr[i]) > amax) amax = fabsf(wr[i]);
        float sc = amax / 7.0f;
        if (sc < 1e-8f) sc = 1e-8f;
        s[o] = sc;
        for (int64_t j = 0; j < I / 2; ++j) {
            int v[2];
            for (int h = 0; h < 2; ++h) {
                v[h] = (int)rintf(wr[2 * j + h] / sc);
                if (v[h] > 7) v[h] = 7;
                if (v[h] < -8) v[h] = -8;
            }
            q[o * (I / 2) + j] = (uint8_t)((v[0] + 8) | ((v[1] + 8) << 4));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O2: affine int4, group size 64 along the input dim ([EDGE0] §三)           */
/* ------------------------------------------------------------------------ */

/* w [O][I] -> q [O][I/2] (unsigned nibbles), scmn [O][I/64][2] bf16
 * (element 0 = scale, element 1 = min).  I must be a multiple of 64. */
void orc_pack_affine_g64(const float *w, int64_t O, int64_t I, uint8_t *q, uint16_t *scmn)
{
    int64_t G = I / 64, rb = I / 2;
    for (int64_t o = 0; o < O; ++o) {
        uint8_t *qr = q + o * rb;
        memset(qr, 0, (size_t)rb);
        for (int64_t g = 0; g < G; ++g) {
            const float *wg = w + o * I + g * 64;
            float lo = wg[0], hi = wg[0];
            for (int i = 1; i < 64; ++i) {
                if (wg[i] < lo) lo = wg[i];
                if (wg[i] > hi) hi = wg[i];
            }
            uint16_t sc = f32_to_bf16_rne((hi - lo) / 15.0f);
            uint16_t mn = f32_to_bf16_rne(lo);
            float scv = bf16_to_f32(sc), mnv = bf16_to_f32(mn);
            for (int i = 0; i < 64; ++i) {
                int v = 0;
                if (scv != 0.0f) {
                    v = (int)rintf((wg[i] - mnv) / scv);
                    if (v < 0) v = 0;
                    if (v > 15) v = 15;
                }
                int64_t col = g * 64 + i;
                if (col & 1) qr[col >> 1] |= (uint8_t)(v << 4);
                else qr[col >> 1] |= (uint8_t)v;
            }
            scmn[(o * G + g) * 2 + 0] = sc;
            scmn[(o * G + g) * 2 + 1] = mn;
        }
    }
}

/* O3 (affine): w' = q * scale + min in fp64 (exact). */
void orc_dequant_affine_g64(const uint8_t *q, const uint16_t *scmn, int64_t O, int64_t I, double *w)
{
    int64_t G = I / 64, rb = I / 2;
    for (int64_t o = 0; o < O; ++o)
        for (int64_t i = 0; i < I; ++i) {
            int64_t g = i / 64;
            double sc = bf16_to_f32(scmn[(o * G + g) * 2 + 0]);
            double mn = bf16_to_f32(scmn[(o * G + g) * 2 + 1]);
            w[o * I + i] = (double)nib_unsigned(q + o * rb, i) * sc + mn;
        }
}

/* ------------------------------------------------------------------------ */
/* Expert blob: gate | up | down packed codes, then their scales             */
/* ([GLM-C] §13 contiguous slab; [COLI] §2.2 ESlot slab + fslab).            */
/*   row:    Qg[I][H/2] Qu[I][H/2] Qd[H][I/2] sg[I] su[I] sd[H] (fp32)         */
/*   affine: Qg Qu Qd Ag[I][H/64][2] Au[I][H/64][2] Ad[H][I/64][2] (bf16)     */
/* ------------------------------------------------------------------------ */

int orc_pack_expert(int fmt, int64_t H, int64_t I, const float *Wg, const float *Wu,
                    const float *Wd, uint8_t *blob)
{
    if (fmt == ORC_W_INT8_ROW) {
        int8_t *q = (int8_t *)blob;
        float *sc = (float *)(blob + 3 * H * I);
        orc_pack_int8_row(Wg, I, H, q, sc);
        orc_pack_int8_row(Wu, I, H, q + I * H, sc + I);
        orc_pack_int8_row(Wd, H, I, q + 2 * I * H, sc + 2 * I);
        return 0;
    }
    int64_t gq = I * (H / 2), dq = H * (I / 2);
    uint8_t *qg = blob, *qu = blob + gq, *qd = blob + 2 * gq, *sc = blob + 2 * gq + dq;
    if (fmt == ORC_W_INT4_ROW) {
        orc_pack_int4_row(Wg, I, H, qg, (float *)sc);
        orc_pack_int4_row(Wu, I, H, qu, (float *)(sc + 4 * I));
        orc_pack_int4_row(Wd, H, I, qd, (float *)(sc + 8 * I));
        return 0;
    }
    if (fmt == ORC_W_INT4_AFFINE_G64) {
        int64_t ga = I * (H / 64) * 2 * 2;
        orc_pack_affine_g64(Wg, I, H, qg, (uint16_t *)sc);
        orc_pack_affine_g64(Wu, I, H, qu, (uint16_t *)(sc + ga));
        orc_pack_affine_g64(Wd, H, I, qd, (uint16_t *)(sc + 2 * ga));
        return 0;
    }
    return -1;
}

/* Dequantise all three matrices of a blob into fp64 arrays
 * wg [I][H], wu [I][H], wd [H][I]. */
int orc_dequant_expert(int fmt, int64_t H, int64_t I, const uint8_t *blob, double *wg,
                       double *wu, double *wd)
{
    if (fmt == ORC_W_INT8_ROW) {
        const int8_t *q = (const int8_t *)blob;
        const float *s = (const float *)(blob + 3 * H * I);
        for (int64_t i = 0; i < I * H; ++i) wg[i] = (double)q[i] * (double)s[i / H];
        for (int64_t i = 0; i < I * H; ++i) wu[i] = (double)q[I * H + i] * (double)s[I + i / H];
        for (int64_t i = 0; i < H * I; ++i) wd[i] = (double)q[2 * I * H + i] * (double)s[2 * I + i / I];
        return 0;
    }
    int64_t gq = I * (H / 2), dq = H * (I / 2);
    const uint8_t *qg = blob, *qu = blob + gq, *qd = blob + 2 * gq, *sc = blob + 2 * gq + dq;
    if (fmt == ORC_W_INT4_ROW) {
        const float *s = (const float *)sc;
        orc_dequant_int4_row(qg, s, I, H, wg);
        orc_dequant_int4_row(qu, s + I, I, H, wu);
        orc_dequant_int4_row(qd, s + 2 * I, H, I, wd);
        return 0;
    }
    if (fmt == ORC_W_INT4_AFFINE_G64) {
        int64_t ga = I * (H / 64) * 2;
        const uint16_t *a = (const uint16_t *)sc;
        orc_dequant_affine_g64(qg, a, I, H, wg);
        orc_dequant_affine_g64(qu, a + ga, I, H, wu);
        orc_dequant_affine_g64(qd, a + 2 * ga, H, I, wd);
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* O6: one SwiGLU expert on one token ([GLM-C] §11 expert_gate_up ->          */
/* silu(g)*u -> down; [FLOW] Step 6b; [GLM-C] §04 siluf).                     */
/* The plain definition: dequantise, then fp64 dot products.                 */
/* ------------------------------------------------------------------------ */

static double silu_d(double z) { return z / (1.0 + exp(-z)); }

/* One row of a blob matrix, dequantised into fp64. */
static void dequant_row(int fmt, const uint8_t *q, const uint8_t *sc, int64_t row, int64_t in,
                        double *out)
{
    if (fmt == ORC_W_INT4_ROW) {
        const uint8_t *r = q + row * (in / 2);
        double s = (double)((const float *)sc)[row];
        for (int64_t i = 0; i < in; ++i) out[i] = (double)nib_signed(r, i) * s;
    } else if (fmt == ORC_W_INT8_ROW) {
        const int8_t *r = (const int8_t *)q + row * in;
        double s = (double)((const float *)sc)[row];
        for (int64_t i = 0; i < in; ++i) out[i] = (double)r[i] * s;
    } else {
        const uint8_t *r = q + row * (in / 2);
        const uint16_t *a = (const uint16_t *)sc + row * (in / 64) * 2;
        for (int64_t i = 0; i < in; ++i) {
            double s = bf16_to_f32(a[(i / 64) * 2 + 0]);
            double m = bf16_to_f32(a[(i / 64) * 2 + 1]);
            out[i] = (double)nib_unsigned(r, i) * s + m;
        }
    }
}

/* x [H] -> y [H]; h [I] (optional) receives silu(g)*u. */
int orc_expert(int fmt, int64_t H, int64_t I, const uint8_t *blob, const float *x, float *y,
               float *h_out)
{
    if (fmt != ORC_W_INT4_ROW && fmt != ORC_W_INT4_AFFINE_G64 && fmt != ORC_W_INT8_ROW) return -1;
    int64_t gq = I * (H / 2), dq = H * (I / 2);
    if (fmt == ORC_W_INT8_ROW) {
        gq = I * H;
        dq = H * I;
    }
    const uint8_t *qg = blob, *qu = blob + gq, *qd = blob + 2 * gq, *sc = blob + 2 * gq + dq;
    const uint8_t *scg, *scu, *scd;
    if (fmt == ORC_W_INT4_ROW || fmt == ORC_W_INT8_ROW) {
        scg = sc;
        scu = sc + 4 * I;
        scd = sc + 8 * I;
    } else {
        int64_t ga = I * (H / 64) * 2 * 2;
        scg = sc;
        scu = sc + ga;
        scd = sc + 2 * ga;
    }
    int64_t mx = H > I ? H : I;
    double *row = (double *)malloc(sizeof(double) * (size_t)mx);
    float *h = (float *)malloc(sizeof(float) * (size_t)I);
    if (!row || !h) {
        free(row);
        free(h);
        return -2;
    }
    for (int64_t o = 0; o < I; ++o) {
        double ag = 0.0, au = 0.0;
        dequant_row(fmt, qg, scg, o, H, row);
        for (int64_t i = 0; i < H; ++i) ag += row[i] * (double)x[i];
        dequant_row(fmt, qu, scu, o, H, row);
        for (int64_t i = 0; i < H; ++i) au += row[i] * (double)x[i];
        float g = (float)ag, u = (float)au;
        h[o] = (float)(silu_d((double)g) * (double)u);
    }
    for (int64_t d = 0; d < H; ++d) {
        double acc = 0.0;
        dequant_row(fmt, qd, scd, d, I, row);
        for (int64_t o = 0; o < I; ++o) acc += row[o] * (double)h[o];
        y[d] = (float)acc;
    }
    if (h_out) memcpy(h_out, h, sizeof(float) * (size_t)I);
    free(row);
    free(h);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O4: router -- fp32 GEMV, sigmoid, selection on sigmoid + bias, weights    */
/* from the unbiased sigmoid ([GLM-C] §11; [EDGE0] §七 sigmoid-group formula  */
/* with n_group = 1, as [COLI] §1.2 asserts; [FLOW] Step 6a sizes).           */
/* ------------------------------------------------------------------------ */

/* x [T][H], Wr [E][H], bias [E] -> ids [T][K] (rank order), wts [T][K].
 * logits_out [T][E], sig_out [T][E] (optional) receive the fp32 logit and
 * sigmoid.  gap_k [T] (optional) = c(K-th) - c((K+1)-th) (or +inf when
 * K == E); gap_in [T] (optional) = smallest gap between consecutive chosen
 * ranks (or +inf when K == 1).  Selection: K passes, each taking the
 * not-yet-taken expert with the strictly largest c, scanning ids upward from
 * a start value of -1e30 (so equal scores go to the lower id). */
/* O4b: group-limited selection ([EDGE0] §七, the sigmoid-group family, rule
 * ②: rank the groups by the sum of their two best scores, keep G groups, mask
 * the rest, then take the top K among the kept groups; rule ① makes the
 * scores the biased c = σ + b).  The E experts form n_group groups of
 * E/n_group consecutive ids.  A group's score is the fp32 sum of its two
 * largest c.  topk_group passes each keep the not-yet-kept group with the
 * strictly largest score (scanning groups upward from -1e30, so equal scores
 * keep the lower group); the experts of the other groups are excluded, and
 * the K experts are taken from the rest exactly as in O4.  n_group = 1 is O4.
 * gap_g [T] (optional) = score of the last kept group - the largest score of
 * an excluded group (+inf when every group is kept).  gap_k is then taken
 * among the kept experts (+inf when they are exactly K). */
/* O4c: softmax scoring ([EDGE0] §七 softmax-top-k family; [GLM-C] §05 the
 * olmoe prototype's moe step): g = softmax(l) over all E logits, shifted by
 * the largest logit, in fp64 and rounded to fp32; the selection scans g (no
 * bias) as O4 scans c; the weights are g (norm_topk = 0, the prototype's
 * w = val) or g / (sum of the chosen g) (norm_topk = 1, renormalised to one),
 * times routed_scale.  Groups apply to sigmoid scoring only.  For softmax,
 * gap_k and gap_in are logit differences (the order of g is that of l). */
int orc_route_full(const float *x, int T, int64_t H, const float *Wr, const float *bias, int E,
                   int K, int scoring, int n_group, int topk_group, float routed_scale,
                   int norm_topk, int32_t *ids, float *wts, float *logits_out, float *sig_out,
                   double *gap_k, double *gap_in, double *gap_g)
{
    if (K < 1 || K > E) return -1;
    if (scoring != 0 && scoring != 1) return -1;
    if (scoring == 1 && n_group != 1) return -1;
    if (n_group < 1 || E % n_group != 0 || topk_group < 1 || topk_group > n_group) return -1;
    const int gsz = E / n_group;
    if (n_group > 1 && gsz < 2) return -1;
    const int n_kept = topk_group * gsz;  /* experts left after the group step */
    if (K > n_kept) return -1;
    float *sig = (float *)malloc(sizeof(float) * (size_t)E);
    float *c = (float *)malloc(sizeof(float) * (size_t)E);
    char *taken = (char *)malloc((size_t)E);
    int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    float *gs = (float *)malloc(sizeof(float) * (size_t)n_group);
    char *gkept = (char *)malloc((size_t)n_group);
    float *lg = (float *)malloc(sizeof(float) * (size_t)E);
    if (!sig || !c || !taken || !rank || !gs || !gkept || !lg) {
        free(sig);
        free(c);
        free(taken);
        free(rank);
        free(gs);
        free(gkept);
        free(lg);
        return -2;
    }
    for (int t = 0; t < T; ++t) {
        const float *xt = x + (int64_t)t * H;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            const float *wr = Wr + (int64_t)e * H;
            for (int64_t i = 0; i < H; ++i) acc += (double)wr[i] * (double)xt[i];
            float l = (float)acc;
            lg[e] = l;
            if (scoring == 0) {
                sig[e] = (float)(1.0 / (1.0 + exp(-(double)l)));
                c[e] = sig[e] + bias[e];
            }
            if (logits_out) logits_out[(int64_t)t * E + e] = l;
        }
        if (scoring == 1) {
            double m = -INFINITY, z = 0.0;
            for (int e = 0; e < E; ++e)
                if ((double)lg[e] > m) m = (double)lg[e];
            for (int e = 0; e < E; ++e) z += exp((double)lg[e] - m);
            for (int e = 0; e < E; ++e) {
                sig[e] = (float)(exp((double)lg[e] - m) / z);
                c[e] = sig[e];
            }
        }
        if (sig_out)
            for (int e = 0; e < E; ++e) sig_out[(int64_t)t * E + e] = sig[e];
        memset(taken, 0, (size_t)E);
        if (n_group > 1) {
            /* group scores: the sum of each group's two largest c */
            for (int g = 0; g < n_group; ++g) {
                float a = -INFINITY, b2 = -INFINITY;
                for (int e = g * gsz; e < (g + 1) * gsz; ++e) {
                    if (c[e] > a) {
                        b2 = a;
                        a = c[e];
                    } else if (c[e] > b2) {
                        b2 = c[e];
                    }
                }
                gs[g] = a + b2;
            }
            memset(gkept, 0, (size_t)n_group);
            float last = 0.f;
            for (int kg = 0; kg < topk_group; ++kg) {
                int best = -1;
                float bv = -1e30f;
                for (int g = 0; g < n_group; ++g)
                    if (!gkept[g] && gs[g] > bv) {
                        bv = gs[g];
                        best = g;
                    }
                if (best < 0) { /* non-finite scores: not a valid input */
                    free(sig);
                    free(c);
                    free(taken);
                    free(rank);
                    free(gs);
                    free(gkept);
                    free(lg);
                    return -3;
                }
                gkept[best] = 1;
                last = bv;
            }
            double next = -INFINITY;
            for (int g = 0; g < n_group; ++g)
                if (!gkept[g] && (double)gs[g] > next) next = (double)gs[g];
            if (gap_g) gap_g[t] = topk_group < n_group ? (double)last - next : INFINITY;
            /* the excluded groups' experts are never selectable */
            for (int e = 0; e < E; ++e)
                if (!gkept[e / gsz]) taken[e] = 1;
        } else if (gap_g) {
            gap_g[t] = INFINITY;
        }
        int npass = K < n_kept ? K + 1 : K;
        for (int kk = 0; kk < npass; ++kk) {
            int best = -1;
            float bv = -1e30f;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && c[e] > bv) {
                    bv = c[e];
                    best = e;
                }
            if (best < 0) { /* non-finite scores: not a valid input */
                free(sig);
                free(c);
                free(taken);
                free(rank);
                free(gs);
                free(gkept);
                free(lg);
                return -3;
            }
            rank[kk] = best;
            taken[best] = 1;
        }
        double ssum = 0.0;
        for (int kk = 0; kk < K; ++kk) ssum += (double)sig[rank[kk]];
        for (int kk = 0; kk < K; ++kk) {
            double w = (double)sig[rank[kk]];
            if (norm_topk) w = w / (ssum + 1e-20);
            ids[(int64_t)t * K + kk] = rank[kk];
            wts[(int64_t)t * K + kk] = (float)(w * (double)routed_scale);
        }
        /* gaps in selection-score units (sigmoid) or logit units (softmax) */
        const float *gv = scoring == 1 ? lg : c;
        if (gap_k) gap_k[t] = K < n_kept ? (double)gv[rank[K - 1]] - (double)gv[rank[K]] : INFINITY;
        if (gap_in) {
            double m = INFINITY;
            for (int kk = 0; kk + 1 < K; ++kk) {
                double gdiff = (double)gv[rank[kk]] - (double)gv[rank[kk + 1]];
                if (gdiff < m) m = gdiff;
            }
            gap_in[t] = m;
        }
    }
    free(sig);
    free(c);
    free(taken);
    free(rank);
    free(gs);
    free(gkept);
    free(lg);
    return 0;
}

/* O4b with sigmoid scoring. */
int orc_route_groups(const float *x, int T, int64_t H, const float *Wr, const float *bias, int E,
                     int K, int n_group, int topk_group, float routed_scale, int norm_topk,
                     int32_t *ids, float *wts, float *logits_out, float *sig_out, double *gap_k,
                     double *gap_in, double *gap_g)
{
    return orc_route_full(x, T, H, Wr, bias, E, K, 0, n_group, topk_group, routed_scale, norm_topk,
                          ids, wts, logits_out, sig_out, gap_k, gap_in, gap_g);
}

/* O4 (one group: every expert selectable). */
int orc_route(const float *x, int T, int64_t H, const float *Wr, const float *bias, int E, int K,
              float routed_scale, int norm_topk, int32_t *ids, float *wts, float *logits_out,
              float *sig_out, double *gap_k, double *gap_in)
{
    return orc_route_groups(x, T, H, Wr, bias, E, K, 1, 1, routed_scale, norm_topk, ids, wts,
                            logits_out, sig_out, gap_k, gap_in, NULL);
}

/* ------------------------------------------------------------------------ */
/* O5: token -> expert bucketing, a stable counting sort of the T*K          */
/* assignments a = t*K + k by expert id ([GLM-C] §11 batch expert union:     */
/* each expert the batch uses is read once).                                 */
/* ------------------------------------------------------------------------ */

/* ids [T*K] -> cnt [E], off [E+1], perm [T*K], active [E] (ascending ids of
 * experts with cnt > 0), *n_active. */
int orc_bucket(const int32_t *ids, int T, int K, int E, int32_t *cnt, int32_t *off,
               int32_t *perm, int32_t *active, int32_t *n_active)
{
    int64_t n = (int64_t)T * K;
    for (int e = 0; e < E; ++e) cnt[e] = 0;
    for (int64_t a = 0; a < n; ++a) {
        if (ids[a] < 0 || ids[a] >= E) return -1;
        cnt[ids[a]]++;
    }
    off[0] = 0;
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];
    int32_t *fill = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    if (!fill) return -2;
    for (int e = 0; e < E; ++e) fill[e] = off[e];
    for (int64_t a = 0; a < n; ++a) perm[fill[ids[a]]++] = (int32_t)a;
    free(fill);
    int na = 0;
    for (int e = 0; e < E; ++e)
        if (cnt[e] > 0) active[na++] = e;
    *n_active = na;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* O7: combine -- out_t = sum_s shared_s(x_t) + sum_k w_tk * y_tk             */
/* ([FLOW] Step 6d; [GLM-C] §11 scatter-add of w * h).                        */
/* ------------------------------------------------------------------------ */

/* y_routed [T*K][H] (row t*K+k), wts [T*K], y_shared [n_shared][T][H]. */
void orc_combine(int T, int K, int64_t H, int n_shared, const float *y_routed, const float *wts,
                 const float *y_shared, float *out)
{
    for (int t = 0; t < T; ++t)
        for (int64_t d = 0; d < H; ++d) {
            double acc = 0.0;
            for (int s = 0; s < n_shared; ++s)
                acc += (double)y_shared[((int64_t)s * T + t) * H + d];
            for (int k = 0; k < K; ++k)
                acc += (double)wts[(int64_t)t * K + k] *
                       (double)y_routed[((int64_t)t * K + k) * H + d];
            out[(int64_t)t * H + d] = (float)acc;
        }
}

/* ------------------------------------------------------------------------ */
/* Whole layer: route -> experts (looked up by id) -> combine.               */
/* blobs[e] is expert e's blob, or NULL if it is not resident.               */
/* Returns 0, or -5 if a selected expert is not resident.                    */
/* ------------------------------------------------------------------------ */

int orc_moe_layer_full(const float *x, int T, int64_t H, int64_t I, int E, int K, int fmt,
                       int shared_fmt, const float *Wr, const float *bias, int scoring,
                       int n_group, int topk_group, float routed_scale, int norm_topk,
                       const uint8_t *const *blobs, int n_shared,
                       const uint8_t *const *shared_blobs, float *out, int32_t *ids, float *wts)
{
    if (shared_fmt == 0) shared_fmt = fmt;
    int rc = orc_route_full(x, T, H, Wr, bias, E, K, scoring, n_group, topk_group, routed_scale,
                            norm_topk, ids, wts, NULL, NULL, NULL, NULL, NULL);
    if (rc) return rc;
    float *yr = (float *)malloc(sizeof(float) * (size_t)((int64_t)T * K * H));
    float *ys = (float *)malloc(sizeof(float) * (size_t)((int64_t)(n_shared > 0 ? n_shared : 1) * T * H));
    if (!yr || !ys) {
        free(yr);
        free(ys);
        return -2;
    }
    for (int t = 0; t < T && rc == 0; ++t) {
        const float *xt = x + (int64_t)t * H;
        for (int k = 0; k < K && rc == 0; ++k) {
            const uint8_t *b = blobs[ids[(int64_t)t * K + k]];
            if (!b) rc = -5;
            else rc = orc_expert(fmt, H, I, b, xt, yr + ((int64_t)t * K + k) * H, NULL);
        }
        for (int s = 0; s < n_shared && rc == 0; ++s)
            rc = orc_expert(shared_fmt, H, I, shared_blobs[s], xt, ys + ((int64_t)s * T + t) * H,
                            NULL);
    }
    if (rc == 0) orc_combine(T, K, H, n_shared, yr, wts, ys, out);
    free(yr);
    free(ys);
    return rc;
}

int orc_moe_layer(const float *x, int T, int64_t H, int64_t I, int E, int K, int fmt,
                  const float *Wr, const float *bias, float routed_scale, int norm_topk,
                  const uint8_t *const *blobs, int n_shared, const uint8_t *const *shared_blobs,
                  float *out, int32_t *ids, float *wts)
{
    return orc_moe_layer_full(x, T, H, I, E, K, fmt, 0, Wr, bias, 0, 1, 1, routed_scale, norm_topk,
                              blobs, n_shared, shared_blobs, out, ids, wts);
}

/* ------------------------------------------------------------------------ */
/* O8: chaining -- unit-weight RMSNorm ([GLM-C] §04 rmsnorm, double mean     */
/* square) and the residual x <- x + moe(rmsnorm(x)) ([GLM-C] §04 layer order) */
/* ------------------------------------------------------------------------ */

void orc_rmsnorm(const float *x, int T, int64_t H, float eps, float *out)
{
    for (int t = 0; t < T; ++t) {
        const float *xt = x + (int64_t)t * H;
        double ms = 0.0;
        for (int64_t i = 0; i < H; ++i) ms += (double)xt[i] * (double)xt[i];
        double r = 1.0 / sqrt(ms / (double)H + (double)eps);
        for (int64_t i = 0; i < H; ++i) out[(int64_t)t * H + i] = (float)((double)xt[i] * r);
    }
}

/* x [T][H] updated in place: x <- x + moe(rmsnorm(x)), the layer of
 * orc_moe_layer_full (any scoring, grouping and shared format). */
int orc_residual_layer(float *x, int T, int64_t H, int64_t I, int E, int K, int fmt,
                       int shared_fmt, const float *Wr, const float *bias, int scoring,
                       int n_group, int topk_group, float routed_scale, int norm_topk,
                       const uint8_t *const *blobs, int n_shared,
                       const uint8_t *const *shared_blobs, float eps, int32_t *ids, float *wts)
{
    float *xn = (float *)malloc(sizeof(float) * (size_t)((int64_t)T * H));
    float *m = (float *)malloc(sizeof(float) * (size_t)((int64_t)T * H));
    if (!xn || !m) {
        free(xn);
        free(m);
        return -2;
    }
    orc_rmsnorm(x, T, H, eps, xn);
    int rc = orc_moe_layer_full(xn, T, H, I, E, K, fmt, shared_fmt, Wr, bias, scoring, n_group,
                                topk_group, routed_scale, norm_topk, blobs, n_shared,
                                shared_blobs, m, ids, wts);
    if (rc == 0)
        for (int64_t j = 0; j < (int64_t)T * H; ++j) x[j] = x[j] + m[j];
    free(xn);
    free(m);
    return rc;
}
