/*
 * moe.h -- C ABI of the MI355X (gfx950) int4-weight MoE FFN library.
 *
 * The library computes one MoE FFN step of a GLM-5.2-style decoder layer:
 *   router:   logits = x . Wr^T (fp32), sigma = 1/(1+exp(-logits)),
 *             choose top-K experts by sigma + bias (equal scores: lower id),
 *             w_k = routed_scale * sigma_k / (sum_j sigma_j + 1e-20)
 *   experts:  y_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)), weights int4
 *   combine:  out = sum_s shared_s(x) + sum_k w_k y_{id_k}(x)
 * Sources, cited by page title and section:
 *   [GLM-C] "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" (reader.mx) §11 (routing
 *           and expert execution: sigmoid + correction bias picks, the plain
 *           sigmoid weighs; batch expert union; SwiGLU on gathered rows),
 *           §06 (int4 pack: per-row absmax scale, two codes per byte, first
 *           code in the low nibble), §13 (one contiguous g|u|d slab per
 *           expert, a GPU hot tier of resident experts);
 *   [FLOW]  GLM-5.2 dataflow page (devpress.csdn.net) §三 Step 6 (6a router
 *           6144->256 top-8, 6b SwiGLU experts 6144->2048->6144, 6c the
 *           always-active shared expert, 6d output = routed sum + shared);
 *   [COLI]  "初始化与权重加载" (colibrì analysis) §1.1-1.2 (n_group,
 *           topk_group, norm_topk, routed_scale; GLM-5.2 has n_group = 1),
 *           §2.2 (ESlot: an expert slot addressed by expert id);
 *   [EDGE0] Edge0 write-up (magicnetworld.com) §三 (affine int4, group size
 *           64), §七 (sigmoid-group routing: biased selection scores, group
 *           ranking by the sum of the two best scores, G groups kept, weights
 *           with the 1e-20 term), §十四 (routing indices mapped through a
 *           slot table on the device).
 *
 * Conventions for every entry point:
 *   - return MOE_OK (0) or a negative MOE_E_* code; nothing calls exit();
 *   - argument, size and range checks are synchronous and leave no work
 *     enqueued when they fail;
 *   - "device pointer" means memory the HIP runtime can address from the
 *     context's device (hipMalloc or a torch CUDA tensor's data_ptr());
 *     "host or device pointer" accepts either (copied with hipMemcpyDefault);
 *   - all GPU work is enqueued on the context's stream (see moe_set_stream)
 *     and is asynchronous unless stated otherwise;
 *   - a context is used by one host thread at a time (not thread-safe).
 * There is no CPU fallback: without a gfx950 device, moe_layer_create
 * fails with MOE_E_HIP.
 */
#ifndef MOE_INT4_H
#define MOE_INT4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;

/* status codes */
#define MOE_OK 0
#define MOE_E_ARG (-1)          /* bad argument: null, range, aliasing */
#define MOE_E_NOMEM (-2)        /* device allocation failed */
#define MOE_E_SIZE (-3)         /* blob size differs from moe_expert_bytes() */
#define MOE_E_SLOT (-4)         /* slot index out of range */
#define MOE_E_NOT_RESIDENT (-5) /* a selected expert had no slot (moe_status) */
#define MOE_E_HIP (-6)          /* a HIP runtime call failed */
#define MOE_E_UNSUPPORTED (-7)  /* configuration outside what the kernels do */
#define MOE_E_RANGE (-8)        /* an input row was not finite (moe_status) */
#define MOE_E_BUSY (-9)         /* slot still named by the slot table (asynchronous loads) */
#define MOE_E_WAIT (-10)        /* a kernel's bounded wait for other workgroups gave up (moe_status) */

/* slot-table value of an expert held by another GPU (see moe_map_expert) */
#define MOE_SLOT_REMOTE (-2)

/* expert weight formats (layout of an expert blob, see moe_load_expert) */
#define MOE_W_INT4_ROW 1        /* symmetric int4, one fp32 scale per output row */
#define MOE_W_INT4_AFFINE_G64 2 /* affine int4, bf16 scale and min per 64 inputs */
#define MOE_W_INT8_ROW 3        /* symmetric int8, one fp32 scale per output row (shared experts) */

/* router scoring (moe_config.scoring) */
#define MOE_SCORE_SIGMOID 0 /* sigma(l) + bias selects, sigma weighs ([GLM-C] §11, [EDGE0] §七) */
#define MOE_SCORE_SOFTMAX 1 /* softmax(l) over all experts selects (no bias) and weighs: raw
                               (norm_topk = 0, the [GLM-C] §05 olmoe step) or renormalised
                               to one (norm_topk = 1, [EDGE0] §七 softmax-top-k); one group */

typedef struct moe_config {
    int hidden;         /* H, multiple of 256, at most 16384 (affine: multiple of 512) */
    int inter;          /* I, multiple of 256 */
    int n_experts;      /* E, 1..256 routed experts */
    int top_k;          /* K, 1..min(8, E) */
    int n_shared;       /* 0 or 1 always-active shared experts (weight 1) */
    int n_layers;       /* layers whose router/shared/slot table are held */
    int wfmt;           /* MOE_W_INT4_ROW or MOE_W_INT4_AFFINE_G64 */
    int n_group;        /* expert groups of the router, 1..64 dividing E, >= 2
                           experts each; 1 = plain top-K (GLM-5.2, [COLI] §1.2).
                           More: a group's score is the fp32 sum of its two
                           largest sigma + bias, the topk_group best groups are
                           kept (ties: lower group), top-K among their experts
                           ([EDGE0] §七) */
    int topk_group;     /* groups kept, 1..n_group, with K <= topk_group * E / n_group */
    float routed_scale; /* routed scaling factor (GLM-5.2: 2.5) */
    int norm_topk;      /* 1: renormalise chosen sigmas before scaling ([EDGE0] §七) */
    int n_slots;        /* expert slots in the HBM pool */
    int max_tokens;     /* largest T passed to moe_forward / moe_route */
    float rms_eps;      /* eps of the RMSNorm used by moe_forward_residual */
    int scoring;        /* MOE_SCORE_SIGMOID or MOE_SCORE_SOFTMAX */
    int shared_fmt;     /* shared experts' format: 0 (= wfmt) or MOE_W_INT8_ROW, the per-row
                         * int8 of [GLM-C] §05 quantize_rows (bits = 8), the dense precision
                         * of the converted model (§06-07).  Blob: Qg[I][H] Qu[I][H] Qd[H][I]
                         * int8 (two's complement), then sg[I] su[I] sd[H] fp32; weight =
                         * code * scale.  With int8 shared experts every forward runs the
                         * expert GEMVs (the grouped GEMM is not used). */
} moe_config;

/* Creates a context on the current HIP device ([GLM-C] §11: the layer's
 * shape and routing constants; [COLI] §1.1-1.2: n_group, topk_group,
 * norm_topk and routed_scale read from the model's config, an unsupported
 * combination stopping the load): allocates the slot pool
 * (n_slots * moe_expert_bytes), per-layer router weights, bias, shared
 * experts and slot table (all entries -1 = not resident), and a workspace
 * sized for max_tokens.  stream: a hipStream_t (NULL = default stream).
 * Errors: MOE_E_ARG (null/invalid field, topk_group outside 1..n_group),
 * MOE_E_UNSUPPORTED (n_group > 64 or not dividing E into groups of >= 2,
 * K > topk_group * E / n_group, E > 256, K > 8, H or I not a multiple of 256),
 * MOE_E_NOMEM, MOE_E_HIP (no device or not gfx950). */
int moe_layer_create(const moe_config *cfg, void *stream, moe_ctx **out);

/* Frees every allocation of the context (synchronises its stream first). */
void moe_destroy(moe_ctx *ctx);

/* Changes the stream later calls enqueue on. */
int moe_set_stream(moe_ctx *ctx, void *stream);

/* Bytes of one expert blob for the context's format and shape:
 *   MOE_W_INT4_ROW:        3*H*I/2 + 4*(2I + H)    (GLM 6144/2048: 18,915,328)
 *   MOE_W_INT4_AFFINE_G64: 3*H*I/2 + 12*H*I/64     (Edge0 2048/512: 1,769,472)
 * Returns 0 for a null context. */
size_t moe_expert_bytes(const moe_ctx *ctx);

/* Sets layer's router ([FLOW] §三 Step 6a: the 6144 -> 256 gate; [GLM-C]
 * §11: its fp32 weight and the correction bias added to the sigmoid before
 * the top-K): W [E][H] fp32 row-major, bias [E] fp32; host or device
 * pointers.  Synchronous: returns after the data is copied in.
 * Errors: MOE_E_ARG (null, layer out of range). */
int moe_set_router(moe_ctx *ctx, int layer, const float *W, const float *bias);

/* moe_set_router for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same result, staged through a fixed device array of the
 * library (16 MiB per device, enough for every router a context accepts:
 * E * H <= 256 * 16384) instead of a temporary; calls no allocating
 * routine.  Synchronous on the context's stream.  The array is shared by
 * every context on a device and keeps the last call's contents: calls that
 * overlap on one device (other threads, other streams) race; calls from
 * one thread never overlap.  Errors: MOE_E_ARG, MOE_E_SIZE (E * H beyond
 * the array), MOE_E_HIP. */
int moe_set_router_noalloc(moe_ctx *ctx, int layer, const float *W, const float *bias);

/* Copies one expert blob (host or device pointer, nbytes ==
 * moe_expert_bytes) into a pool slot ([GLM-C] §13 contiguous slab).
 * Blob layout, little-endian, row-major, output rows:
 *   MOE_W_INT4_ROW:  Qg[I][H/2] Qu[I][H/2] Qd[H][I/2] sg[I] su[I] sd[H]
 *     Q bytes hold two's-complement codes in [-7, 7]; column 2j in the low
 *     nibble of byte j, column 2j+1 in the high nibble; s fp32 row scales;
 *     weight = code * s.
 *   MOE_W_INT4_AFFINE_G64: Qg Qu Qd (as above, unsigned codes 0..15), then
 *     Ag[I][H/64][2] Au[I][H/64][2] Ad[H][I/64][2] bf16 pairs (scale, min);
 *     weight = code * scale + min for the group of 64 inputs it falls in.
 * The slot keeps the bytes in the library's own order (8-row interleave);
 * moe_read_slot gives the blob back.  Synchronous.  Does not map the slot.
 * Errors: MOE_E_SLOT, MOE_E_SIZE, MOE_E_ARG, MOE_E_HIP. */
int moe_load_expert(moe_ctx *ctx, int slot, const void *blob, size_t nbytes);

/* Quantises and packs fp32 weights already in device memory straight into
 * a slot: Wg [I][H], Wu [I][H], Wd [H][I] row-major device pointers.  Same
 * quantiser as moe_pack_int4_rows / moe_pack_affine_g64.  Asynchronous. */
int moe_pack_expert(moe_ctx *ctx, int slot, const float *Wg, const float *Wu, const float *Wd);

/* Checkpoint source kinds of the requantiser ([GLM-C] §06 FP8 to int4). */
#define MOE_SRC_F32 0      /* fp32 */
#define MOE_SRC_BF16 1     /* bf16 bit patterns (uint16) */
#define MOE_SRC_FP8_E4M3 2 /* FP8 E4M3 (fn: bias 7, no inf) codes with fp32 inverse scales,
                            * one per 128 x 128 block, [ceil(O/128)][ceil(In/128)] row-major;
                            * weight = fp8 value * its block's inverse scale (fp32 product) */

/* The converter step on the device ([GLM-C] §06): decodes a checkpoint
 * expert (Wg, Wu [I][H], Wd [H][I] row-major device pointers of kind src;
 * sinv_* the FP8 inverse scales, ignored otherwise) to fp32 and quantises
 * it into a slot in the layer's format, as moe_pack_expert does from fp32.
 * NaN codes give unspecified codes.  Asynchronous on the context's stream.
 * Errors: MOE_E_SLOT, MOE_E_ARG (null, unknown src, FP8 without scales),
 * MOE_E_HIP. */
int moe_requant_expert(moe_ctx *ctx, int slot, int src, const void *Wg, const void *Wu,
                       const void *Wd, const float *sinv_g, const float *sinv_u,
                       const float *sinv_d);

/* Imports one expert of the converter's int4 container ([GLM-C] §06: per
 * tensor, U8 codes [O][In/2] stored as code + 8, first column in the low
 * nibble, and fp32 row scales; weight = code * scale) into a slot: qg, qu
 * [I][H/2], qd [H][I/2], sg, su [I], sd [H]; host or device pointers.
 * Codes -8..7 are all accepted.  Row format only.  Synchronous.
 * Errors: MOE_E_SLOT, MOE_E_ARG, MOE_E_UNSUPPORTED (affine layer), MOE_E_HIP. */
int moe_import_expert(moe_ctx *ctx, int slot, const uint8_t *qg, const uint8_t *qu,
                      const uint8_t *qd, const float *sg, const float *su, const float *sd);

/* Shared expert s of a layer, from a blob (host or device; synchronous) or
 * from device fp32 weights (asynchronous), in the shared experts' format
 * (moe_config.shared_fmt; nbytes == moe_shared_bytes).  Errors: MOE_E_ARG,
 * MOE_E_SIZE (moe_import_shared: MOE_E_UNSUPPORTED for int8). */
int moe_set_shared(moe_ctx *ctx, int layer, int s, const void *blob, size_t nbytes);
int moe_pack_shared(moe_ctx *ctx, int layer, int s, const float *Wg, const float *Wu,
                    const float *Wd);
/* The shared expert s of a layer from a checkpoint source or the container,
 * as moe_requant_expert / moe_import_expert.  Errors: MOE_E_ARG and theirs. */
int moe_requant_shared(moe_ctx *ctx, int layer, int s, int src, const void *Wg, const void *Wu,
                       const void *Wd, const float *sinv_g, const float *sinv_u,
                       const float *sinv_d);
int moe_import_shared(moe_ctx *ctx, int layer, int s, const uint8_t *qg, const uint8_t *qu,
                      const uint8_t *qd, const float *sg, const float *su, const float *sd);

/* Points (layer, expert_id) at a slot, or unmaps it with slot = -1
 * ([COLI] §2.2 ESlot, [EDGE0] §十四 slot table).  Several layers or ids may
 * share a slot.  slot = MOE_SLOT_REMOTE marks an expert that lives on
 * another GPU (expert parallelism): a token that selects it gets no
 * contribution from it here and no status is raised (its partial sum comes
 * from the GPU that holds it), where an unmapped (-1) expert is skipped and
 * reported as MOE_E_NOT_RESIDENT.  Errors: MOE_E_ARG, MOE_E_SLOT. */
int moe_map_expert(moe_ctx *ctx, int layer, int expert_id, int slot);

/* --- residency: asynchronous loads, staged (sticky) slots, whole layers ---
 *
 * Edge0 write-up §十四: the staged executor keeps fixed slots reached
 * through a slot table and per step rewrites only the experts that changed;
 * the whole-layer path loads a layer's experts at once, overlapped with the
 * previous layer's GPU work.  "惊呆了！…" §13: an expert's three matrices
 * stored contiguously are read with one read into its slab.
 *
 * Asynchronous loads copy a slot image (an expert's bytes already in the
 * slot's own order, see moe_blob_to_image) from host memory (pinned for
 * the copy to overlap compute; device memory also works) on a copy stream
 * of the library's own.  Ordering is kept per slot: the compute stream
 * waits for a slot's load before the table names the slot or before the
 * library touches the slot on it; a load waits until forwards enqueued
 * before the slot's last table entry went (or before a synchronous write
 * into it) are done.  A slot still named by the table takes no
 * asynchronous load (MOE_E_BUSY).  The caller keeps an image valid until
 * the load is done (moe_sync_copies, or a synchronised forward that
 * follows the map). */

/* Table updates, in stream order on the context's stream, without a sync:
 * (layer, expert_ids[i]) -> slots[i] (-1 unmaps, MOE_SLOT_REMOTE marks an
 * expert held by another GPU).  Later entries for the
 * same id win.  Errors: MOE_E_ARG, MOE_E_SLOT, MOE_E_HIP. */
int moe_map_experts_async(moe_ctx *ctx, int layer, int n, const int *expert_ids,
                          const int *slots);

/* Loads one slot image (nbytes == moe_expert_bytes) into a slot that the
 * table does not name.  Returns once the copy is enqueued.
 * Errors: MOE_E_SLOT, MOE_E_SIZE, MOE_E_BUSY, MOE_E_ARG, MOE_E_HIP. */
int moe_load_image_async(moe_ctx *ctx, int slot, const void *image, size_t nbytes);

/* Whole-layer load: n slot images stored back to back (experts 0..n-1 of
 * the layer, nbytes == n * moe_expert_bytes) in one copy into slots
 * first_slot .. first_slot+n-1, then (layer, e) -> first_slot + e.
 * Errors: as moe_load_image_async. */
int moe_load_layer_async(moe_ctx *ctx, int layer, int first_slot, int n, const void *images,
                         size_t nbytes);

/* Waits for every load enqueued so far.  Errors: MOE_E_ARG, MOE_E_HIP. */
int moe_sync_copies(moe_ctx *ctx);

/* Staged slots: layer l owns slots first_slot + l*per_layer .. +per_layer-1
 * (none of them named by the table when staging starts).  Resets what the
 * staged slots are known to hold.  Errors: MOE_E_ARG, MOE_E_SLOT. */
int moe_set_staging(moe_ctx *ctx, int first_slot, int per_layer);

/* One step of the staged executor for a layer: the n distinct experts
 * expert_ids (n <= per_layer) become resident in the layer's staged slots.
 * Experts already held stay where they are (sticky); the others are loaded
 * from images[i] (slot images; only those loaded are read) into empty
 * slots first, then into the slots least recently wanted, whose old
 * experts leave the table.  Experts held but not wanted stay mapped.
 * *n_loaded (optional) = number of images loaded.  Asynchronous.
 * Errors: MOE_E_ARG (staging not set, n too large, bad or repeated id,
 * missing image), MOE_E_BUSY, MOE_E_HIP. */
int moe_stage_experts(moe_ctx *ctx, int layer, int n, const int *expert_ids,
                      const void *const *images, int *n_loaded);

/* The staged executor's slot choice, on the host (no context, no GPU):
 * held[n_slots] = expert held by each slot (-1 empty), last_used[n_slots]
 * = step it was last wanted; want[n_want] distinct ids.  slot_of[i] = slot
 * for want[i], load[i] = 1 if it must be loaded.  Wanted experts already
 * held keep their slot; the rest take empty slots (ascending), then the
 * slots with the smallest last_used (ties: lower slot).  Returns the
 * number of loads, or -1 for bad arguments (n_want > n_slots, a repeated
 * or negative id). */
int moe_sticky_plan(const int *held, const int64_t *last_used, int n_slots, const int *want,
                    int n_want, int *slot_of, int *load);

/* The slot image of an expert blob, on the host (no context, no GPU): the
 * blob's bytes in the slot's own order (8-row interleave, row-format codes
 * offset binary, affine pairs interleaved).  hidden and inter multiples of
 * 64.  Returns MOE_OK, MOE_E_ARG or MOE_E_SIZE. */
size_t moe_image_bytes(int wfmt, int hidden, int inter);
int moe_blob_to_image(int wfmt, int hidden, int inter, const void *blob, size_t nbytes,
                      void *image);

/* Shared expert s of a layer back out in its blob layout (nbytes ==
 * moe_shared_bytes).  Synchronous.  Errors: MOE_E_ARG, MOE_E_SIZE, MOE_E_HIP. */
int moe_read_shared(moe_ctx *ctx, int layer, int s, void *dst, size_t nbytes);
size_t moe_shared_bytes(const moe_ctx *ctx);

/* Copies a slot back out in blob layout to dst (host or device pointer).
 * Synchronous.  Errors: MOE_E_SLOT, MOE_E_SIZE, MOE_E_ARG. */
int moe_read_slot(moe_ctx *ctx, int slot, void *dst, size_t nbytes);

/* The MoE step: out[T][H] = moe(x[T][H]) for the given layer ([GLM-C] §11
 * moe(); [FLOW] Step 6).  x, out: device pointers to fp32 row-major
 * arrays that must not overlap; out is fully overwritten.  1 <= T <=
 * max_tokens.  A selected expert whose slot entry is -1 contributes zero
 * and is reported by moe_status.  Deterministic: the same inputs give
 * bitwise the same outputs.  Errors: MOE_E_ARG. */
int moe_forward(moe_ctx *ctx, const float *x, int T, int layer, float *out);

/* One chained layer in place: x <- x + moe(rmsnorm(x)), unit-weight
 * RMSNorm with eps = rms_eps ([GLM-C] §04 rmsnorm and layer order).
 * x: device pointer [T][H].  Errors: MOE_E_ARG. */
int moe_forward_residual(moe_ctx *ctx, float *x, int T, int layer);

/* Router only ([GLM-C] §11 routing: sigmoid + bias picks the top K, the
 * plain sigmoid of the picked experts weighs; [EDGE0] §七 renormalised
 * weights): ids [T][K] int32 (descending score), w [T][K] fp32, device
 * pointers.  Errors: MOE_E_ARG. */
int moe_route(moe_ctx *ctx, const float *x, int T, int layer, int32_t *ids, float *w);

/* The GPU path's success-or-failure report ([GLM-C] §12: the matmul
 * dispatcher tries the GPU entry first and takes another route when it
 * reports failure; here nothing falls back, the caller decides).  Synchronises
 * the context's stream (not the whole device) and reports errors found on
 * the device since the last call: MOE_E_NOT_RESIDENT (a selected expert had
 * no slot; up to cap missing (layer*E + id) codes go to missing_ids,
 * *n_missing = their count), MOE_E_RANGE (a row of x held a NaN or an
 * infinity, or values whose squares overflow fp32; those rows' outputs are
 * unspecified), MOE_E_WAIT (the one-token router's selecting workgroup gave
 * up its bounded wait for the other workgroups' logits; that forward's
 * output is unspecified; not expected in practice), or MOE_OK.  Clears the
 * device status on the same stream.
 * missing_ids/n_missing may be null.  Errors: MOE_E_ARG, MOE_E_HIP. */
int moe_status(moe_ctx *ctx, int32_t *missing_ids, int cap, int *n_missing);

/* Description of the last HIP error a call of this context hit (the cause
 * of its MOE_E_HIP), or "" if none; a static string. */
const char *moe_last_error(moe_ctx *ctx);

/* Which path moe_forward takes: tokens at or above this count use the MFMA
 * grouped GEMM (row format only), below it the int4 GEMV kernels.
 * Default 64.  0 restores the default. */
int moe_set_gemm_min_tokens(moe_ctx *ctx, int min_tokens);

/* Per-kernel timing with HIP events on the context's stream.  While timing
 * is on, every moe_forward / moe_forward_residual / moe_route records a
 * marker event (created without a system-scope fence, so recording it writes
 * back no caches) before each of its kernels and one after the last; a
 * kernel's duration is the time between its marker and the next.
 * moe_timing_summary synchronises on the last marker and returns, for each
 * kernel name in launch order, the average duration in milliseconds over
 * the forwards recorded since timing was switched on (or since the last
 * summary), then clears the record.  ms[i] and names[i] (static strings)
 * receive up to cap entries, *n their count, *n_forwards (optional) the
 * number of forwards averaged.  Markers are not meant for graph capture.
 * Errors: MOE_E_ARG, MOE_E_HIP (moe_last_error names the HIP error). */
int moe_set_timing(moe_ctx *ctx, int on);
int moe_timing_summary(moe_ctx *ctx, float *ms, const char **names, int cap, int *n,
                       int *n_forwards);

/* --- stand-alone steps, for callers that quantise or bucket themselves --- */

/* Per-row symmetric int4 pack ([GLM-C] §05 quantize_rows, §06 pack_int4):
 * s[o] = max(max_i |w[o][i]| / 7, 1e-8); code = rint(w / s) clamped to
 * [-7, 7] (round half to even, fp32 division); q [O][I/2] in the blob's
 * nibble order.  w, q, s: device pointers; I even.  Asynchronous on
 * stream (hipStream_t).  Errors: MOE_E_ARG, MOE_E_HIP. */
int moe_pack_int4_rows(const float *w, int64_t O, int64_t I, uint8_t *q, float *s, void *stream);

/* Affine g64 pack ([EDGE0] §三): per row and group of 64 inputs, scale =
 * bf16((max - min) / 15), min = bf16(min), code = rint((w - min) / scale)
 * clamped to [0, 15] (0 when scale is 0); q [O][I/2], scmn [O][I/64][2]
 * bf16 (scale, min).  Device pointers; I a multiple of 64. */
int moe_pack_affine_g64(const float *w, int64_t O, int64_t I, uint8_t *q, uint16_t *scmn,
                        void *stream);

/* The same two quantisers from a checkpoint source (src, sinv as for
 * moe_requant_expert; w a device pointer of that kind).  Rows a multiple
 * of 32 wide up to 8192 run one wavefront per row with each element read
 * once.  Errors: MOE_E_ARG, MOE_E_HIP. */
int moe_requant_int4_rows(const void *w, int src, const float *sinv, int64_t O, int64_t I,
                          uint8_t *q, float *s, void *stream);
int moe_requant_affine_g64(const void *w, int src, const float *sinv, int64_t O, int64_t I,
                           uint8_t *q, uint16_t *scmn, void *stream);
/* Per-row int8 ([GLM-C] §05 quantize_rows, bits = 8): s = max|w|/127
 * floored at 1e-8, code = rint(w / s) clamped to [-128, 127] (fp32 IEEE
 * division, round half to even); q [O][I] int8.  Device pointers.
 * Errors: MOE_E_ARG, MOE_E_HIP. */
int moe_requant_int8_rows(const void *w, int src, const float *sinv, int64_t O, int64_t I,
                          int8_t *q, float *s, void *stream);

/* Token -> expert bucketing of ids [T][K] (device) ([GLM-C] §11 batch
 * expert union): cnt [E], off [E+1] (exclusive scan), perm [T*K] =
 * assignment indices t*K+k in a stable sort by expert id, active [E] =
 * ids with cnt > 0 ascending and n_active [1].  Device pointers.
 * T*K <= 65536.  Errors: MOE_E_ARG. */
int moe_bucket(const int32_t *ids, int T, int K, int E, int32_t *cnt, int32_t *off,
               int32_t *perm, int32_t *active, int32_t *n_active, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_INT4_H */
