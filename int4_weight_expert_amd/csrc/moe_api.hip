// moe_api.hip -- the C ABI of include/moe.h: context, HBM slot pool, slot
// table, argument checks and kernel dispatch.
//
// The slot pool follows the expert-slot idea of "初始化与权重加载" (colibrì
// analysis) §2.2 (ESlot: one expert's gate/up/down held together, looked up
// by expert id) and of the Edge0 write-up §十四 (routing indices mapped
// through a slot table that never leaves the GPU): experts live in HBM
// slots, and a per-layer table expert id -> slot (-1 = not resident) is
// read by the kernels, so a forward touches whichever experts are resident.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "moe_ctx.h"

using namespace moe;


namespace moe {

int hip_ok(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_E_HIP; }

int hip_rc(moe_ctx* c, hipError_t e)
{
    if (e != hipSuccess) c->last_err = e;
    return hip_ok(e);
}

}  // namespace moe

namespace {

constexpr int kDefaultGemmMin = 64;

// Staging of moe_set_router_noalloc: the caller's router matrix is copied
// here before the layout kernel reads it, in place of the temporary that
// moe_set_router allocates.  One copy per device, held until the process
// ends; its size covers the largest router a context accepts (256 experts x
// 16384 inputs, 16 MiB).  Host code uses only the per-device address that
// hipGetSymbolAddress returns (the array's name is not a device address on
// the host).
constexpr size_t kRouterScratchFloats = (size_t)256 * 16384;
__device__ __align__(256) float scratch[kRouterScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Looks up (once per device, with that device current) the address of this
// device's scratch array.  Returns nullptr on failure.
float* router_scratch(int dev)
{
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = (float*)p;
    }
    return g_scratch_ptr[dev];
}

template <typename P>
int dalloc(moe_ctx* c, P** p, size_t bytes)
{
    void* q = nullptr;
    if (bytes == 0) bytes = 256;
    if (hipMalloc(&q, bytes) != hipSuccess) {
        (void)hipGetLastError();  // a failed allocation must not surface in a later call
        return MOE_E_NOMEM;
    }
    c->allocs.push_back(q);
    *p = (P*)q;
    return MOE_OK;
}

size_t expert_bytes_for(int fmt, size_t H, size_t I)
{
    const size_t packed = 3 * H * I / 2;
    if (fmt == MOE_W_INT4_ROW) return packed + 4 * (2 * I + H);
    if (fmt == MOE_W_INT4_AFFINE_G64) return packed + 12 * H * I / 64;
    if (fmt == MOE_W_INT8_ROW) return 3 * H * I + 4 * (2 * I + H);
    return 0;
}

// k-slices per (group, 64-row block) for a row of `chunks` 16-byte chunks:
// the fewest that give about 3072 single-wavefront units (12 per CU) whose
// activation slices are small enough in LDS for 32 units to stay resident
// per CU (with several tokens per pass the slice grows with the tokens),
// each slice a whole number of rolling steps, within the partial buffer and
// the LDS a unit may use.
constexpr size_t GEMV_LDS_RESIDENT = 160 * 1024 / 32;

int pick_ks(int chunks, int blocks, int step, int max_ks, size_t part_need_per_ks,
            size_t part_bytes, int T, int lds_max)
{
    static const int cand[] = {1, 2, 3, 4, 6, 8, 12, 16};
    int best = 1;
    for (int ks : cand) {
        if (ks > max_ks) break;
        if (chunks % ks != 0 || (chunks / ks) % step != 0) continue;
        if (ks > 1 && part_need_per_ks * ks > part_bytes) break;
        const size_t lds = gemv_lds_bytes(chunks / ks, T);
        if (lds > (size_t)lds_max) continue;
        best = ks;
        if ((int64_t)blocks * ks >= 3072 && lds <= GEMV_LDS_RESIDENT) break;
    }
    return best;
}

// Work plan of the GEMVs for T tokens.
void plan_gemv(moe_ctx* c, Fwd& f)
{
    const moe_config& g = c->cfg;
    const int max_groups = g.n_shared + std::min(g.n_experts, f.T * g.top_k);
    const size_t rows = (size_t)f.T * (g.top_k + g.n_shared);
    f.gu_ks = pick_ks(g.hidden / 32, max_groups * (g.inter / 64), gemv_step_chunks(0), 16,
                      rows * g.inter * 2 * 4, c->gpart_bytes, f.T, c->lds_max);
    f.dn_ks = pick_ks(g.inter / 32, max_groups * (g.hidden / 64), gemv_step_chunks(1),
                      gemv_max_dn_ks(), rows * g.hidden * 4, c->ypart_bytes, f.T, c->lds_max);
    // few (group, block) pairs: one workgroup each, its k-slices reduced in LDS
    const int gu_blocks = max_groups * (g.inter / 64);
    f.gu_wg = gu_blocks <= 128 && f.gu_ks > 1 && f.gu_ks <= 16 &&
              gemv_wg_lds_bytes(g.hidden / 32 / f.gu_ks, f.T, f.gu_ks) <= (size_t)c->lds_max &&
              !(g.n_shared > 0 && c->shared_fmt == MOE_W_INT8_ROW);
}

// Shared expert s of a layer: the layer's n_shared shared slots are
// consecutive, each shared_bytes long (the shared format may differ from the
// routed experts', so the routed slot size is not the stride).
uint8_t* shared_slot(const moe_ctx* c, int layer, int s)
{
    return c->shared + ((size_t)layer * c->cfg.n_shared + s) * c->shared_bytes;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

// Timing: a marker event before each kernel (named for it) and one after
// the last kernel of a forward (name == nullptr).
void mark(moe_ctx* c, const char* name)
{
    if (!c->timing) return;
    if (c->n_marks >= (int)c->events.size()) {
        // no system-scope fence on record: a marker then costs no cache
        // write-back and brackets the kernels closely
        hipEvent_t e;
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
        c->events.push_back(e);
        c->names.push_back(nullptr);
    }
    c->names[c->n_marks] = name;
    if (hipEventRecord(c->events[c->n_marks], c->stream) == hipSuccess) c->n_marks++;
}

Fwd make_fwd(moe_ctx* c, const float* x, float* out, int T, int layer, int residual)
{
    const moe_config& g = c->cfg;
    Fwd f{};
    f.x = x;
    f.out = out;
    f.T = T;
    f.rslices = router_t_ok(T, g.hidden, c->wr_rows) ? 1 : router_slices(T, g.hidden);
    f.magic = 0x64006400u;
    f.H = g.hidden;
    f.I = g.inter;
    f.E = g.n_experts;
    f.K = g.top_k;
    f.n_shared = g.n_shared;
    f.fmt = g.wfmt;
    f.Epad = c->Epad;
    f.residual = residual;
    f.routed_scale = g.routed_scale;
    f.eps = g.rms_eps;
    f.norm_topk = g.norm_topk;
    f.layer = layer;
    f.wr = c->wr + (size_t)layer * c->Epad * g.hidden;
    f.wr_rows = c->wr_rows ? c->wr_rows + (size_t)layer * g.n_experts * g.hidden : nullptr;
    f.wr16 = c->wr16 ? c->wr16 + (size_t)layer * c->Epad * g.hidden / 4 : nullptr;
    f.wr16s = c->wr16s ? c->wr16s + (size_t)layer * c->Epad : nullptr;
    f.bias = c->bias + (size_t)layer * g.n_experts;
    f.tbl = c->tbl + (size_t)layer * g.n_experts;
    f.pool = c->pool;
    f.slot_bytes = c->slot_bytes;
    f.shared_fmt = c->shared_fmt;
    f.shared_bytes = c->shared_bytes;
    f.shared = shared_slot(c, layer, 0);
    f.part = c->part;
    f.tpart = c->tpart;
    f.S = router_small_slices(g.hidden);
    f.logits = c->logits;
    f.ids = c->ids;
    f.wts = c->wts;
    f.tok = c->tok;
    f.xq = c->xq;
    f.xsc = c->xsc;
    f.cnt = c->cnt;
    f.off = c->off;
    f.perm = c->perm;
    f.active = c->active;
    f.n_active = c->n_active;
    f.groups = c->groups;
    f.n_groups = c->n_groups;
    f.hq = c->hq;
    f.hsc = c->hsc;
    f.gpart = c->gpart;
    f.ypart = c->ypart;
    f.xrow = c->xrow;
    f.hrow = c->hrow;
    f.hbuf = c->hbuf;
    f.hf = c->hf;
    f.tiles = c->tiles;
    f.n_tiles = c->n_tiles;
    f.counters = c->counters;
    f.dn_cnt = c->dn_cnt;
    f.rt_cnt = c->rt_cnt;
    f.rt_tag = c->rt_tag;
    f.rt_epoch = c->rt_epoch;
    f.n_group = g.n_group;
    f.scoring = g.scoring;
    f.topk_group = g.topk_group;
    f.status = c->status;
    f.n_layers = g.n_layers;
    f.lds_max = c->lds_max;
    return f;
}

// router + bucketing; leaves ids/wts/groups in the workspace
int run_router(moe_ctx* c, const Fwd& f)
{
    hipError_t e;
    if (f.sel_in_gateup || f.sel_in_router) {  // the one-token router (logits, or logits and selection)
        mark(c, "router_logits");
        return hip_rc(c, launch_router1(f, c->stream));
    }
    if (f.T <= ROUTER_SMALL_MAX_T && !f.row_staging) {
        mark(c, "router_topk_bucket");
        return hip_rc(c, launch_router_small(f, c->stream));
    }
    static const char* names[4] = {"token_stats", "router_gemm", "topk", "bucket"};
    for (int s = 0; s < 4; ++s) {
        mark(c, names[s]);
        e = launch_router_large(f, c->stream, s);
        if (e != hipSuccess) return hip_rc(c, e);
    }
    return MOE_OK;
}

// Many tokens (row format): the expert FFN as MFMA grouped GEMMs.
bool uses_gemm(const moe_ctx* c, int T)
{
    return c->hbuf != nullptr && T > ROUTER_SMALL_MAX_T && T >= c->gemm_min_tokens &&
           gemm_shape_ok(c->cfg.hidden, c->cfg.inter);
}

int run_forward_gemm(moe_ctx* c, Fwd& f)
{
    f.gu_ks = 1;
    f.dn_ks = 1;  // combine reads ypart as [rows][H]
    f.row_staging = 1;
    int rc = run_router(c, f);
    if (rc) return rc;
    mark(c, "gemm_tiles");
    rc = hip_rc(c, launch_gemm_prep(f, c->stream));
    if (rc) return rc;
    mark(c, "gemm_gateup");
    rc = hip_rc(c, launch_gemm_gateup(f, c->stream));
    if (rc) return rc;
    mark(c, "gemm_hstage");
    rc = hip_rc(c, launch_gemm_hstage(f, c->stream));
    if (rc) return rc;
    mark(c, "gemm_down");
    rc = hip_rc(c, launch_gemm_down(f, c->stream));
    if (rc) return rc;
    mark(c, "combine");
    rc = hip_rc(c, launch_combine(f, c->stream));
    if (rc) return rc;
    mark(c, nullptr);
    return MOE_OK;
}

// A few tokens, row format: the large-T router (it stages x per row), the
// matrix-core gate/up units, the h rows (slices summed, SiLU * up, staged
// per row), the matrix-core down units and the combine.
int run_forward_midt(moe_ctx* c, Fwd& f)
{
    f.row_staging = 1;
    midt_plan(f, c->gpart_bytes, c->ypart_bytes);
    int rc = run_router(c, f);
    if (rc) return rc;
    mark(c, "gateup_mfma");
    rc = hip_rc(c, launch_midt_gateup(f, c->stream));
    if (rc) return rc;
    mark(c, "h_rows");
    rc = hip_rc(c, launch_midt_hrows(f, c->stream));
    if (rc) return rc;
    mark(c, "down_mfma");
    rc = hip_rc(c, launch_midt_down(f, c->stream));
    if (rc) return rc;
    mark(c, "combine");
    rc = hip_rc(c, launch_combine(f, c->stream));
    if (rc) return rc;
    mark(c, nullptr);
    return MOE_OK;
}

int run_forward(moe_ctx* c, const float* x, int T, int layer, float* out, int residual)
{
    if (!c || !x || !out) return MOE_E_ARG;
    const moe_config& g = c->cfg;
    if (T < 1 || T > g.max_tokens || layer < 0 || layer >= g.n_layers) return MOE_E_ARG;
    const size_t nb = (size_t)T * g.hidden * sizeof(float);
    if (!residual && overlaps(x, nb, out, nb)) return MOE_E_ARG;
    Fwd f = make_fwd(c, x, out, T, layer, residual);
    if (uses_gemm(c, T)) return run_forward_gemm(c, f);
    if (midt_ok(f)) return run_forward_midt(c, f);
    plan_gemv(c, f);
    if (c->tok1 && router1_ok(f) && tok1_sel_ok(f)) {
        // the selection in the router's last workgroup (large layers) or in
        // every routed gate/up workgroup (small ones)
        if (tok1_sel_in_router(f)) f.sel_in_router = 1;
        else f.sel_in_gateup = 1;
    } else if (c->tok1 && router1_ok(f) && tok1_ok(f) && f.E <= 256) {
        // softmax scoring or group-limited selection: the general router
        // tail in the one-token router's last workgroup, its logits one
        // partial per expert
        f.sel_in_router = 2;
        f.S = 1;
    }
    int rc = run_router(c, f);
    if (rc) return rc;
    if (c->tok1 && tok1_ok(f)) {
        // one token: gate/up straight to h (no k-slice partials, no
        // finalize); small layers then run down with the combine in one
        // kernel, large ones the down GEMV (its h slices staged from fp32)
        // and the combine
        mark(c, "gateup_gemv");
        rc = hip_rc(c, launch_tok1_gateup(f, c->stream));
        if (rc) return rc;
        if (tok1_down_ok(f)) {
            mark(c, "down_combine");
            rc = hip_rc(c, launch_tok1_down(f, c->stream));
            if (rc) return rc;
            mark(c, nullptr);
            return MOE_OK;
        }
        if (c->dn_fused && tok1_dnb_ok(f)) {
            mark(c, "down_combine");
            rc = hip_rc(c, launch_tok1_down_blocks(f, c->stream));
            if (rc) return rc;
            mark(c, nullptr);
            return MOE_OK;
        }
        f.h_f32 = 1;
        f.dn_fused = c->dn_fused;
        mark(c, f.dn_fused ? "down_combine" : "down_gemv");
        rc = hip_rc(c, launch_down_gemv(f, c->stream));
        if (rc) return rc;
        if (f.dn_fused) {
            mark(c, nullptr);
            return MOE_OK;
        }
        mark(c, "combine");
        rc = hip_rc(c, launch_combine(f, c->stream));
        if (rc) return rc;
        mark(c, nullptr);
        return MOE_OK;
    }
    mark(c, "gateup_gemv");
    rc = hip_rc(c, launch_gateup_gemv(f, c->stream));
    if (rc) return rc;
    if (gateup_needs_finalize(f)) {
        mark(c, "gateup_finalize");
        rc = hip_rc(c, launch_gateup_finalize(f, c->stream));
        if (rc) return rc;
    }
    if (down_combine1_ok(f)) {
        mark(c, "down_combine");
        rc = hip_rc(c, launch_down_combine1(f, c->stream));
        if (rc) return rc;
        mark(c, nullptr);
        return MOE_OK;
    }
    mark(c, "down_gemv");
    rc = hip_rc(c, launch_down_gemv(f, c->stream));
    if (rc) return rc;
    mark(c, "combine");
    rc = hip_rc(c, launch_combine(f, c->stream));
    if (rc) return rc;
    mark(c, nullptr);
    return MOE_OK;
}

// Format and size of the expert slot at dst: the shared experts' slots may
// use their own format.
bool in_shared(const moe_ctx* c, const uint8_t* dst)
{
    return c->shared && dst >= c->shared &&
           dst < c->shared + (size_t)c->cfg.n_layers * c->cfg.n_shared * c->shared_bytes;
}
int fmt_of(const moe_ctx* c, const uint8_t* dst)
{
    return in_shared(c, dst) ? c->shared_fmt : c->cfg.wfmt;
}
size_t bytes_of(const moe_ctx* c, const uint8_t* dst)
{
    return in_shared(c, dst) ? c->shared_bytes : c->slot_bytes;
}

int copy_in_blob_impl(moe_ctx* c, uint8_t* dst_slot, const void* blob, size_t nbytes)
{
    if (!blob) return MOE_E_ARG;
    if (nbytes != bytes_of(c, dst_slot)) return MOE_E_SIZE;
    if (hipMemcpyAsync(c->staging, blob, nbytes, hipMemcpyDefault, c->stream) != hipSuccess)
        return MOE_E_HIP;
    if (launch_blob_to_slot(c->staging, dst_slot, fmt_of(c, dst_slot), c->cfg.hidden,
                            c->cfg.inter, c->stream) != hipSuccess)
        return MOE_E_HIP;
    return hip_ok(hipStreamSynchronize(c->stream));
}

int requant_into_impl(moe_ctx* c, uint8_t* dst_slot, int src, const void* Wg, const void* Wu,
                 const void* Wd, const float* sg, const float* su, const float* sd)
{
    if (!Wg || !Wu || !Wd) return MOE_E_ARG;
    if (src != MOE_SRC_F32 && src != MOE_SRC_BF16 && src != MOE_SRC_FP8_E4M3) return MOE_E_ARG;
    if (src == MOE_SRC_FP8_E4M3 && (!sg || !su || !sd)) return MOE_E_ARG;
    const int64_t H = c->cfg.hidden, I = c->cfg.inter;
    if (fmt_of(c, dst_slot) == MOE_W_INT8_ROW) {
        int8_t* q = (int8_t*)c->staging;
        float* sc = (float*)(c->staging + 3 * H * I);
        hipError_t e = launch_requant_int8_rows(Wg, src, sg, I, H, q, sc, c->stream);
        if (e == hipSuccess) e = launch_requant_int8_rows(Wu, src, su, I, H, q + I * H, sc + I, c->stream);
        if (e == hipSuccess)
            e = launch_requant_int8_rows(Wd, src, sd, H, I, q + 2 * I * H, sc + 2 * I, c->stream);
        if (e == hipSuccess)
            e = launch_blob_to_slot(c->staging, dst_slot, MOE_W_INT8_ROW, (int)H, (int)I, c->stream);
        return hip_ok(e);
    }
    if (c->cfg.wfmt == MOE_W_INT4_ROW && requant_slot_ok(Wg, Wu, Wd, dst_slot, (int)H, (int)I))
        return hip_ok(launch_requant_slot(src, Wg, Wu, Wd, sg, su, sd, (int)H, (int)I, dst_slot,
                                          c->stream));
    const int64_t gq = I * (H / 2), dq = H * (I / 2);
    uint8_t* b = c->staging;
    uint8_t* sc = b + 2 * gq + dq;
    hipError_t e;
    if (c->cfg.wfmt == MOE_W_INT4_ROW) {
        e = launch_requant_rows(Wg, src, sg, I, H, b, (float*)sc, c->stream);
        if (e == hipSuccess)
            e = launch_requant_rows(Wu, src, su, I, H, b + gq, (float*)sc + I, c->stream);
        if (e == hipSuccess)
            e = launch_requant_rows(Wd, src, sd, H, I, b + 2 * gq, (float*)sc + 2 * I, c->stream);
    } else {
        const int64_t ga = I * (H / 64) * 2;
        e = launch_requant_affine(Wg, src, sg, I, H, b, (uint16_t*)sc, c->stream);
        if (e == hipSuccess)
            e = launch_requant_affine(Wu, src, su, I, H, b + gq, (uint16_t*)sc + ga, c->stream);
        if (e == hipSuccess)
            e = launch_requant_affine(Wd, src, sd, H, I, b + 2 * gq, (uint16_t*)sc + 2 * ga,
                                      c->stream);
    }
    if (e != hipSuccess) return MOE_E_HIP;
    return hip_ok(launch_blob_to_slot(b, dst_slot, c->cfg.wfmt, (int)H, (int)I, c->stream));
}

int import_into_impl(moe_ctx* c, uint8_t* dst_slot, const uint8_t* qg, const uint8_t* qu,
                const uint8_t* qd, const float* sg, const float* su, const float* sd)
{
    if (fmt_of(c, dst_slot) != MOE_W_INT4_ROW) return MOE_E_UNSUPPORTED;
    if (!qg || !qu || !qd || !sg || !su || !sd) return MOE_E_ARG;
    const size_t H = c->cfg.hidden, I = c->cfg.inter;
    const size_t gq = I * (H / 2), dq = H * (I / 2), sb = 2 * gq + dq;
    uint8_t* b = c->staging;
    const struct { void* dst; const void* src; size_t n; } parts[6] = {
        {b, qg, gq}, {b + gq, qu, gq}, {b + 2 * gq, qd, dq},
        {b + sb, sg, 4 * I}, {b + sb + 4 * I, su, 4 * I}, {b + sb + 8 * I, sd, 4 * H}};
    for (const auto& p : parts)
        if (hipMemcpyAsync(p.dst, p.src, p.n, hipMemcpyDefault, c->stream) != hipSuccess)
            return MOE_E_HIP;
    if (launch_container_to_slot(b, dst_slot, (int)H, (int)I, c->stream) != hipSuccess)
        return MOE_E_HIP;
    return hip_ok(hipStreamSynchronize(c->stream));
}

// The three slot writers, ordered against asynchronous loads into the same slot.
int copy_in_blob(moe_ctx* c, uint8_t* dst, const void* blob, size_t nbytes)
{
    int rc = slot_compute_ready(c, dst);
    rc = rc ? rc : copy_in_blob_impl(c, dst, blob, nbytes);
    return rc ? rc : slot_compute_written(c, dst);
}

int requant_into(moe_ctx* c, uint8_t* dst, int src, const void* Wg, const void* Wu,
                 const void* Wd, const float* sg, const float* su, const float* sd)
{
    int rc = slot_compute_ready(c, dst);
    rc = rc ? rc : requant_into_impl(c, dst, src, Wg, Wu, Wd, sg, su, sd);
    return rc ? rc : slot_compute_written(c, dst);
}

int import_into(moe_ctx* c, uint8_t* dst, const uint8_t* qg, const uint8_t* qu,
                const uint8_t* qd, const float* sg, const float* su, const float* sd)
{
    int rc = slot_compute_ready(c, dst);
    rc = rc ? rc : import_into_impl(c, dst, qg, qu, qd, sg, su, sd);
    return rc ? rc : slot_compute_written(c, dst);
}

}  // namespace

extern "C" {

int moe_layer_create(const moe_config* cfg, void* stream, moe_ctx** out)
{
    if (!cfg || !out) return MOE_E_ARG;
    *out = nullptr;
    const moe_config& g = *cfg;
    if (g.hidden <= 0 || g.inter <= 0 || g.n_experts <= 0 || g.top_k <= 0 || g.n_layers <= 0 ||
        g.n_slots < 0 || g.max_tokens <= 0 || g.n_shared < 0)
        return MOE_E_ARG;
    if (g.wfmt != MOE_W_INT4_ROW && g.wfmt != MOE_W_INT4_AFFINE_G64) return MOE_E_ARG;
    if (g.shared_fmt != 0 && g.shared_fmt != g.wfmt && g.shared_fmt != MOE_W_INT8_ROW)
        return MOE_E_ARG;
    if (g.n_group < 1 || g.topk_group < 1 || g.topk_group > g.n_group) return MOE_E_ARG;
    if (g.scoring != MOE_SCORE_SIGMOID && g.scoring != MOE_SCORE_SOFTMAX) return MOE_E_ARG;
    if (g.scoring == MOE_SCORE_SOFTMAX && g.n_group != 1) return MOE_E_UNSUPPORTED;
    if (g.n_group > 1 &&
        (g.n_group > 64 || g.n_experts % g.n_group || g.n_experts / g.n_group < 2 ||
         g.top_k > g.topk_group * (g.n_experts / g.n_group)))
        return MOE_E_UNSUPPORTED;
    if (g.n_experts > 256 || g.top_k > 8 || g.top_k > g.n_experts || g.n_shared > 1)
        return MOE_E_UNSUPPORTED;
    if (g.hidden % 256 || g.inter % 256 || g.hidden > 16384) return MOE_E_UNSUPPORTED;
    if (g.wfmt == MOE_W_INT4_AFFINE_G64 && g.hidden % 512) return MOE_E_UNSUPPORTED;
    if ((size_t)g.max_tokens * g.top_k > 65536) return MOE_E_UNSUPPORTED;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_E_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_E_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MOE_E_HIP;
    int lds_max = 65536;
    if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
        hipSuccess)
        lds_max = 65536;

    moe_ctx* c = new moe_ctx();
    c->cfg = g;
    c->stream = (hipStream_t)stream;
    c->device = dev;
    c->lds_max = lds_max;
    c->slot_bytes = expert_bytes_for(g.wfmt, g.hidden, g.inter);
    c->shared_fmt = g.shared_fmt ? g.shared_fmt : g.wfmt;
    c->shared_bytes = expert_bytes_for(c->shared_fmt, g.hidden, g.inter);
    c->Epad = (g.n_experts + 63) / 64 * 64;
    const size_t H = g.hidden, I = g.inter, E = g.n_experts, L = g.n_layers, Tm = g.max_tokens;
    const size_t K = g.top_k, rows = Tm * K + Tm * g.n_shared;
    int rc = MOE_OK;
    rc = rc ? rc : dalloc(c, &c->pool, (size_t)g.n_slots * c->slot_bytes);
    rc = rc ? rc : dalloc(c, &c->wr, L * c->Epad * H * 4);
    rc = rc ? rc : dalloc(c, &c->wr_rows, L * E * H * 4);
    if (Tm > ROUTER_SMALL_MAX_T) {  // the large-T router's split fp16 copy
        rc = rc ? rc : dalloc(c, &c->wr16, L * c->Epad * H * 4);
        rc = rc ? rc : dalloc(c, &c->wr16s, L * c->Epad * 8);
    }
    rc = rc ? rc : dalloc(c, &c->bias, L * E * 4);
    rc = rc ? rc : dalloc(c, &c->tbl, L * E * 4);
    rc = rc ? rc : dalloc(c, &c->shared, L * g.n_shared * c->shared_bytes);
    rc = rc ? rc : dalloc(c, &c->staging, std::max(c->slot_bytes, c->shared_bytes));
    rc = rc ? rc : dalloc(c, &c->part, (H / 64) * ROUTER_SMALL_MAX_T * c->Epad * 4);
    rc = rc ? rc : dalloc(c, &c->tpart, (H / 64) * ROUTER_SMALL_MAX_T * 2 * 4);
    rc = rc ? rc : dalloc(c, &c->logits, router_logit_rows((int)Tm) * c->Epad * 4);
    rc = rc ? rc : dalloc(c, &c->ids, Tm * K * 4);
    rc = rc ? rc : dalloc(c, &c->wts, Tm * K * 4);
    rc = rc ? rc : dalloc(c, &c->tok, Tm * sizeof(TokStat));
    rc = rc ? rc : dalloc(c, &c->xq, Tm * (H / 8) * 16);
    rc = rc ? rc : dalloc(c, &c->xsc, Tm * (H / 64) * 8);
    rc = rc ? rc : dalloc(c, &c->cnt, E * 4);
    rc = rc ? rc : dalloc(c, &c->off, (E + 1) * 4);
    rc = rc ? rc : dalloc(c, &c->perm, Tm * K * 4);
    rc = rc ? rc : dalloc(c, &c->active, E * 4);
    rc = rc ? rc : dalloc(c, &c->n_active, 4);
    rc = rc ? rc : dalloc(c, &c->groups, (E + g.n_shared) * sizeof(Group));
    rc = rc ? rc : dalloc(c, &c->n_groups, 4);
    rc = rc ? rc : dalloc(c, &c->hq, rows * (I / 8) * 16);
    rc = rc ? rc : dalloc(c, &c->hsc, rows * (I / 64) * 8);
    rc = rc ? rc : dalloc(c, &c->hf, (K + g.n_shared) * I * 4);
    {
        // k-split partials for up to 16 tokens (gate/up, 16 slices) and 64
        // tokens (down, 4 slices); beyond that the plan falls back to fewer
        // slices, down to one (gate/up then needs no partials at all).
        const size_t r16 = std::min<size_t>(Tm, 16) * (K + g.n_shared);
        const size_t r64 = std::min<size_t>(Tm, 64) * (K + g.n_shared);
        c->gpart_bytes = r16 * I * 2 * 4 * 16;
        c->ypart_bytes = std::max(rows * H * 4, r64 * H * 4 * 4);
    }
    rc = rc ? rc : dalloc(c, &c->gpart, c->gpart_bytes);
    rc = rc ? rc : dalloc(c, &c->ypart, c->ypart_bytes);
    if (g.wfmt == MOE_W_INT4_ROW && Tm > ROUTER_SMALL_MAX_T) {
        // per-row staging (the few-token matrix-core path and the grouped
        // GEMM) and the grouped-GEMM workspace
        rc = rc ? rc : dalloc(c, &c->xrow, Tm * 8);
        rc = rc ? rc : dalloc(c, &c->hrow, rows * 8);
        rc = rc ? rc : dalloc(c, &c->hbuf, rows * I * 4);
        rc = rc ? rc : dalloc(c, &c->tiles, (size_t)gemm_max_tiles((int)Tm, (int)K, E, g.n_shared) * 8);
        rc = rc ? rc : dalloc(c, &c->n_tiles, 4);
    }
    rc = rc ? rc : dalloc(c, &c->counters, (1 + H / 64) * 4);
    rc = rc ? rc : dalloc(c, &c->dn_cnt, (size_t)(H / 64) * 256);
    rc = rc ? rc : dalloc(c, &c->rt_cnt, (size_t)17 * 256);
    rc = rc ? rc : dalloc(c, &c->rt_tag, (size_t)256 * 8);
    rc = rc ? rc : dalloc(c, &c->rt_epoch, 256);
    c->status_words = 1 + (L * E + 31) / 32;
    rc = rc ? rc : dalloc(c, &c->status, c->status_words * 4);
    if (rc == MOE_OK) {
        c->tbl_host.assign(L * E, -1);
        hipError_t e = hipMemcpy(c->tbl, c->tbl_host.data(), L * E * 4, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemset(c->counters, 0, (1 + H / 64) * 4);
        if (e == hipSuccess) e = hipMemset(c->dn_cnt, 0, (size_t)(H / 64) * 256);
        if (e == hipSuccess) e = hipMemset(c->rt_cnt, 0, (size_t)17 * 256);
        if (e == hipSuccess) e = hipMemset(c->rt_tag, 0, (size_t)256 * 8);
        if (e == hipSuccess) e = hipMemset(c->rt_epoch, 0, 256);
        if (e == hipSuccess) e = hipMemset(c->status, 0, c->status_words * 4);
        if (e == hipSuccess) e = hipMemset(c->bias, 0, L * E * 4);
        if (e == hipSuccess) e = hipMemset(c->wr, 0, L * c->Epad * H * 4);
        if (e == hipSuccess) e = hipMemset(c->wr_rows, 0, L * E * H * 4);
        if (e == hipSuccess && c->wr16) e = hipMemset(c->wr16, 0, L * c->Epad * H * 4);
        if (e == hipSuccess && c->wr16s) e = hipMemset(c->wr16s, 0, L * c->Epad * 8);
        if (e == hipSuccess && g.n_shared) e = hipMemset(c->shared, 0, L * g.n_shared * c->shared_bytes);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess) rc = MOE_E_HIP;
    }
    rc = rc ? rc : residency_init(c);
    if (rc == MOE_OK && !router_scratch(dev)) rc = MOE_E_HIP;
    if (rc != MOE_OK) {
        moe_destroy(c);
        return rc;
    }
    *out = c;
    return MOE_OK;
}

void moe_destroy(moe_ctx* c)
{
    if (!c) return;
    hipStreamSynchronize(c->stream);
    residency_destroy(c);
    for (hipEvent_t e : c->events) hipEventDestroy(e);
    for (void* p : c->allocs) hipFree(p);
    delete c;
}

int moe_set_stream(moe_ctx* c, void* stream)
{
    if (!c) return MOE_E_ARG;
    c->stream = (hipStream_t)stream;
    return MOE_OK;
}

size_t moe_expert_bytes(const moe_ctx* c) { return c ? c->slot_bytes : 0; }

int moe_set_router(moe_ctx* c, int layer, const float* W, const float* bias)
{
    if (!c || !W || !bias || layer < 0 || layer >= c->cfg.n_layers) return MOE_E_ARG;
    const size_t H = c->cfg.hidden, E = c->cfg.n_experts;
    float* tmp = nullptr;
    if (hipMalloc(&tmp, E * H * 4) != hipSuccess) {
        (void)hipGetLastError();
        return MOE_E_NOMEM;
    }
    hipError_t e = hipMemcpyAsync(tmp, W, E * H * 4, hipMemcpyDefault, c->stream);
    if (e == hipSuccess)
        e = launch_router_to_internal(tmp, c->wr + (size_t)layer * c->Epad * H, (int)E, c->Epad,
                                      (int)H, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->wr_rows + (size_t)layer * E * H, tmp, E * H * 4,
                           hipMemcpyDeviceToDevice, c->stream);
    if (e == hipSuccess && c->wr16)
        e = launch_router_split(tmp, c->wr16 + (size_t)layer * c->Epad * H / 4,
                                c->wr16s + (size_t)layer * c->Epad, (int)E, c->Epad, (int)H,
                                c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->bias + (size_t)layer * E, bias, E * 4, hipMemcpyDefault, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    hipFree(tmp);
    return hip_ok(e);
}

int moe_set_router_noalloc(moe_ctx* c, int layer, const float* W, const float* bias)
{
    if (!c || !W || !bias || layer < 0 || layer >= c->cfg.n_layers) return MOE_E_ARG;
    const size_t H = c->cfg.hidden, E = c->cfg.n_experts;
    if (E * H > kRouterScratchFloats) return MOE_E_SIZE;
    float* tmp = router_scratch(c->device);  // set up by create on this device
    if (!tmp) return MOE_E_HIP;
    hipError_t e = hipMemcpyAsync(tmp, W, E * H * 4, hipMemcpyDefault, c->stream);
    if (e == hipSuccess)
        e = launch_router_to_internal(tmp, c->wr + (size_t)layer * c->Epad * H, (int)E, c->Epad,
                                      (int)H, c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->wr_rows + (size_t)layer * E * H, tmp, E * H * 4,
                           hipMemcpyDeviceToDevice, c->stream);
    if (e == hipSuccess && c->wr16)
        e = launch_router_split(tmp, c->wr16 + (size_t)layer * c->Epad * H / 4,
                                c->wr16s + (size_t)layer * c->Epad, (int)E, c->Epad, (int)H,
                                c->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(c->bias + (size_t)layer * E, bias, E * 4, hipMemcpyDefault, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    return hip_rc(c, e);
}

int moe_load_expert(moe_ctx* c, int slot, const void* blob, size_t nbytes)
{
    if (!c) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    return copy_in_blob(c, c->pool + (size_t)slot * c->slot_bytes, blob, nbytes);
}

int moe_pack_expert(moe_ctx* c, int slot, const float* Wg, const float* Wu, const float* Wd)
{
    if (!c) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    return requant_into(c, c->pool + (size_t)slot * c->slot_bytes, MOE_SRC_F32, Wg, Wu, Wd,
                        nullptr, nullptr, nullptr);
}

int moe_requant_expert(moe_ctx* c, int slot, int src, const void* Wg, const void* Wu,
                       const void* Wd, const float* sinv_g, const float* sinv_u,
                       const float* sinv_d)
{
    if (!c) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    return requant_into(c, c->pool + (size_t)slot * c->slot_bytes, src, Wg, Wu, Wd, sinv_g,
                        sinv_u, sinv_d);
}

int moe_import_expert(moe_ctx* c, int slot, const uint8_t* qg, const uint8_t* qu,
                      const uint8_t* qd, const float* sg, const float* su, const float* sd)
{
    if (!c) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    return import_into(c, c->pool + (size_t)slot * c->slot_bytes, qg, qu, qd, sg, su, sd);
}

int moe_set_shared(moe_ctx* c, int layer, int s, const void* blob, size_t nbytes)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || s < 0 || s >= c->cfg.n_shared)
        return MOE_E_ARG;
    return copy_in_blob(c, shared_slot(c, layer, s),
                        blob, nbytes);
}

int moe_pack_shared(moe_ctx* c, int layer, int s, const float* Wg, const float* Wu,
                    const float* Wd)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || s < 0 || s >= c->cfg.n_shared)
        return MOE_E_ARG;
    return requant_into(c, shared_slot(c, layer, s),
                        MOE_SRC_F32, Wg, Wu, Wd, nullptr, nullptr, nullptr);
}

int moe_requant_shared(moe_ctx* c, int layer, int s, int src, const void* Wg, const void* Wu,
                       const void* Wd, const float* sinv_g, const float* sinv_u,
                       const float* sinv_d)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || s < 0 || s >= c->cfg.n_shared)
        return MOE_E_ARG;
    return requant_into(c, shared_slot(c, layer, s),
                        src, Wg, Wu, Wd, sinv_g, sinv_u, sinv_d);
}

int moe_import_shared(moe_ctx* c, int layer, int s, const uint8_t* qg, const uint8_t* qu,
                      const uint8_t* qd, const float* sg, const float* su, const float* sd)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || s < 0 || s >= c->cfg.n_shared)
        return MOE_E_ARG;
    return import_into(c, shared_slot(c, layer, s), qg,
                       qu, qd, sg, su, sd);
}

int moe_read_slot(moe_ctx* c, int slot, void* dst, size_t nbytes)
{
    if (!c || !dst) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    if (nbytes != c->slot_bytes) return MOE_E_SIZE;
    const int rc = slot_compute_ready(c, c->pool + (size_t)slot * c->slot_bytes);
    if (rc) return rc;
    hipError_t e = launch_slot_to_blob(c->pool + (size_t)slot * c->slot_bytes, c->staging,
                                       c->cfg.wfmt, c->cfg.hidden, c->cfg.inter, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(dst, c->staging, nbytes, hipMemcpyDefault, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    return hip_ok(e);
}

int moe_forward(moe_ctx* c, const float* x, int T, int layer, float* out)
{
    const int rc = run_forward(c, x, T, layer, out, 0);
    return rc ? rc : forward_done(c, layer);
}

int moe_forward_residual(moe_ctx* c, float* x, int T, int layer)
{
    const int rc = run_forward(c, x, T, layer, x, 1);
    return rc ? rc : forward_done(c, layer);
}

int moe_route(moe_ctx* c, const float* x, int T, int layer, int32_t* ids, float* w)
{
    if (!c || !x || !ids || !w) return MOE_E_ARG;
    const moe_config& g = c->cfg;
    if (T < 1 || T > g.max_tokens || layer < 0 || layer >= g.n_layers) return MOE_E_ARG;
    Fwd f = make_fwd(c, x, nullptr, T, layer, 0);
    plan_gemv(c, f);
    int rc = run_router(c, f);
    if (rc) return rc;
    mark(c, nullptr);
    const size_t n = (size_t)T * g.top_k;
    hipError_t e = hipMemcpyAsync(ids, c->ids, n * 4, hipMemcpyDeviceToDevice, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(w, c->wts, n * 4, hipMemcpyDeviceToDevice, c->stream);
    return hip_ok(e);
}

int moe_status(moe_ctx* c, int32_t* missing, int cap, int* n_missing)
{
    if (!c) return MOE_E_ARG;
    std::vector<uint32_t> st(c->status_words, 0);
    // read and clear on the context's stream only (other streams of the
    // device are not waited for)
    hipError_t e = hipMemcpyAsync(st.data(), c->status, c->status_words * 4,
                                  hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->status, 0, c->status_words * 4, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_rc(c, e);
    int n = 0;
    for (size_t wd = 1; wd < c->status_words; ++wd)
        for (int bit = 0; bit < 32; ++bit)
            if (st[wd] & (1u << bit)) {
                if (missing && n < cap) missing[n] = (int32_t)((wd - 1) * 32 + bit);
                ++n;
            }
    if (n_missing) *n_missing = n;
    if (st[0] & STATUS_WAIT) return MOE_E_WAIT;
    if (st[0] & STATUS_NOT_RESIDENT) return MOE_E_NOT_RESIDENT;
    if (st[0] & STATUS_RANGE) return MOE_E_RANGE;
    return MOE_OK;
}

const char* moe_last_error(moe_ctx* c)
{
    if (!c) return "null context";
    return c->last_err == hipSuccess ? "" : hipGetErrorString(c->last_err);
}

int moe_set_gemm_min_tokens(moe_ctx* c, int min_tokens)
{
    if (!c || min_tokens < 0) return MOE_E_ARG;
    c->gemm_min_tokens = min_tokens ? min_tokens : kDefaultGemmMin;
    return MOE_OK;
}

int moe_set_timing(moe_ctx* c, int on)
{
    if (!c) return MOE_E_ARG;
    c->timing = on != 0;
    c->n_marks = 0;
    return MOE_OK;
}

int moe_timing_summary(moe_ctx* c, float* ms, const char** names, int cap, int* n,
                       int* n_forwards)
{
    if (!c || !n) return MOE_E_ARG;
    *n = 0;
    if (n_forwards) *n_forwards = 0;
    if (c->n_marks < 2) {
        c->n_marks = 0;
        return MOE_OK;
    }
    if (hipEventSynchronize(c->events[c->n_marks - 1]) != hipSuccess) return hip_rc(c, hipErrorUnknown);
    std::vector<const char*> order;
    std::vector<double> sum;
    std::vector<int> count;
    int forwards = 0;
    for (int i = 0; i + 1 < c->n_marks; ++i) {
        if (c->names[i] == nullptr) continue;  // end marker of a forward
        float v = 0.f;
        const hipError_t e = hipEventElapsedTime(&v, c->events[i], c->events[i + 1]);
        if (e != hipSuccess) return hip_rc(c, e);
        size_t k = 0;
        while (k < order.size() && strcmp(order[k], c->names[i]) != 0) ++k;
        if (k == order.size()) {
            order.push_back(c->names[i]);
            sum.push_back(0.0);
            count.push_back(0);
        }
        sum[k] += v;
        count[k] += 1;
        if (c->names[i + 1] == nullptr) ++forwards;
    }
    for (size_t k = 0; k < order.size() && (int)k < cap; ++k) {
        if (ms) ms[k] = (float)(sum[k] / count[k]);
        if (names) names[k] = order[k];
    }
    *n = (int)std::min(order.size(), (size_t)cap);
    if (n_forwards) *n_forwards = forwards;
    c->n_marks = 0;
    return MOE_OK;
}

int moe_requant_int8_rows(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                          int8_t* q, float* s, void* stream)
{
    if (!w || !q || !s || O <= 0 || I <= 0) return MOE_E_ARG;
    if (src != MOE_SRC_F32 && src != MOE_SRC_BF16 && !(src == MOE_SRC_FP8_E4M3 && sinv))
        return MOE_E_ARG;
    return hip_ok(launch_requant_int8_rows(w, src, sinv, O, I, q, s, (hipStream_t)stream));
}

int moe_read_shared(moe_ctx* c, int layer, int s, void* dst, size_t nbytes)
{
    if (!c || !dst || layer < 0 || layer >= c->cfg.n_layers || s < 0 || s >= c->cfg.n_shared)
        return MOE_E_ARG;
    if (nbytes != c->shared_bytes) return MOE_E_SIZE;
    const uint8_t* src = shared_slot(c, layer, s);
    hipError_t e = launch_slot_to_blob(src, c->staging, c->shared_fmt, c->cfg.hidden,
                                       c->cfg.inter, c->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(dst, c->staging, nbytes, hipMemcpyDefault, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    return hip_rc(c, e);
}

size_t moe_shared_bytes(const moe_ctx* c) { return c ? c->shared_bytes : 0; }

int moe_pack_int4_rows(const float* w, int64_t O, int64_t I, uint8_t* q, float* s, void* stream)
{
    return moe_requant_int4_rows(w, MOE_SRC_F32, nullptr, O, I, q, s, stream);
}

int moe_pack_affine_g64(const float* w, int64_t O, int64_t I, uint8_t* q, uint16_t* scmn,
                        void* stream)
{
    return moe_requant_affine_g64(w, MOE_SRC_F32, nullptr, O, I, q, scmn, stream);
}

static bool src_ok(int src, const float* sinv)
{
    if (src == MOE_SRC_F32 || src == MOE_SRC_BF16) return true;
    return src == MOE_SRC_FP8_E4M3 && sinv != nullptr;
}

int moe_requant_int4_rows(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                          uint8_t* q, float* s, void* stream)
{
    if (!w || !q || !s || O <= 0 || I <= 0 || (I & 1) || !src_ok(src, sinv)) return MOE_E_ARG;
    return hip_ok(launch_requant_rows(w, src, sinv, O, I, q, s, (hipStream_t)stream));
}

int moe_requant_affine_g64(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                           uint8_t* q, uint16_t* scmn, void* stream)
{
    if (!w || !q || !scmn || O <= 0 || I <= 0 || (I % 64) || !src_ok(src, sinv))
        return MOE_E_ARG;
    return hip_ok(launch_requant_affine(w, src, sinv, O, I, q, scmn, (hipStream_t)stream));
}

int moe_bucket(const int32_t* ids, int T, int K, int E, int32_t* cnt, int32_t* off,
               int32_t* perm, int32_t* active, int32_t* n_active, void* stream)
{
    if (!ids || !cnt || !off || !perm || !active || !n_active) return MOE_E_ARG;
    if (T < 1 || K < 1 || E < 1 || E > 256 || (int64_t)T * K > 65536) return MOE_E_ARG;
    return hip_ok(launch_bucket(ids, T, K, E, cnt, off, perm, active, n_active,
                                (hipStream_t)stream));
}

}  // extern "C"
