// moe_internal.h -- shared declarations of the MI355X int4 MoE library
// (context, device work descriptors, kernel launchers).  Internal to the
// library; the public ABI is include/moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// Slot layout (the library's own order of an expert's bytes in HBM).
//
// Every int4 matrix [O][In] is stored as 8-row groups: group q, 16-byte
// chunk c (32 consecutive inputs) of its 8 rows are 128 bytes contiguous,
//   byte offset ((q * (In/32) + c) * 8 + r) * 16  holds row 8q+r,
//   inputs 32c .. 32c+31,
// so a group's codes are one run of In/2 * 8 bytes and a 64-row block (8
// groups) is In/2 * 64 bytes.  A workgroup that owns 8 rows over all inputs
// (the one-token kernels) reads one contiguous run per matrix; a wavefront
// whose lanes are 64 rows of a block reads eight 128-byte runs per chunk.
// Row format codes are stored offset-binary (code + 8, i.e. blob byte ^ 0x88)
// so that unsigned byte conversion gives code + 8 directly.
// Scales follow the three matrices: row format keeps fp32 sg[I] su[I] sd[H]
// unchanged; affine format stores the (scale, min) bf16 pair of row 8q+r,
// group g at ((q * (In/64) + g) * 8 + r) * 4.
// Sizes equal the blob sizes, so a slot is moe_expert_bytes() long.
// ---------------------------------------------------------------------------

struct Group {
    const uint8_t* base;  // slot bytes; nullptr = expert not resident
    int cnt;              // tokens in this group
    int off;              // routed: first index into perm; shared: shared index s
    int kind;             // 0 routed, 1 shared
    int expert;           // expert id (routed) or -1
};

struct TokStat {
    float xsum;    // sum of x over the row (offset correction of int4 codes)
    float rscale;  // RMSNorm factor (1 when the forward does not normalise)
    float xscale;  // 2^k with sqrt(sum of squares) * 2^k in [2^11, 2^12): the large-T router's x scale
};

// Launch-time description of one forward (all device pointers).
struct Fwd {
    const float* x;       // [T][H]
    float* out;           // [T][H]
    int T, H, I, E, K, n_shared, fmt, Epad;
    int shared_fmt;       // the shared experts' format (fmt, or MOE_W_INT8_ROW)
    size_t shared_bytes;  // bytes of one shared expert's slot
    int residual;         // 1: out = x + moe(rmsnorm(x)), x may equal out
    float routed_scale, eps;
    int norm_topk;
    int n_group, topk_group;  // group-limited selection (n_group = 1: none)
    int scoring;          // MOE_SCORE_SIGMOID or MOE_SCORE_SOFTMAX
    int layer;
    const float* wr;      // router, interleaved [Epad/64][H/4][64] float4
    const float* wr_rows; // router, row-major [E][H] (the one-token router)
    const uint4* wr16;    // router as split fp16 (hi, lo) operands [Epad/32][H/16][64][2] (large-T router)
    const float2* wr16s;  // [Epad] per expert (2^k its weights were scaled by, 2^-k)
    const float* bias;    // [E]
    const int* tbl;       // [E] slot table row of this layer
    const uint8_t* pool;  // slot pool base
    size_t slot_bytes;
    const uint8_t* shared;  // n_shared shared experts of this layer (slot layout)
    // workspace
    float* part;          // small-T router partial logits [S][T][Epad]
    float* tpart;         // small-T router partial token sums [S][T][2] (sum, sum of squares)
    int S;                // router K-slices of 64 columns (S = H/64)
    float* logits;        // [rslices][T][Epad] partial logits (large-T router)
    int32_t* ids;         // [T][K]
    float* wts;           // [T][K]
    TokStat* tok;         // [T]
    uint4* xq;            // [T][H/8] x staged as fp16 spans (pair order, see k_common.h)
    float2* xsc;          // [T][H/64] per span (2^-k, sum of its fp16 values)
    int32_t* cnt;         // [E]
    int32_t* off;         // [E+1]
    int32_t* perm;        // [T*K]
    int32_t* active;      // [E]
    int32_t* n_active;    // [1]
    Group* groups;        // [n_shared + E]
    int32_t* n_groups;    // [1]
    uint4* hq;            // [rows][I/8] h = silu(g) * u staged as fp16 spans
    float2* hsc;          // [rows][I/64]
    uint32_t* counters;   // [0]: router arrivals
    uint32_t* dn_cnt;     // one-token down GEMV: per 64-output block arrival counters, 256 bytes apart
    uint32_t* rt_cnt;     // one- and few-token routers: 16 arrival sub-counters and a top counter, 256 bytes apart
    uint64_t* rt_tag;     // one-token router: per expert (call tag << 32) | logit bits [256]
    uint32_t* rt_epoch;   // one-token router: tag of the last selection [1]
    uint32_t* status;     // [0] flags, [1..] missing bitmap over layer*E+id
    int n_layers;
    int lds_max;          // device LDS bytes per workgroup
    // GEMV work plan (see k_gemv.hip); rows = T*K + T*n_shared token rows
    int gu_ks;            // gate/up: k-slices (units) per (group, 64-row block)
    int dn_ks;            // down: same, at most gemv_max_dn_ks()
    int gu_wg;            // gate/up as one workgroup per (group, block), k-slices as its waves
    float* gpart;         // [rows][I/64][gu_ks][2][64] gate/up partials (gu_ks > 1)
    float* ypart;         // [rows][H/64][dn_ks][64] down partials ([rows][H] when dn_ks = 1)
    // grouped-GEMM path (many tokens): x and h staged per row in xq / hq
    int row_staging;      // 1: stage x per row (grouped GEMM), 0: in spans of 64 (GEMVs)
    int rslices;          // H slices (partial logit planes) of the large-T router
    uint32_t magic;       // 0x64006400 (fp16 pair 1024, 1024), opaque to the compiler
    float2* xrow;         // [T] per token (2^-k, sum of its fp16 values)
    float2* hrow;         // [rows]
    float* hbuf;          // [rows][I] h in fp32 (gate/up GEMM output)
    float* hf;            // [K + n_shared][I] h in fp32 of the one-token kernels
    int h_f32;            // 1: the down GEMV stages its h slices from hf (one token)
    int sel_in_gateup;    // 1: the one-token gate/up kernel selects the experts itself
    int sel_in_router;    // the one-token router's last workgroup selects: 1 plain sigmoid top-K, 2 the general tail
    int dn_fused;         // 1: the one-token down GEMV combines each output block in its last unit
    int2* tiles;          // [max tiles] (group index, first row) of each 128-row tile
    int32_t* n_tiles;     // [1]
};

enum { STATUS_NOT_RESIDENT = 1u, STATUS_RANGE = 2u, STATUS_WAIT = 4u };

// launchers (return hipError_t)
hipError_t launch_requant_rows(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                               uint8_t* q, float* s, hipStream_t st);
hipError_t launch_requant_affine(const void* w, int src, const float* sinv, int64_t O, int64_t I,
                                 uint8_t* q, uint16_t* scmn, hipStream_t st);
hipError_t launch_requant_int8_rows(const void* w, int src, const float* sinv, int64_t O,
                                    int64_t I, int8_t* q, float* s, hipStream_t st);
bool shared_int8(const Fwd& f);
bool requant_slot_ok(const void* wg, const void* wu, const void* wd, const uint8_t* slot, int H,
                     int I);
hipError_t launch_requant_slot(int src, const void* wg, const void* wu, const void* wd,
                               const float* sg, const float* su, const float* sd, int H, int I,
                               uint8_t* slot, hipStream_t st);
hipError_t launch_container_to_slot(const uint8_t* staged, uint8_t* slot, int H, int I,
                                    hipStream_t st);
hipError_t launch_blob_to_slot(const uint8_t* blob, uint8_t* slot, int fmt, int H, int I,
                               hipStream_t st);
hipError_t launch_slot_to_blob(const uint8_t* slot, uint8_t* blob, int fmt, int H, int I,
                               hipStream_t st);
hipError_t launch_router_to_internal(const float* W, float* wr, int E, int Epad, int H,
                                     hipStream_t st);
hipError_t launch_router_split(const float* W, uint4* w16, float2* w16s, int E, int Epad, int H,
                               hipStream_t st);
hipError_t launch_bucket(const int32_t* ids, int T, int K, int E, int32_t* cnt, int32_t* off,
                         int32_t* perm, int32_t* active, int32_t* n_active, hipStream_t st);

// Typed kernel launch (arguments converted to the kernel's parameter types).
template <typename... KArgs, typename... Args>
hipError_t launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                    hipStream_t st, Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    hipLaunchKernelGGL(kernel, grid, block, lds, st, static_cast<KArgs>(args)...);
    return hipGetLastError();
}

// forward pieces
hipError_t launch_router_small(const Fwd& f, hipStream_t st);
bool router1_ok(const Fwd& f);
hipError_t launch_router1(const Fwd& f, hipStream_t st);
int router_small_slices(int H);  // partial rows of the small-T router
hipError_t launch_router_large(const Fwd& f, hipStream_t st, int stage);
hipError_t launch_gateup_gemv(const Fwd& f, hipStream_t st);
hipError_t launch_down_gemv(const Fwd& f, hipStream_t st);
bool gateup_needs_finalize(const Fwd& f);
size_t gemv_wg_lds_bytes(int chunks_per_slice, int T, int ks);
int gemm_max_tiles(int T, int K, int E, int n_shared);
bool gemm_shape_ok(int H, int I);
hipError_t launch_gemm_prep(const Fwd& f, hipStream_t st);
hipError_t launch_gemm_gateup(const Fwd& f, hipStream_t st);
hipError_t launch_gemm_hstage(const Fwd& f, hipStream_t st);
hipError_t launch_gemm_down(const Fwd& f, hipStream_t st);
hipError_t launch_gateup_finalize(const Fwd& f, hipStream_t st);
hipError_t launch_combine(const Fwd& f, hipStream_t st);
bool tok1_ok(const Fwd& f);
bool tok1_down_ok(const Fwd& f);
bool tok1_sel_ok(const Fwd& f);
bool tok1_sel_in_router(const Fwd& f);
hipError_t launch_tok1_gateup(const Fwd& f, hipStream_t st);
hipError_t launch_tok1_down(const Fwd& f, hipStream_t st);
bool tok1_dnb_ok(const Fwd& f);
hipError_t launch_tok1_down_blocks(const Fwd& f, hipStream_t st);
// few tokens (MIDT_MIN_T .. the grouped GEMM's threshold), row format,
// matrix cores; below MIDT_MIN_T the GEMVs (as fast at 8 tokens, measured)
constexpr int MIDT_MIN_T = 9;
bool midt_ok(const Fwd& f);
void midt_plan(Fwd& f, size_t gpart_bytes, size_t ypart_bytes);
hipError_t launch_midt_gateup(const Fwd& f, hipStream_t st);
hipError_t launch_midt_hrows(const Fwd& f, hipStream_t st);
hipError_t launch_midt_down(const Fwd& f, hipStream_t st);
bool down_combine1_ok(const Fwd& f);
hipError_t launch_down_combine1(const Fwd& f, hipStream_t st);
size_t gemv_lds_bytes(int chunks_per_slice, int T);
int gemv_step_chunks(int which);
int gemv_max_dn_ks();

constexpr int ROUTER_SMALL_MAX_T = 8;
constexpr int ROUTER_SLICES = 8;      // H slices of the large-T router at its largest T
constexpr int ROUTER_SLICES_MAX = 64;  // ... and at its smallest (one 64-token tile)
// H slices of the large-T router for T tokens: 8, doubled while the grid
// has fewer than 256 workgroups (up to 64, and while each slice keeps a
// whole number of 32-input chunks), so that a few tokens do not read the
// whole router through a handful of workgroups.
int router_slices(int T, int H);
// the few-token row router (2 .. 16 tokens; rslices = 1)
bool router_t_ok(int T, int H, const float* wr_rows);
size_t router_logit_rows(int Tmax);  // rslices * T at most, over T <= Tmax

}  // namespace moe
