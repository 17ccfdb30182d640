// moe_ctx.h -- the library context (internal; the public ABI is include/moe.h).
#pragma once

#include <vector>

#include "moe_internal.h"

struct moe_ctx {
    moe_config cfg;
    hipStream_t stream = nullptr;
    int device = 0;
    size_t slot_bytes = 0;
    int shared_fmt = 0;        // resolved format of the shared experts
    size_t shared_bytes = 0;   // bytes of one shared expert's slot
    int Epad = 0;
    uint8_t* pool = nullptr;
    float* wr = nullptr;
    float* wr_rows = nullptr;  // the router weights again, row-major [L][E][H]
    uint4* wr16 = nullptr;     // and as split fp16 operands [L][Epad/32][H/16][64][2] (large T)
    float2* wr16s = nullptr;   // [L][Epad] their per-expert scales
    float* bias = nullptr;
    int* tbl = nullptr;
    std::vector<int> tbl_host;
    uint8_t* shared = nullptr;
    uint8_t* staging = nullptr;
    // workspace
    float* part = nullptr;
    float* tpart = nullptr;
    float* logits = nullptr;
    int32_t* ids = nullptr;
    float* wts = nullptr;
    moe::TokStat* tok = nullptr;
    uint4* xq = nullptr;
    float2* xsc = nullptr;
    int32_t* cnt = nullptr;
    int32_t* off = nullptr;
    int32_t* perm = nullptr;
    int32_t* active = nullptr;
    int32_t* n_active = nullptr;
    moe::Group* groups = nullptr;
    int32_t* n_groups = nullptr;
    uint4* hq = nullptr;
    float2* hsc = nullptr;
    float* gpart = nullptr;
    size_t gpart_bytes = 0;
    float* ypart = nullptr;
    size_t ypart_bytes = 0;
    float2* xrow = nullptr;
    float2* hrow = nullptr;
    float* hbuf = nullptr;
    float* hf = nullptr;
    int2* tiles = nullptr;
    int32_t* n_tiles = nullptr;
    uint32_t* counters = nullptr;
    uint32_t* dn_cnt = nullptr;  // [H/64][64]: one counter per 256-byte line
    uint32_t* rt_cnt = nullptr;  // [17][64]: the one-token router's arrival counters
    uint64_t* rt_tag = nullptr;  // [256]: the one-token router's tagged logits
    uint32_t* rt_epoch = nullptr;  // [1]: tag of its last selection
    uint32_t* status = nullptr;
    size_t status_words = 0;
    int gemm_min_tokens = 64;
    bool tok1 = true;          // one token: the k_tok1 kernels where the shape allows
    bool dn_fused = true;      // one token: the down GEMV's last unit per block combines
    int lds_max = 65536;
    hipError_t last_err = hipSuccess;
    // timing
    bool timing = false;
    std::vector<hipEvent_t> events;  // marker pool, reused after each summary
    std::vector<const char*> names;  // per marker: kernel that follows; nullptr = end of a forward
    int n_marks = 0;
    std::vector<void*> allocs;
    // residency (moe_stage.hip): asynchronous loads on copy streams of the
    // library's own, ordered against the compute stream per slot
    static constexpr int kCopyStreams = 2;
    hipStream_t copy_streams[kCopyStreams] = {nullptr, nullptr};
    int next_copy = 0;
    std::vector<int> slot_refs;            // slot-table entries naming each slot
    std::vector<hipEvent_t> copy_done;     // per slot: its last asynchronous load
    std::vector<hipEvent_t> slot_free;     // per slot: compute-stream point after a write by it
    std::vector<uint8_t> copy_pending;     // copy_done recorded, not yet waited by the compute stream
    std::vector<uint8_t> free_pending;     // slot_free recorded, not yet waited by a load
    std::vector<std::vector<int>> slot_layers;  // layers whose table named the slot since its load
    std::vector<uint64_t> copy_seq;        // per slot: order of its last load
    std::vector<uint8_t> copy_sid;         // per slot: copy stream of its last load
    uint64_t copy_counter = 0;
    std::vector<std::pair<int, int>> pending_ups;  // table updates not yet launched
    bool track_fwd = false;                // record layer_fwd after each forward
    std::vector<hipEvent_t> layer_fwd;     // per layer: after its latest forward
    std::vector<uint8_t> layer_fwd_rec;    // layer_fwd recorded at least once
    int stage_first = -1, stage_per_layer = 0;
    std::vector<int> stage_ids;            // [layer][per_layer] expert held by each staging slot
    std::vector<int64_t> stage_used;       // step at which that expert was last wanted
    int64_t stage_step = 0;
};

namespace moe {

int hip_ok(hipError_t e);
int hip_rc(moe_ctx* c, hipError_t e);  // records a failing HIP call for moe_last_error

// Residency bookkeeping shared by the synchronous and asynchronous paths.
int residency_init(moe_ctx* c);
void residency_destroy(moe_ctx* c);
// Before the compute stream writes or reads a slot's bytes itself: wait for
// an asynchronous load into it that the compute stream has not waited for.
int slot_compute_ready(moe_ctx* c, uint8_t* dst);
// After the compute stream has enqueued a write into a slot: later
// asynchronous loads into that slot wait for it.
int slot_compute_written(moe_ctx* c, uint8_t* dst);
// After a forward of a layer is enqueued (reads the slots its table names).
int forward_done(moe_ctx* c, int layer);

}  // namespace moe
