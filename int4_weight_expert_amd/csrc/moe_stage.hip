// moe_stage.hip -- expert residency around the slot pool: the slot table
// (synchronous and asynchronous updates), asynchronous loads of slot images
// from host memory on copy streams of the library's own, the staged
// executor's sticky slots, whole-layer loads, and the slot image on the host.
//
// Sources, cited by page title and section:
//   Edge0 write-up (magicnetworld.com) §十四: the staged executor keeps fixed,
//     double-buffered slots whose routing goes through a slot table, and per
//     step rewrites only the experts that changed (sticky slots updated in
//     place) instead of rebuilding the layer's stacked tensors; the
//     whole-layer path reads every expert of a layer at once for prefill,
//     overlapped with the previous layer's GPU work;
//   "惊呆了！25GB 内存上运行 GLM 5.2 744B 模型" §13: an expert's three
//     matrices stored contiguously are read with one read into its slab.
//
// Ordering.  Loads run on two copy streams used in turn; the forward runs on
// the compute stream.  Per slot, the library keeps
//   - copy_done: recorded on the copy stream after a load into the slot;
//     the compute stream waits for it before the table names the slot or
//     before it touches the slot's bytes itself;
//   - the layers whose table named the slot since its last load: a load
//     into the slot waits for the latest forward of each of them (an event
//     recorded after every forward once asynchronous loads are in use), so
//     a forward that may still read the old expert finishes first, and a
//     load never waits for compute enqueued after the slot left the table;
//     where a layer had no recorded forward, the load waits for everything
//     enqueued on the compute stream so far;
//   - slot_free: recorded on the compute stream after the compute stream
//     wrote the slot itself (synchronous loads); a later load waits for it.
// A slot still named by the table cannot take an asynchronous load.
#include <string.h>

#include <algorithm>
#include <map>
#include <vector>

#include "moe_ctx.h"

using namespace moe;

namespace {

constexpr int kTblBatch = 64;

struct TblUpd {
    int n;
    int idx[kTblBatch];
    int val[kTblBatch];
};

__global__ void __launch_bounds__(kTblBatch) k_set_table(int* __restrict__ tbl, TblUpd u)
{
    const int t = threadIdx.x;
    if (t < u.n) tbl[u.idx[t]] = u.val[t];
}

hipEvent_t slot_event(std::vector<hipEvent_t>& v, int slot)
{
    if (!v[slot]) {
        if (hipEventCreateWithFlags(&v[slot], hipEventDisableTiming) != hipSuccess) v[slot] = nullptr;
    }
    return v[slot];
}

int slot_index(const moe_ctx* c, const uint8_t* p)
{
    if (!c->pool || p < c->pool) return -1;
    const size_t off = (size_t)(p - c->pool);
    if (off >= (size_t)c->cfg.n_slots * c->slot_bytes) return -1;
    return (int)(off / c->slot_bytes);
}

// Table updates (entry layer*E + id -> slot, -1 = unmap).  record_update
// keeps the host's view (table mirror, reference counts, the layers that
// named a slot) at once; flush_updates makes the compute stream wait for
// the loads into newly named slots (once per copy stream: its latest such
// load, since a stream's copies finish in order; none if already done) and
// writes the device table, in stream order, later entries winning.
void record_update(moe_ctx* c, int idx, int slot)
{
    const int old = c->tbl_host[idx];
    if (old == slot) return;
    if (old >= 0) --c->slot_refs[old];
    if (slot >= 0) {
        c->slot_refs[slot]++;
        const int layer = idx / c->cfg.n_experts;
        auto& v = c->slot_layers[slot];
        if (std::find(v.begin(), v.end(), layer) == v.end()) v.push_back(layer);
    }
    c->tbl_host[idx] = slot;
    c->pending_ups.push_back({idx, slot});
}

int flush_updates(moe_ctx* c)
{
    if (c->pending_ups.empty()) return MOE_OK;
    std::map<int, int> last;
    for (const auto& u : c->pending_ups) last[u.first] = u.second;
    c->pending_ups.clear();
    int wait_slot[moe_ctx::kCopyStreams];
    for (int& w : wait_slot) w = -1;
    for (const auto& u : last) {
        const int s = u.second;
        if (s < 0 || !c->copy_pending[s]) continue;
        int& w = wait_slot[c->copy_sid[s]];
        if (w < 0 || c->copy_seq[s] > c->copy_seq[w]) w = s;
        c->copy_pending[s] = 0;
    }
    for (int w : wait_slot) {
        if (w < 0 || hipEventQuery(c->copy_done[w]) == hipSuccess) continue;
        const hipError_t e = hipStreamWaitEvent(c->stream, c->copy_done[w], 0);
        if (e != hipSuccess) return hip_rc(c, e);
    }
    std::vector<std::pair<int, int>> ups(last.begin(), last.end());
    for (size_t i = 0; i < ups.size(); i += kTblBatch) {
        TblUpd t{};
        t.n = (int)std::min(ups.size() - i, (size_t)kTblBatch);
        for (int k = 0; k < t.n; ++k) {
            t.idx[k] = ups[i + k].first;
            t.val[k] = ups[i + k].second;
        }
        hipLaunchKernelGGL(k_set_table, dim3(1), dim3(kTblBatch), 0, c->stream, c->tbl, t);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_rc(c, e);
    }
    return MOE_OK;
}

int apply_updates(moe_ctx* c, const std::vector<std::pair<int, int>>& ups)
{
    for (const auto& u : ups) record_update(c, u.first, u.second);
    return flush_updates(c);
}

// The copy stream waits until no forward that may read the slot's old
// expert is left to run.
int wait_slot_readers(moe_ctx* c, int slot, hipStream_t cs)
{
    hipError_t e = hipSuccess;
    bool tail = false;
    for (int layer : c->slot_layers[slot]) {
        if (!c->layer_fwd_rec[layer]) {
            tail = true;
            continue;
        }
        if (hipEventQuery(c->layer_fwd[layer]) == hipSuccess) continue;  // already done
        e = hipStreamWaitEvent(cs, c->layer_fwd[layer], 0);
        if (e != hipSuccess) return hip_rc(c, e);
    }
    if (tail) {
        hipEvent_t ev = slot_event(c->slot_free, slot);
        if (!ev) return MOE_E_HIP;
        e = hipEventRecord(ev, c->stream);
        if (e != hipSuccess) return hip_rc(c, e);
        c->free_pending[slot] = 1;
    }
    if (c->free_pending[slot]) {
        e = hipStreamWaitEvent(cs, c->slot_free[slot], 0);
        if (e != hipSuccess) return hip_rc(c, e);
        c->free_pending[slot] = 0;
    }
    c->slot_layers[slot].clear();
    return MOE_OK;
}

int next_copy_stream(moe_ctx* c)
{
    c->track_fwd = true;
    const int s = c->next_copy;
    c->next_copy = (c->next_copy + 1) % moe_ctx::kCopyStreams;
    return s;
}

int note_copy(moe_ctx* c, int slot, int sid)
{
    hipEvent_t ev = slot_event(c->copy_done, slot);
    if (!ev) return MOE_E_HIP;
    const hipError_t e = hipEventRecord(ev, c->copy_streams[sid]);
    if (e != hipSuccess) return hip_rc(c, e);
    c->copy_pending[slot] = 1;
    c->copy_sid[slot] = (uint8_t)sid;
    c->copy_seq[slot] = ++c->copy_counter;
    return MOE_OK;
}

// An asynchronous copy of one slot image into a slot not named by the table.
int load_async(moe_ctx* c, int slot, const void* image)
{
    if (c->slot_refs[slot] > 0) return MOE_E_BUSY;
    const int sid = next_copy_stream(c);
    hipStream_t cs = c->copy_streams[sid];
    const int rc = wait_slot_readers(c, slot, cs);
    if (rc) return rc;
    const hipError_t e = hipMemcpyAsync(c->pool + (size_t)slot * c->slot_bytes, image,
                                        c->slot_bytes, hipMemcpyDefault, cs);
    if (e != hipSuccess) return hip_rc(c, e);
    return note_copy(c, slot, sid);
}

size_t image_bytes(int fmt, int64_t H, int64_t I)
{
    const int64_t packed = 3 * H * I / 2;
    if (fmt == MOE_W_INT4_ROW) return (size_t)(packed + 4 * (2 * I + H));
    if (fmt == MOE_W_INT4_AFFINE_G64) return (size_t)(packed + 12 * H * I / 64);
    return 0;
}

}  // namespace

namespace moe {

int residency_init(moe_ctx* c)
{
    const int n = c->cfg.n_slots;
    c->slot_refs.assign(n, 0);
    c->copy_done.assign(n, nullptr);
    c->slot_free.assign(n, nullptr);
    c->copy_pending.assign(n, 0);
    c->free_pending.assign(n, 0);
    c->slot_layers.assign(n, {});
    c->copy_seq.assign(n, 0);
    c->copy_sid.assign(n, 0);
    c->layer_fwd.assign(c->cfg.n_layers, nullptr);
    c->layer_fwd_rec.assign(c->cfg.n_layers, 0);
    for (auto& s : c->copy_streams) {
        const hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e != hipSuccess) return hip_ok(e);
    }
    return MOE_OK;
}

void residency_destroy(moe_ctx* c)
{
    for (auto& s : c->copy_streams)
        if (s) hipStreamSynchronize(s);
    for (hipEvent_t e : c->copy_done)
        if (e) hipEventDestroy(e);
    for (hipEvent_t e : c->slot_free)
        if (e) hipEventDestroy(e);
    for (hipEvent_t e : c->layer_fwd)
        if (e) hipEventDestroy(e);
    for (auto& s : c->copy_streams) {
        if (s) hipStreamDestroy(s);
        s = nullptr;
    }
}

int forward_done(moe_ctx* c, int layer)
{
    if (!c->track_fwd) return MOE_OK;
    hipEvent_t ev = slot_event(c->layer_fwd, layer);
    if (!ev) return MOE_E_HIP;
    const hipError_t e = hipEventRecord(ev, c->stream);
    if (e != hipSuccess) return hip_rc(c, e);
    c->layer_fwd_rec[layer] = 1;
    return MOE_OK;
}

int slot_compute_ready(moe_ctx* c, uint8_t* dst)
{
    const int s = slot_index(c, dst);
    if (s < 0 || !c->copy_pending[s]) return MOE_OK;
    c->copy_pending[s] = 0;
    if (hipEventQuery(c->copy_done[s]) == hipSuccess) return MOE_OK;
    return hip_rc(c, hipStreamWaitEvent(c->stream, c->copy_done[s], 0));
}

int slot_compute_written(moe_ctx* c, uint8_t* dst)
{
    const int s = slot_index(c, dst);
    if (s < 0) return MOE_OK;
    hipEvent_t ev = slot_event(c->slot_free, s);
    if (!ev) return MOE_E_HIP;
    const hipError_t e = hipEventRecord(ev, c->stream);
    if (e != hipSuccess) return hip_rc(c, e);
    c->free_pending[s] = 1;
    return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_map_expert(moe_ctx* c, int layer, int expert_id, int slot)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || expert_id < 0 ||
        expert_id >= c->cfg.n_experts)
        return MOE_E_ARG;
    if (slot < MOE_SLOT_REMOTE || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    const int rc = apply_updates(c, {{layer * c->cfg.n_experts + expert_id, slot}});
    if (rc) return rc;
    return hip_rc(c, hipStreamSynchronize(c->stream));
}

int moe_map_experts_async(moe_ctx* c, int layer, int n, const int* expert_ids, const int* slots)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || n < 0 || (n && (!expert_ids || !slots)))
        return MOE_E_ARG;
    std::vector<std::pair<int, int>> ups;
    for (int i = 0; i < n; ++i) {
        if (expert_ids[i] < 0 || expert_ids[i] >= c->cfg.n_experts) return MOE_E_ARG;
        if (slots[i] < MOE_SLOT_REMOTE || slots[i] >= c->cfg.n_slots) return MOE_E_SLOT;
        ups.push_back({layer * c->cfg.n_experts + expert_ids[i], slots[i]});
    }
    return apply_updates(c, ups);
}

int moe_load_image_async(moe_ctx* c, int slot, const void* image, size_t nbytes)
{
    if (!c || !image) return MOE_E_ARG;
    if (slot < 0 || slot >= c->cfg.n_slots) return MOE_E_SLOT;
    if (nbytes != c->slot_bytes) return MOE_E_SIZE;
    return load_async(c, slot, image);
}

int moe_load_layer_async(moe_ctx* c, int layer, int first_slot, int n, const void* images,
                         size_t nbytes)
{
    if (!c || !images || layer < 0 || layer >= c->cfg.n_layers || n < 1 ||
        n > c->cfg.n_experts)
        return MOE_E_ARG;
    if (first_slot < 0 || first_slot + n > c->cfg.n_slots) return MOE_E_SLOT;
    if (nbytes != (size_t)n * c->slot_bytes) return MOE_E_SIZE;
    for (int s = first_slot; s < first_slot + n; ++s)
        if (c->slot_refs[s] > 0) return MOE_E_BUSY;
    const int sid = next_copy_stream(c);
    hipStream_t cs = c->copy_streams[sid];
    for (int s = first_slot; s < first_slot + n; ++s) {
        const int rc = wait_slot_readers(c, s, cs);
        if (rc) return rc;
    }
    const hipError_t e = hipMemcpyAsync(c->pool + (size_t)first_slot * c->slot_bytes, images,
                                        nbytes, hipMemcpyDefault, cs);
    if (e != hipSuccess) return hip_rc(c, e);
    for (int s = first_slot; s < first_slot + n; ++s) {
        const int rc = note_copy(c, s, sid);
        if (rc) return rc;
    }
    std::vector<std::pair<int, int>> ups;
    for (int i = 0; i < n; ++i) ups.push_back({layer * c->cfg.n_experts + i, first_slot + i});
    return apply_updates(c, ups);
}

int moe_sync_copies(moe_ctx* c)
{
    if (!c) return MOE_E_ARG;
    for (auto& s : c->copy_streams) {
        const hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_rc(c, e);
    }
    return MOE_OK;
}

int moe_set_staging(moe_ctx* c, int first_slot, int per_layer)
{
    if (!c || per_layer < 1 || per_layer > c->cfg.n_experts) return MOE_E_ARG;
    if (first_slot < 0 || first_slot + (int64_t)per_layer * c->cfg.n_layers > c->cfg.n_slots)
        return MOE_E_SLOT;
    c->stage_first = first_slot;
    c->stage_per_layer = per_layer;
    c->stage_ids.assign((size_t)per_layer * c->cfg.n_layers, -1);
    c->stage_used.assign((size_t)per_layer * c->cfg.n_layers, -1);
    c->stage_step = 0;
    return MOE_OK;
}

int moe_sticky_plan(const int* held, const int64_t* last_used, int n_slots, const int* want,
                    int n_want, int* slot_of, int* load)
{
    if (n_slots < 0 || n_want < 0 || n_want > n_slots) return -1;
    if ((n_slots && (!held || !last_used)) || (n_want && (!want || !slot_of || !load))) return -1;
    for (int i = 0; i < n_want; ++i) {
        if (want[i] < 0) return -1;
        for (int k = 0; k < i; ++k)
            if (want[k] == want[i]) return -1;
    }
    std::vector<char> taken(n_slots, 0);
    for (int i = 0; i < n_want; ++i) {
        slot_of[i] = -1;
        load[i] = 0;
        for (int j = 0; j < n_slots; ++j)
            if (held[j] == want[i] && !taken[j]) {
                slot_of[i] = j;
                taken[j] = 1;
                break;
            }
    }
    // free slots: empty ones first, then the least recently wanted
    std::vector<int> order;
    for (int j = 0; j < n_slots; ++j)
        if (!taken[j]) order.push_back(j);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        const bool ea = held[a] < 0, eb = held[b] < 0;
        if (ea != eb) return ea;
        return last_used[a] < last_used[b];
    });
    int next = 0, n_load = 0;
    for (int i = 0; i < n_want; ++i)
        if (slot_of[i] < 0) {
            slot_of[i] = order[next++];
            load[i] = 1;
            ++n_load;
        }
    return n_load;
}

int moe_stage_experts(moe_ctx* c, int layer, int n, const int* expert_ids,
                      const void* const* images, int* n_loaded)
{
    if (!c || layer < 0 || layer >= c->cfg.n_layers || n < 0 || (n && (!expert_ids || !images)))
        return MOE_E_ARG;
    if (c->stage_first < 0) return MOE_E_ARG;
    const int P = c->stage_per_layer, E = c->cfg.n_experts;
    if (n > P) return MOE_E_ARG;
    for (int i = 0; i < n; ++i)
        if (expert_ids[i] < 0 || expert_ids[i] >= E) return MOE_E_ARG;
    int* held = c->stage_ids.data() + (size_t)layer * P;
    int64_t* used = c->stage_used.data() + (size_t)layer * P;
    const int base = c->stage_first + layer * P;
    std::vector<int> slot_of(n), load(n);
    const int nl = moe_sticky_plan(held, used, P, expert_ids, n, slot_of.data(), load.data());
    if (nl < 0) return MOE_E_ARG;
    for (int i = 0; i < n; ++i)
        if (load[i] && !images[i]) return MOE_E_ARG;
    // evict: the replaced experts leave the table (the device table is
    // written once, after the loads are enqueued: no forward can come in
    // between, and the loads wait for the forwards that may read the slots)
    for (int i = 0; i < n; ++i) {
        if (!load[i]) continue;
        const int j = slot_of[i], old = held[j];
        if (old >= 0 && c->tbl_host[layer * E + old] == base + j) record_update(c, layer * E + old, -1);
        held[j] = -1;
    }
    int rc = MOE_OK;
    for (int i = 0; i < n && rc == MOE_OK; ++i)
        if (load[i]) rc = load_async(c, base + slot_of[i], images[i]);
    if (rc) {
        flush_updates(c);
        return rc;
    }
    for (int i = 0; i < n; ++i) {
        const int j = slot_of[i];
        held[j] = expert_ids[i];
        used[j] = c->stage_step;
        record_update(c, layer * E + expert_ids[i], base + j);
    }
    ++c->stage_step;
    rc = flush_updates(c);
    if (rc) return rc;
    if (n_loaded) *n_loaded = nl;
    return MOE_OK;
}

size_t moe_image_bytes(int wfmt, int hidden, int inter)
{
    if (hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64) return 0;
    return image_bytes(wfmt, hidden, inter);
}

int moe_blob_to_image(int wfmt, int hidden, int inter, const void* blob, size_t nbytes,
                      void* image)
{
    const size_t want = moe_image_bytes(wfmt, hidden, inter);
    if (!want || !blob || !image || blob == image) return MOE_E_ARG;
    if (nbytes != want) return MOE_E_SIZE;
    const uint8_t* src = (const uint8_t*)blob;
    uint8_t* dst = (uint8_t*)image;
    const int64_t H = hidden, I = inter;
    const int64_t gq = I * (H / 2), dq = H * (I / 2);
    const uint8_t flip = wfmt == MOE_W_INT4_ROW ? 0x88 : 0x00;
    const int64_t mats[3][3] = {{0, I, H}, {gq, I, H}, {2 * gq, H, I}};  // offset, O, In
    for (const auto& m : mats) {
        const int64_t C = m[2] / 32;  // 8-row groups, 128 bytes per chunk
        for (int64_t q = 0; q < m[1] / 8; ++q)
            for (int64_t c = 0; c < C; ++c)
                for (int64_t r = 0; r < 8; ++r) {
                    const uint8_t* s = src + m[0] + (q * 8 + r) * (m[2] / 2) + c * 16;
                    uint8_t* d = dst + m[0] + ((q * C + c) * 8 + r) * 16;
                    for (int k = 0; k < 16; ++k) d[k] = s[k] ^ flip;
                }
    }
    const int64_t sb = 2 * gq + dq;
    if (wfmt == MOE_W_INT4_ROW) {
        memcpy(dst + sb, src + sb, (size_t)(2 * I + H) * 4);
    } else {
        const int64_t ga = I * (H / 64) * 4;
        const int64_t pm[3][3] = {{sb, I, H / 64}, {sb + ga, I, H / 64}, {sb + 2 * ga, H, I / 64}};
        for (const auto& m : pm)
            for (int64_t q = 0; q < m[1] / 8; ++q)
                for (int64_t g = 0; g < m[2]; ++g)
                    for (int64_t r = 0; r < 8; ++r)
                        memcpy(dst + m[0] + ((q * m[2] + g) * 8 + r) * 4,
                               src + m[0] + ((q * 8 + r) * m[2] + g) * 4, 4);
    }
    return MOE_OK;
}

}  // extern "C"
