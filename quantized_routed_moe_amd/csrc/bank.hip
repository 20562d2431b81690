// Slot bank: N < E expert slots resident in HBM, paged from a pool of all E
// experts in pinned host memory -- the MI355X counterpart of the pages' SSD
// sidecar, where routed experts stay outside the dense model and are paged
// through a bounded cache of expert slots (Anemll/ds4-ssd README, section
// "Run SSD Sidecar Mode": --moe-slot-bank / --ssd-cache; the 10100.com
// article on ds4-ssd, section 核心功能).  The pages name no replacement
// policy; the bank evicts its least recently used slot.
//
// Host bookkeeping (moe_bank_reset / moe_bank_plan), the host -> device
// copies of planned loads (moe_bank_fetch: DMA from pinned memory, queued on
// the caller's stream), and moe_layer_banked, which composes the public
// entry points: route, dispatch, one synchronisation to learn which experts
// have rows, then per pass of at most N experts the loads, the device slot
// map and the expert FFN, and one combine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/moe.h"
#include "common.hpp"
#include "workspace.hpp"

namespace qrmoe {

// Slot map of one pass, passed by value so the launch carries it (no host
// staging buffer that a later pass could overwrite before the copy ran).
struct SlotMap {
    int32_t v[kMaxExperts];
};

__global__ void write_slot_map_kernel(int32_t* __restrict__ map, SlotMap m, int E) {
    if (static_cast<int>(threadIdx.x) < E) map[threadIdx.x] = m.v[threadIdx.x];
}

namespace {

int check_bank(const moe_bank* b) {
    if (!b || !b->slot_of_expert || !b->expert_of_slot || !b->last_use) return MOE_ERR_NULL;
    if (b->E < 1 || b->E > kMaxExperts || b->num_slots < 1 || b->num_slots > b->E) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Bytes of one slot of each array of a tile-layout matrix of n rows x K.
bool slot_bytes(int fmt, int n, int K, size_t* codes, size_t* scales) {
    size_t mins = 0;
    return moe_qmat_bytes(fmt, MOE_LAYOUT_TILES, 1, n, K, codes, scales, &mins) > 0;
}

int check_pack(const moe_experts* ex, int fmt) {
    if (!ex) return MOE_ERR_NULL;
    const moe_qmat* m[3] = {&ex->gate, &ex->up, &ex->down};
    for (const moe_qmat* q : m) {
        if (q->fmt != fmt || q->layout != MOE_LAYOUT_TILES || q->mins) return MOE_ERR_FORMAT;
        if (!q->codes || !q->scales) return MOE_ERR_NULL;
    }
    return MOE_OK;
}

}  // namespace
}  // namespace qrmoe

using qrmoe::kMaxExperts;

extern "C" {

int moe_bank_reset(moe_bank* b) {
    const int rc = qrmoe::check_bank(b);
    if (rc != MOE_OK) return rc;
    for (int e = 0; e < b->E; ++e) b->slot_of_expert[e] = -1;
    for (int s = 0; s < b->num_slots; ++s) {
        b->expert_of_slot[s] = -1;
        b->last_use[s] = 0;
    }
    b->clock = 0;
    return MOE_OK;
}

int moe_bank_plan(moe_bank* b, const int32_t* want, int32_t n_want, int32_t* load_expert, int32_t* load_slot,
                  int32_t* n_load) {
    int rc = qrmoe::check_bank(b);
    if (rc != MOE_OK) return rc;
    if (!n_load || (n_want > 0 && (!want || !load_expert || !load_slot))) return MOE_ERR_NULL;
    if (n_want < 0 || n_want > b->num_slots) return MOE_ERR_SHAPE;
    bool wanted[kMaxExperts] = {};
    for (int i = 0; i < n_want; ++i) {
        const int e = want[i];
        if (e < 0 || e >= b->E || wanted[e]) return MOE_ERR_SHAPE;
        wanted[e] = true;
    }
    int n = 0;
    for (int i = 0; i < n_want; ++i) {
        const int e = want[i];
        if (b->slot_of_expert[e] >= 0) continue;          // hit
        // victim: lowest empty slot, else the least recently used slot whose
        // expert this pass does not want (ties: lowest slot)
        int victim = -1;
        for (int s = 0; s < b->num_slots && victim < 0; ++s)
            if (b->expert_of_slot[s] < 0) victim = s;
        if (victim < 0) {
            for (int s = 0; s < b->num_slots; ++s) {
                if (wanted[b->expert_of_slot[s]]) continue;
                if (victim < 0 || b->last_use[s] < b->last_use[victim]) victim = s;
            }
        }
        // n_want <= num_slots and every wanted resident expert holds its own
        // slot, so a slot is always free for a miss
        const int old = b->expert_of_slot[victim];
        if (old >= 0) b->slot_of_expert[old] = -1;
        b->expert_of_slot[victim] = e;
        b->slot_of_expert[e] = victim;
        load_expert[n] = e;
        load_slot[n] = victim;
        ++n;
    }
    for (int i = 0; i < n_want; ++i) b->last_use[b->slot_of_expert[want[i]]] = ++b->clock;
    *n_load = n;
    return MOE_OK;
}

int moe_bank_fetch(const moe_experts* pool, const moe_experts* slots, int32_t d, int32_t f,
                   const int32_t* load_expert, const int32_t* load_slot, int32_t n_load, hipStream_t stream) {
    if (!pool || !slots) return MOE_ERR_NULL;
    const int fmt = pool->gate.fmt;
    int rc;
    if ((rc = qrmoe::check_pack(pool, fmt)) != MOE_OK) return rc;
    if ((rc = qrmoe::check_pack(slots, fmt)) != MOE_OK) return rc;
    if (n_load < 0) return MOE_ERR_SHAPE;
    if (n_load > 0 && (!load_expert || !load_slot)) return MOE_ERR_NULL;
    const moe_qmat* src[3] = {&pool->gate, &pool->up, &pool->down};
    const moe_qmat* dst[3] = {&slots->gate, &slots->up, &slots->down};
    const int n_of[3] = {f, f, d}, k_of[3] = {d, d, f};
    size_t cb[3], sb[3];
    for (int m = 0; m < 3; ++m)
        if (!qrmoe::slot_bytes(fmt, n_of[m], k_of[m], &cb[m], &sb[m])) return MOE_ERR_SHAPE;
    for (int i = 0; i < n_load; ++i) {
        const int e = load_expert[i], s = load_slot[i];
        if (e < 0 || e >= pool->num_slots || s < 0 || s >= slots->num_slots) return MOE_ERR_SHAPE;
    }
    for (int i = 0; i < n_load; ++i) {
        const size_t e = static_cast<size_t>(load_expert[i]), s = static_cast<size_t>(load_slot[i]);
        for (int m = 0; m < 3; ++m) {
            const char* sc = static_cast<const char*>(src[m]->codes);
            const char* ss = static_cast<const char*>(src[m]->scales);
            char* dc = static_cast<char*>(const_cast<void*>(dst[m]->codes));
            char* ds = static_cast<char*>(const_cast<void*>(dst[m]->scales));
            if (hipMemcpyAsync(dc + s * cb[m], sc + e * cb[m], cb[m], hipMemcpyHostToDevice, stream) != hipSuccess ||
                hipMemcpyAsync(ds + s * sb[m], ss + e * sb[m], sb[m], hipMemcpyHostToDevice, stream) != hipSuccess)
                return MOE_ERR_HIP;
        }
    }
    return MOE_OK;
}

int moe_layer_banked(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                     float* logits, const moe_experts* pool, moe_bank* bank, const moe_experts* slots,
                     int32_t* slot_map, int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream, moe_bank_stats* stats) {
    if (!shape || !pool || !slots || !slot_map || !ws) return MOE_ERR_NULL;
    int rc = qrmoe::check_bank(bank);
    if (rc != MOE_OK) return rc;
    const size_t need = moe_layer_workspace_bytes(shape);      // 0: invalid shape
    if (need == 0) return MOE_ERR_SHAPE;
    const moe_shape& s = *shape;
    if (bank->E != s.E || pool->num_slots < s.E || slots->num_slots != bank->num_slots) return MOE_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(slot_map) & 3) != 0) return MOE_ERR_ALIGN;
    if (stats) *stats = moe_bank_stats{0, 0, 0, 0, 0};
    if (s.T == 0) return MOE_OK;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    const qrmoe::LayerCarve c = qrmoe::layer_carve(s);
    char* base = static_cast<char*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(base + c.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(base + c.inv);
    float* y = reinterpret_cast<float*>(base + c.y);
    if ((rc = moe_route_topk(shape, x, w_router, bias, logits, topk_ids, topk_w, stream)) != MOE_OK) return rc;
    if ((rc = moe_dispatch(shape, topk_ids, offsets, perm, inv, ws, ws_bytes, stream)) != MOE_OK) return rc;
    int32_t off[kMaxExperts + 1];
    if (hipMemcpyAsync(off, offsets, (s.E + 1) * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MOE_ERR_HIP;
    // active experts: resident ones first, then the rest, each in id order
    int32_t order[kMaxExperts];
    int n_act = 0, hits = 0;
    for (int e = 0; e < s.E; ++e)
        if (off[e + 1] > off[e] && bank->slot_of_expert[e] >= 0) order[n_act++] = e;
    hits = n_act;
    for (int e = 0; e < s.E; ++e)
        if (off[e + 1] > off[e] && bank->slot_of_expert[e] < 0) order[n_act++] = e;
    const int N = bank->num_slots;
    const int passes = n_act == 0 ? 1 : (n_act + N - 1) / N;
    moe_experts ex = *slots;
    ex.slot_of_expert = slot_map;
    size_t per_expert = 0;
    {
        size_t cb, sb;
        const int n_of[3] = {s.f, s.f, s.d}, k_of[3] = {s.d, s.d, s.f};
        for (int m = 0; m < 3; ++m) {
            if (!qrmoe::slot_bytes(pool->gate.fmt, n_of[m], k_of[m], &cb, &sb)) return MOE_ERR_SHAPE;
            per_expert += cb + sb;
        }
    }
    int misses = 0;
    for (int p = 0; p < passes; ++p) {
        const int lo = p * N, n_want = std::min(N, n_act - lo);
        int32_t load_e[kMaxExperts], load_s[kMaxExperts], n_load = 0;
        if ((rc = moe_bank_plan(bank, order + lo, n_want, load_e, load_s, &n_load)) != MOE_OK) return rc;
        if ((rc = moe_bank_fetch(pool, slots, s.d, s.f, load_e, load_s, n_load, stream)) != MOE_OK) return rc;
        misses += n_load;
        qrmoe::SlotMap m;
        for (int e = 0; e < kMaxExperts; ++e) m.v[e] = MOE_SLOT_SKIP;
        for (int i = 0; i < n_want; ++i) m.v[order[lo + i]] = bank->slot_of_expert[order[lo + i]];
        qrmoe::write_slot_map_kernel<<<1, kMaxExperts, 0, stream>>>(slot_map, m, s.E);
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
        if ((rc = moe_expert_ffn(shape, x, &ex, offsets, perm, y, ws, ws_bytes, stream)) != MOE_OK) return rc;
    }
    if ((rc = moe_combine(shape, y, inv, topk_w, out, stream)) != MOE_OK) return rc;
    if (stats) *stats = moe_bank_stats{n_act, hits, misses, passes, static_cast<int64_t>(misses) * static_cast<int64_t>(per_expert)};
    return MOE_OK;
}

}  // extern "C"
