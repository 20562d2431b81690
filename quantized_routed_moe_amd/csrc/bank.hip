// Slot bank: N < E expert slots resident in HBM, paged from a pool of all E
// experts in pinned host memory -- the MI355X counterpart of the pages' SSD
// sidecar, where routed experts stay outside the dense model and are paged
// through a bounded cache of expert slots whose size is a slot count or a
// byte budget, `auto` taking what memory is left, clamped so that a prefill
// chunk still fits (Anemll/ds4-ssd README, section "Run SSD Sidecar Mode":
// --moe-slot-bank / --ssd-cache; the 10100.com article on ds4-ssd, section
// 核心功能).  The pages name no replacement policy; the bank evicts its least
// recently used slot.
//
// Host bookkeeping (moe_bank_reset / moe_bank_plan), bank sizing
// (moe_bank_slots, moe_slab_layout), the host -> device copies of planned
// loads (moe_bank_fetch: DMA from pinned memory, one copy per expert when
// both packs keep an expert's six arrays in one slab), and moe_layer_banked,
// which composes the public entry points: route, dispatch, one
// synchronisation to learn which experts have rows, then per pass of at most
// N experts the loads and the expert FFN, and one combine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "../../include/moe.h"
#include "common.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace qrmoe {

// Slot map of one FFN call, passed by value so the launch carries it (no
// host staging buffer that a later call could overwrite before the copy ran).
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
    return check::qmat_sizes(fmt, MOE_LAYOUT_TILES, 1, n, K, codes, scales, &mins);
}

// Offsets of the six arrays of one expert in a slab (gate codes, gate
// scales, up codes, up scales, down codes, down scales), each rounded up to
// 256 bytes; returns the slab size, 0 when invalid.
size_t slab_layout(int fmt, int d, int f, size_t* off) {
    if (d < 32 || f < 32 || d % 32 || f % 32) return 0;
    const int n_of[3] = {f, f, d}, k_of[3] = {d, d, f};
    size_t pos = 0;
    for (int m = 0; m < 3; ++m) {
        size_t cb, sb;
        if (!slot_bytes(fmt, n_of[m], k_of[m], &cb, &sb)) return 0;
        if (off) off[2 * m] = pos;
        pos = align256(pos + cb);
        if (off) off[2 * m + 1] = pos;
        pos = align256(pos + sb);
    }
    return pos;
}

int check_pack(const moe_experts* ex, int fmt) {
    if (!ex) return MOE_ERR_NULL;
    const moe_qmat* m[3] = {&ex->gate, &ex->up, &ex->down};
    for (const moe_qmat* q : m) {
        if (q->fmt != fmt || q->layout != MOE_LAYOUT_TILES || q->mins) return MOE_ERR_FORMAT;
        if (!q->codes || !q->scales) return MOE_ERR_NULL;
    }
    if (ex->slot_bytes % 256) return MOE_ERR_ALIGN;
    return MOE_OK;
}

// Whether every array of `ex` sits at its slab offset from gate.codes with
// slot_bytes == the slab size: then slot s of the whole expert is the one
// contiguous range [gate.codes + s * slab, + slab).
bool is_slab_pack(const moe_experts* ex, int fmt, int d, int f) {
    size_t off[6];
    const size_t slab = slab_layout(fmt, d, f, off);
    if (slab == 0 || ex->slot_bytes != slab) return false;
    const char* base = static_cast<const char*>(ex->gate.codes);
    const void* p[6] = {ex->gate.codes, ex->gate.scales, ex->up.codes, ex->up.scales, ex->down.codes, ex->down.scales};
    for (int i = 0; i < 6; ++i)
        if (static_cast<const char*>(p[i]) != base + off[i]) return false;
    return true;
}

// Checks of moe_bank_fetch's packs and sizes (no loads).
int check_fetch(const moe_experts* pool, const moe_experts* slots, int d, int f) {
    if (!pool || !slots) return MOE_ERR_NULL;
    const int fmt = pool->gate.fmt;
    int rc;
    if ((rc = check_pack(pool, fmt)) != MOE_OK) return rc;
    if ((rc = check_pack(slots, fmt)) != MOE_OK) return rc;
    if (pool->num_slots < 1 || slots->num_slots < 1) return MOE_ERR_SHAPE;
    if (slab_layout(fmt, d, f, nullptr) == 0) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// The copies of moe_bank_fetch (arguments already checked).
int enqueue_fetch(const moe_experts* pool, const moe_experts* slots, int d, int f, const int32_t* load_expert,
                  const int32_t* load_slot, int n_load, hipStream_t stream) {
    const int fmt = pool->gate.fmt;
    if (is_slab_pack(pool, fmt, d, f) && is_slab_pack(slots, fmt, d, f)) {
        const size_t slab = static_cast<size_t>(pool->slot_bytes);
        const char* src = static_cast<const char*>(pool->gate.codes);
        char* dst = static_cast<char*>(const_cast<void*>(slots->gate.codes));
        for (int i = 0; i < n_load; ++i) {
            const size_t e = static_cast<size_t>(load_expert[i]), s = static_cast<size_t>(load_slot[i]);
            if (hipMemcpyAsync(dst + s * slab, src + e * slab, slab, hipMemcpyHostToDevice, stream) != hipSuccess)
                return MOE_ERR_HIP;
        }
        return MOE_OK;
    }
    const moe_qmat* src[3] = {&pool->gate, &pool->up, &pool->down};
    const moe_qmat* dst[3] = {&slots->gate, &slots->up, &slots->down};
    const int n_of[3] = {f, f, d}, k_of[3] = {d, d, f};
    for (int m = 0; m < 3; ++m) {
        size_t cb, sb;
        slot_bytes(fmt, n_of[m], k_of[m], &cb, &sb);
        const size_t src_c = pool->slot_bytes ? pool->slot_bytes : cb, src_s = pool->slot_bytes ? pool->slot_bytes : sb;
        const size_t dst_c = slots->slot_bytes ? slots->slot_bytes : cb, dst_s = slots->slot_bytes ? slots->slot_bytes : sb;
        for (int i = 0; i < n_load; ++i) {
            const size_t e = static_cast<size_t>(load_expert[i]), s = static_cast<size_t>(load_slot[i]);
            const char* sc = static_cast<const char*>(src[m]->codes) + e * src_c;
            const char* ss = static_cast<const char*>(src[m]->scales) + e * src_s;
            char* dc = static_cast<char*>(const_cast<void*>(dst[m]->codes)) + s * dst_c;
            char* ds = static_cast<char*>(const_cast<void*>(dst[m]->scales)) + s * dst_s;
            if (hipMemcpyAsync(dc, sc, cb, hipMemcpyHostToDevice, stream) != hipSuccess ||
                hipMemcpyAsync(ds, ss, sb, hipMemcpyHostToDevice, stream) != hipSuccess)
                return MOE_ERR_HIP;
        }
    }
    return MOE_OK;
}

}  // namespace
}  // namespace qrmoe

using qrmoe::kMaxExperts;

extern "C" {

size_t moe_slab_layout(int32_t fmt, int32_t d, int32_t f, size_t* offsets) {
    size_t off[6] = {0, 0, 0, 0, 0, 0};
    const size_t slab = qrmoe::slab_layout(fmt, d, f, off);
    if (offsets)
        for (int i = 0; i < 6; ++i) offsets[i] = slab ? off[i] : 0;
    return slab;
}

int moe_bank_slots(int32_t fmt, const moe_shape* prefill_shape, uint64_t budget_bytes, uint64_t free_bytes,
                   uint64_t reserve_bytes, int32_t* num_slots) {
    if (!prefill_shape || !num_slots) return MOE_ERR_NULL;
    *num_slots = 0;
    int rc = qrmoe::check::check_shape(prefill_shape);
    if (rc != MOE_OK) return rc;
    const moe_shape& s = *prefill_shape;
    if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_Q2G32 && fmt != MOE_FMT_Q4G32) return MOE_ERR_FORMAT;
    const uint64_t slab = qrmoe::slab_layout(fmt, s.d, s.f, nullptr);
    const uint64_t ws = qrmoe::layer_carve(s).total;
    const uint64_t taken = reserve_bytes + ws;
    const uint64_t avail = free_bytes > taken ? free_bytes - taken : 0;
    const uint64_t bytes = budget_bytes ? std::min(budget_bytes, avail) : avail;
    const uint64_t n = std::min<uint64_t>(static_cast<uint64_t>(s.E), bytes / slab);
    if (n < 1) return MOE_ERR_WORKSPACE;
    *num_slots = static_cast<int32_t>(n);
    return MOE_OK;
}

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
    int rc = qrmoe::check_fetch(pool, slots, d, f);
    if (rc != MOE_OK) return rc;
    if (n_load < 0) return MOE_ERR_SHAPE;
    if (n_load > 0 && (!load_expert || !load_slot)) return MOE_ERR_NULL;
    for (int i = 0; i < n_load; ++i) {
        const int e = load_expert[i], s = load_slot[i];
        if (e < 0 || e >= pool->num_slots || s < 0 || s >= slots->num_slots) return MOE_ERR_SHAPE;
    }
    return qrmoe::enqueue_fetch(pool, slots, d, f, load_expert, load_slot, n_load, stream);
}

int moe_layer_banked(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                     float* logits, const moe_experts* pool, moe_bank* bank, const moe_experts* slots,
                     int32_t* slot_map, int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                     hipStream_t stream, moe_bank_stats* stats) {
    using namespace qrmoe::check;
    // ---- every check first: an error leaves the bank and the stream untouched
    if (!shape || !pool || !slots || !slot_map || !ws || !out) return MOE_ERR_NULL;
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if ((rc = qrmoe::check_bank(bank)) != MOE_OK) return rc;
    const moe_shape& s = *shape;
    if ((rc = qrmoe::check_fetch(pool, slots, s.d, s.f)) != MOE_OK) return rc;
    if (bank->E != s.E || pool->num_slots < s.E || slots->num_slots != bank->num_slots) return MOE_ERR_SHAPE;
    if (bank->copy_stream && (!bank->ev_copied || !bank->ev_computed)) return MOE_ERR_NULL;
    if (!aligned(slot_map, 4) || !aligned(ws, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
    if (stats) *stats = moe_bank_stats{0, 0, 0, 0, 0};
    if (s.T == 0) return MOE_OK;
    const qrmoe::LayerCarve c = qrmoe::layer_carve(s);
    if (ws_bytes < c.total) return MOE_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(base + c.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(base + c.inv);
    float* y = reinterpret_cast<float*>(base + c.y);
    moe_experts ex = *slots;
    ex.slot_of_expert = slot_map;
    if ((rc = check_route_args(s, x, w_router, bias, logits, topk_ids, topk_w)) != MOE_OK) return rc;
    if ((rc = check_ffn_args(s, x, &ex, offsets, perm, y, ws, ws_bytes)) != MOE_OK) return rc;

    // ---- route and dispatch, then learn which experts have rows
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
    const size_t per_expert = qrmoe::slab_layout(pool->gate.fmt, s.d, s.f, nullptr);
    hipStream_t cs = bank->copy_stream ? bank->copy_stream : stream;

    // One FFN call over the experts `list[0..n)` (the others skipped); with
    // n == 0 only when `always` (a call with no active expert still zeroes
    // the y rows of invalid pairs).
    auto ffn_over = [&](const int32_t* list, int n, bool always = false) -> int {
        if (n == 0 && !always) return MOE_OK;
        qrmoe::SlotMap m;
        for (int e = 0; e < kMaxExperts; ++e) m.v[e] = MOE_SLOT_SKIP;
        for (int i = 0; i < n; ++i) m.v[list[i]] = bank->slot_of_expert[list[i]];
        qrmoe::write_slot_map_kernel<<<1, kMaxExperts, 0, stream>>>(slot_map, m, s.E);
        if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;
        return moe_expert_ffn(shape, x, &ex, offsets, perm, y, ws, ws_bytes, stream);
    };
    auto fail = [&](int code) {
        // copies may not have run: forget every slot rather than keep books
        // that claim them
        moe_bank_reset(bank);
        return code;
    };
    int misses = 0;
    for (int p = 0; p < passes; ++p) {
        const int lo = p * N, n_want = std::min(N, n_act - lo);
        int32_t load_e[kMaxExperts], load_s[kMaxExperts], n_load = 0;
        // cannot fail: the pass's experts are distinct, in range, at most N
        if ((rc = moe_bank_plan(bank, order + lo, n_want, load_e, load_s, &n_load)) != MOE_OK) return fail(rc);
        misses += n_load;
        // the pass's resident experts and its misses
        int32_t res[kMaxExperts], mis[kMaxExperts];
        int n_res = 0, n_mis = 0;
        for (int i = 0; i < n_want; ++i) {
            const int e = order[lo + i];
            bool loaded = false;
            for (int j = 0; j < n_load; ++j) loaded |= load_e[j] == e;
            if (loaded) mis[n_mis++] = e;
            else res[n_res++] = e;
        }
        if (bank->copy_stream) {
            // copies into slots the previous pass's FFN reads wait for it;
            // the resident experts' FFN then runs while they land
            if (p > 0 && n_load > 0 &&
                (hipEventRecord(bank->ev_computed, stream) != hipSuccess ||
                 hipStreamWaitEvent(cs, bank->ev_computed, 0) != hipSuccess))
                return fail(MOE_ERR_HIP);
            if ((rc = qrmoe::enqueue_fetch(pool, slots, s.d, s.f, load_e, load_s, n_load, cs)) != MOE_OK)
                return fail(rc);
            if (n_load > 0 && hipEventRecord(bank->ev_copied, cs) != hipSuccess) return fail(MOE_ERR_HIP);
            if ((rc = ffn_over(res, n_res)) != MOE_OK) return fail(rc);
            if (n_load > 0 && hipStreamWaitEvent(stream, bank->ev_copied, 0) != hipSuccess) return fail(MOE_ERR_HIP);
            if ((rc = ffn_over(mis, n_mis)) != MOE_OK) return fail(rc);
        } else {
            // in stream order: the copies, then one FFN call over the pass
            if ((rc = qrmoe::enqueue_fetch(pool, slots, s.d, s.f, load_e, load_s, n_load, stream)) != MOE_OK)
                return fail(rc);
            if ((rc = ffn_over(order + lo, n_want)) != MOE_OK) return fail(rc);
        }
    }
    if (n_act == 0 && (rc = ffn_over(order, 0, true)) != MOE_OK) return fail(rc);
    if ((rc = moe_combine(shape, y, inv, topk_w, out, stream)) != MOE_OK) return fail(rc);
    if (stats)
        *stats = moe_bank_stats{n_act, hits, misses, passes,
                                static_cast<int64_t>(misses) * static_cast<int64_t>(per_expert)};
    return MOE_OK;
}

}  // extern "C"
