// C ABI of the routed MoE layer: argument validation (entirely on the host,
// before any HIP call), workspace carving and kernel launches.  See
// include/moe.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "kernels.hpp"
#include "validate.hpp"
#include "workspace.hpp"

namespace {

using qrmoe::FfnArgs;

using qrmoe::align256;
using qrmoe::kHeader;
using qrmoe::ffn_ws_bytes;
using qrmoe::LayerCarve;
using qrmoe::layer_carve;
using namespace qrmoe::check;

int hip_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// ---- unchecked bodies (arguments already validated) ----

int do_route(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias, float* logits,
             int32_t* ids, float* w, hipStream_t st) {
    return hip_rc(qrmoe::launch_route(s, x, wr, bias, logits, ids, w, st));
}

int do_dispatch(const moe_shape& s, const int32_t* ids, int32_t* offsets, int32_t* perm, int32_t* inv,
                void* ws, hipStream_t st) {
    return hip_rc(qrmoe::launch_dispatch(s, ids, offsets, perm, inv, static_cast<uint32_t*>(ws), st));
}

// layer: the one-call layer, in which an expert mapped to MOE_SLOT_SKIP
// contributes zero (its y rows are zeroed); moe_expert_ffn leaves them alone.
FfnArgs ffn_args(const moe_shape& s, const uint16_t* x, const moe_experts* ex, const int32_t* offsets,
                 const int32_t* perm, float* y, void* ws, bool layer = false, bool shared = false) {
    FfnArgs a{};
    a.zero_skipped = layer;
    a.T = s.T; a.d = s.d; a.E = s.E; a.k = s.k; a.f = s.f;
    a.x = x;
    a.offsets = offsets;
    a.perm = perm;
    a.slot_of_expert = ex->slot_of_expert;
    a.num_slots = ex->num_slots;
    a.slot_bytes = static_cast<size_t>(ex->slot_bytes);
    const moe_qmat* mats[3] = {&ex->gate, &ex->up, &ex->down};
    for (int i = 0; i < 3; ++i) {
        a.codes[i] = static_cast<const uint8_t*>(mats[i]->codes);
        a.scales[i] = static_cast<const uint8_t*>(mats[i]->scales);
    }
    char* base = static_cast<char*>(ws);
    const qrmoe::FfnCarve c = qrmoe::ffn_carve(s, shared);
    a.act = reinterpret_cast<uint16_t*>(base + c.act);
    a.flags = c.flags ? reinterpret_cast<unsigned long long*>(base + c.flags) : nullptr;
    a.xsum = c.xsum ? reinterpret_cast<uint32_t*>(base + c.xsum) : nullptr;
    a.asum = c.asum ? reinterpret_cast<uint32_t*>(base + c.asum) : nullptr;
    a.y = y;
    a.status = static_cast<uint32_t*>(ws);
    a.header = static_cast<const uint32_t*>(ws);
    return a;
}

int do_ffn(const moe_shape& s, const uint16_t* x, const moe_experts* ex, const int32_t* offsets,
           const int32_t* perm, float* y, void* ws, hipStream_t st, bool layer = false) {
    return hip_rc(qrmoe::launch_ffn(s, ex->gate.fmt, ffn_args(s, x, ex, offsets, perm, y, ws, layer), st));
}

int do_combine(const moe_shape& s, const float* y, const int32_t* inv, const float* w, float* out,
               hipStream_t st) {
    return hip_rc(qrmoe::launch_combine(s, y, inv, w, out, st));
}

// moe_layer's checks (all on the host).  ws may be a stand-in address of
// the right alignment when the workspace is not known yet.
int check_layer(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                const float* logits, const moe_experts* experts, const int32_t* topk_ids, const float* topk_w,
                const float* out, const void* ws, size_t ws_bytes) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    const moe_shape& s = *shape;
    if (!ws || !out) return MOE_ERR_NULL;
    if (!aligned(ws, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
    const LayerCarve c = layer_carve(s);
    if (ws_bytes < c.total) return MOE_ERR_WORKSPACE;
    const char* base = static_cast<const char*>(ws);
    if ((rc = check_route_args(s, x, w_router, bias, logits, topk_ids, topk_w)) != MOE_OK) return rc;
    if (!x) return MOE_ERR_NULL;
    return check_ffn_args(s, x, experts, reinterpret_cast<const int32_t*>(base + c.offsets),
                          reinterpret_cast<const int32_t*>(base + c.perm), reinterpret_cast<const float*>(base + c.y),
                          ws, ws_bytes);
}

// moe_layer's launches on a checked call (T > 0).  status: where the kernels
// raise device status bits -- the workspace header when null, else a word of
// the caller's (the header then holds no poll limit either).
int layer_run(const moe_shape& s, const uint16_t* x, const float* w_router, const float* bias, float* logits,
              const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out, void* ws, uint32_t* status,
              hipStream_t stream) {
    int rc;
    const LayerCarve c = layer_carve(s);
    char* base = static_cast<char*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(base + c.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(base + c.inv);
    float* y = reinterpret_cast<float*>(base + c.y);
    uint32_t* dev_status = status ? status : static_cast<uint32_t*>(ws);
    auto args = [&] {
        FfnArgs a = ffn_args(s, x, experts, offsets, perm, y, ws, true);
        if (status) {
            a.status = status;
            a.header = nullptr;
        }
        return a;
    };
    // Small batches (T <= 8, T*k <= 64): the router launch computes only the
    // logits; every workgroup of the gate/up launch routes the batch itself
    // (top-k and dispatch in LDS) and its workgroup 0 writes the routing
    // outputs; with k <= 2 the combine is a scatter-add inside the down
    // launch.  Same arithmetic as the separate entry points, so the results
    // are identical.
    if (qrmoe::routed_ffn_supported(s, experts->gate.fmt)) {
        if (w_router && (rc = hip_rc(qrmoe::launch_router_logits(s, x, w_router, bias, logits, stream))) != MOE_OK)
            return rc;
        const bool fuse_combine = s.k <= 2;
        FfnArgs a = args();
        a.topk_w = topk_w;
        a.out = fuse_combine ? out : nullptr;
        a.fuse_combine = fuse_combine;
        a.logits = logits;
        a.ids_out = topk_ids;
        a.w_out = topk_w;
        a.offsets_out = offsets;
        a.perm_out = perm;
        a.inv_out = inv;
        if ((rc = hip_rc(qrmoe::launch_ffn_routed(s, experts->gate.fmt, a, stream))) != MOE_OK) return rc;
        return fuse_combine ? MOE_OK : do_combine(s, y, inv, topk_w, out, stream);
    }
    // Other batches: routing (top-k and dispatch in one workgroup for up to
    // 16 tokens), the FFN, and the combine -- on the skinny path with k <= 2
    // a scatter-add inside the down launch (out zeroed by the gate/up launch).
    if (qrmoe::small_route_supported(s)) {
        if ((rc = hip_rc(qrmoe::launch_small_route(s, x, w_router, bias, logits, topk_ids, topk_w, offsets, perm,
                                                   inv, stream))) != MOE_OK)
            return rc;
    } else {
        if ((rc = do_route(s, x, w_router, bias, logits, topk_ids, topk_w, stream)) != MOE_OK) return rc;
        if ((rc = hip_rc(qrmoe::launch_dispatch(s, topk_ids, offsets, perm, inv, dev_status, stream))) != MOE_OK)
            return rc;
    }
    FfnArgs a = args();
    if (s.k <= 2 && !qrmoe::ffn_uses_grouped(s, experts->gate.fmt)) {
        a.topk_w = topk_w;
        a.out = out;
        a.fuse_combine = 1;
        return hip_rc(qrmoe::launch_ffn(s, experts->gate.fmt, a, stream));
    }
    if ((rc = hip_rc(qrmoe::launch_ffn(s, experts->gate.fmt, a, stream))) != MOE_OK) return rc;
    return do_combine(s, y, inv, topk_w, out, stream);
}

// moe_expert_ffn_mx8 / _mx4 (bits = 8 / 4); layer: called by moe_layer_mx8 /
// _mx4 (skipped experts contribute zero).
int ffn_mxq(const moe_shape* shape, const uint16_t* x, const moe_experts* experts, const int32_t* offsets,
            const int32_t* perm, float* y, void* ws, size_t ws_bytes, hipStream_t stream, int bits, bool layer) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    const moe_shape& s = *shape;
    const qrmoe::MxqCarve c = qrmoe::mxq_carve(s, bits);
    if ((rc = check_ffn_args(s, x, experts, offsets, perm, y, ws, ws_bytes, c.total)) != MOE_OK) return rc;
    if (experts->gate.fmt != MOE_FMT_MXFP4 || !qrmoe::grouped_supported(s, MOE_FMT_MXFP4)) return MOE_ERR_UNSUPPORTED;
    char* base = static_cast<char*>(ws);
    FfnArgs a = ffn_args(s, x, experts, offsets, perm, y, ws, layer);
    a.act = nullptr;
    a.flags = reinterpret_cast<unsigned long long*>(base + c.flags);
    a.aq = reinterpret_cast<uint8_t*>(base + c.aq);
    a.as = reinterpret_cast<uint8_t*>(base + c.as);
    a.xq = reinterpret_cast<const uint8_t*>(base + c.xq);
    a.xs = reinterpret_cast<const uint8_t*>(base + c.xs);
    a.rpad = c.rpad;
    return hip_rc(qrmoe::launch_ffn_mxq(s, a, bits, stream));
}

// moe_layer_mx8 / _mx4: route, dispatch, the quantised-activation FFN, combine.
int layer_mxq(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias, float* logits,
              const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
              hipStream_t stream, int bits) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    const moe_shape& s = *shape;
    if (!ws || !out || !x || !experts) return MOE_ERR_NULL;
    if (!aligned(ws, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
    const LayerCarve c = qrmoe::layer_carve_mxq(s, bits);
    if (ws_bytes < c.total) return MOE_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(base + c.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(base + c.inv);
    float* y = reinterpret_cast<float*>(base + c.y);
    if ((rc = check_route_args(s, x, w_router, bias, logits, topk_ids, topk_w)) != MOE_OK) return rc;
    if ((rc = check_ffn_args(s, x, experts, offsets, perm, y, ws, ws_bytes, qrmoe::mxq_carve(s, bits).total)) != MOE_OK)
        return rc;
    if (experts->gate.fmt != MOE_FMT_MXFP4 || !qrmoe::grouped_supported(s, MOE_FMT_MXFP4)) return MOE_ERR_UNSUPPORTED;
    if (qrmoe::small_route_supported(s)) {
        if ((rc = hip_rc(qrmoe::launch_small_route(s, x, w_router, bias, logits, topk_ids, topk_w, offsets, perm,
                                                   inv, stream))) != MOE_OK)
            return rc;
    } else {
        if ((rc = do_route(s, x, w_router, bias, logits, topk_ids, topk_w, stream)) != MOE_OK) return rc;
        if ((rc = do_dispatch(s, topk_ids, offsets, perm, inv, ws, stream)) != MOE_OK) return rc;
    }
    if ((rc = ffn_mxq(shape, x, experts, offsets, perm, y, ws, ws_bytes, stream, bits, true)) != MOE_OK) return rc;
    return do_combine(s, y, inv, topk_w, out, stream);
}

}  // namespace

// ---- moe_layer_noalloc: moe_layer with its workspace in a file-scope
// device array, for callers that cannot allocate.  Every GPU the library
// runs on holds its own copy of `scratch` until the process ends.  In host
// code the array's name is only a stand-in: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and that
// address is what the launches get.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_of_device[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    void* p = g_scratch_of_device[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_of_device[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
            g_scratch_of_device[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return ffn_ws_bytes(*shape);
}

size_t moe_layer_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return layer_carve(*shape).total;
}

size_t moe_qmat_bytes(int32_t fmt, int32_t layout, int32_t slots, int32_t n, int32_t K, size_t* codes_bytes,
                      size_t* scales_bytes, size_t* mins_bytes) {
    size_t c, s, m;
    qmat_sizes(fmt, layout, slots, n, K, &c, &s, &m);
    if (codes_bytes) *codes_bytes = c;
    if (scales_bytes) *scales_bytes = s;
    if (mins_bytes) *mins_bytes = m;
    return c + s + m;
}

int moe_pack_qmat(const moe_qmat* src, const moe_qmat* dst, int32_t slots, int32_t n, int32_t K,
                  hipStream_t stream) {
    if (!src || !dst) return MOE_ERR_NULL;
    if (src->fmt != dst->fmt || src->layout != MOE_LAYOUT_ROWS || dst->layout != MOE_LAYOUT_TILES)
        return MOE_ERR_FORMAT;
    size_t c, s, m;
    if (!qmat_sizes(src->fmt, MOE_LAYOUT_ROWS, slots, n, K, &c, &s, &m)) {
        return src->fmt != MOE_FMT_MXFP4 && src->fmt != MOE_FMT_Q2G32 && src->fmt != MOE_FMT_Q4G32 ? MOE_ERR_FORMAT
                                                                                                : MOE_ERR_SHAPE;
    }
    const bool with_mins = src->fmt == MOE_FMT_Q2G32 || src->fmt == MOE_FMT_Q4G32;
    if (!src->codes || !src->scales || !dst->codes || !dst->scales || (with_mins && !src->mins)) return MOE_ERR_NULL;
    if (dst->mins || (!with_mins && src->mins)) return MOE_ERR_FORMAT;
    if (!aligned(src->codes, 16) || !aligned(dst->codes, 16) || !aligned(src->scales, 4) ||
        !aligned(dst->scales, 4) || (with_mins && !aligned(src->mins, 4)))
        return MOE_ERR_ALIGN;
    return hip_rc(qrmoe::launch_pack(src->fmt, src->codes, src->scales, src->mins, const_cast<void*>(dst->codes),
                                     const_cast<void*>(dst->scales), slots, n, K, stream));
}

int moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!ws) return MOE_ERR_NULL;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGN;
    if (ws_bytes < kHeader) return MOE_ERR_WORKSPACE;
    return hip_rc(qrmoe::launch_clear_header(static_cast<uint32_t*>(ws), stream));
}

int moe_route_topk(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                   float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    rc = check_route_args(*shape, x, w_router, bias, logits, topk_ids, topk_w);
    if (rc != MOE_OK) return rc;
    return do_route(*shape, x, w_router, bias, logits, topk_ids, topk_w, stream);
}

int moe_dispatch(const moe_shape* shape, const int32_t* topk_ids, int32_t* offsets, int32_t* perm,
                 int32_t* inv, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    rc = check_dispatch_args(*shape, topk_ids, offsets, perm, inv, ws, ws_bytes);
    if (rc != MOE_OK) return rc;
    return do_dispatch(*shape, topk_ids, offsets, perm, inv, ws, stream);
}

int moe_expert_ffn(const moe_shape* shape, const uint16_t* x, const moe_experts* experts,
                   const int32_t* offsets, const int32_t* perm, float* y, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    rc = check_ffn_args(*shape, x, experts, offsets, perm, y, ws, ws_bytes);
    if (rc != MOE_OK) return rc;
    return do_ffn(*shape, x, experts, offsets, perm, y, ws, stream);
}

int moe_combine(const moe_shape* shape, const float* y, const int32_t* inv, const float* topk_w,
                float* out, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    rc = check_combine_args(y, inv, topk_w, out);
    if (rc != MOE_OK) return rc;
    return do_combine(*shape, y, inv, topk_w, out, stream);
}

int moe_layer(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
              float* logits, const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out,
              void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_layer(shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, ws, ws_bytes);
    if (rc != MOE_OK || shape->T == 0) return rc;
    return layer_run(*shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, ws, nullptr, stream);
}

int moe_layer_noalloc(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                      float* logits, const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out,
                      uint32_t* status, hipStream_t stream) {
    // every check first, against a stand-in workspace address of the
    // scratch array's alignment and size (no HIP call yet)
    const void* stand_in = reinterpret_cast<const void*>(static_cast<uintptr_t>(256));
    int rc = check_layer(shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, stand_in,
                         MOE_NOALLOC_SCRATCH_BYTES);
    if (rc != MOE_OK || shape->T == 0) return rc;
    if (status && !aligned(status, 4)) return MOE_ERR_ALIGN;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != MOE_OK) return rc;
    // nothing in the scratch array needs to start at zero: every region is
    // written before it is read in a call, and the prefill ready flags hold
    // per-launch values; device status goes to the caller's word (or, with
    // status NULL, to the scratch header, where nobody reads it)
    uint32_t* st = status ? status : static_cast<uint32_t*>(ws);
    return layer_run(*shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, ws, st, stream);
}

size_t moe_layer_shared_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return layer_carve(*shape, true).total;
}

int moe_layer_shared(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias,
                     float* logits, const moe_experts* experts, const moe_experts* shared, int32_t* topk_ids,
                     float* topk_w, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    int rc = check_shape(shape);
    if (rc != MOE_OK) return rc;
    if (shape->T == 0) return MOE_OK;
    const moe_shape& s = *shape;
    if (!ws || !out || !x || !shared || !experts) return MOE_ERR_NULL;
    if (!aligned(ws, 16) || !aligned(out, 16)) return MOE_ERR_ALIGN;
    const LayerCarve c = layer_carve(s, true);
    if (ws_bytes < c.total) return MOE_ERR_WORKSPACE;
    char* base = static_cast<char*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(base + c.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(base + c.inv);
    float* y = reinterpret_cast<float*>(base + c.y);
    if ((rc = check_route_args(s, x, w_router, bias, logits, topk_ids, topk_w)) != MOE_OK) return rc;
    if ((rc = check_ffn_args(s, x, experts, offsets, perm, y, ws, ws_bytes)) != MOE_OK) return rc;
    const int fmt = experts->gate.fmt;
    const moe_qmat* sm[3] = {&shared->gate, &shared->up, &shared->down};
    for (const moe_qmat* m : sm)
        if ((rc = check_qmat(*m, fmt)) != MOE_OK) return rc;
    if (shared->num_slots < 1) return MOE_ERR_SHAPE;
    auto set_shared = [&](FfnArgs& a) {
        a.has_shared = 1;
        for (int i = 0; i < 3; ++i) {
            a.sh_codes[i] = static_cast<const uint8_t*>(sm[i]->codes);
            a.sh_scales[i] = static_cast<const uint8_t*>(sm[i]->scales);
        }
    };
    // Small batches: the gate/up launch routes the batch itself (as in
    // moe_layer) and writes perm[T*k + t] = t*k for the shared expert's rows.
    if (qrmoe::routed_ffn_supported(s, fmt)) {
        if (w_router && (rc = hip_rc(qrmoe::launch_router_logits(s, x, w_router, bias, logits, stream))) != MOE_OK)
            return rc;
        FfnArgs a = ffn_args(s, x, experts, offsets, perm, y, ws, true);
        a.flags = nullptr;
        a.act = reinterpret_cast<uint16_t*>(base + kHeader);
        set_shared(a);
        a.logits = logits;
        a.ids_out = topk_ids;
        a.w_out = topk_w;
        a.offsets_out = offsets;
        a.perm_out = perm;
        a.inv_out = inv;
        if ((rc = hip_rc(qrmoe::launch_ffn_routed(s, fmt, a, stream))) != MOE_OK) return rc;
        return hip_rc(qrmoe::launch_combine(s, y, inv, topk_w, out, stream, true));
    }
    // routing: the dispatch also writes perm[T*k + t] = t*k, the rows of the
    // shared expert
    if (qrmoe::small_route_supported(s)) {
        if ((rc = hip_rc(qrmoe::launch_small_route(s, x, w_router, bias, logits, topk_ids, topk_w, offsets, perm,
                                                   inv, stream, true))) != MOE_OK)
            return rc;
    } else {
        if ((rc = do_route(s, x, w_router, bias, logits, topk_ids, topk_w, stream)) != MOE_OK) return rc;
        if ((rc = hip_rc(qrmoe::launch_dispatch(s, topk_ids, offsets, perm, inv, static_cast<uint32_t*>(ws),
                                                stream, true))) != MOE_OK)
            return rc;
    }
    FfnArgs a = ffn_args(s, x, experts, offsets, perm, y, ws, true, true);
    set_shared(a);
    if ((rc = hip_rc(qrmoe::launch_ffn(s, fmt, a, stream))) != MOE_OK) return rc;
    return hip_rc(qrmoe::launch_combine(s, y, inv, topk_w, out, stream, true));
}

size_t moe_workspace_bytes_mx8(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return qrmoe::mxq_carve(*shape, 8).total;
}

size_t moe_layer_mx8_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return qrmoe::layer_carve_mxq(*shape, 8).total;
}

int moe_expert_ffn_mx8(const moe_shape* shape, const uint16_t* x, const moe_experts* experts, const int32_t* offsets,
                       const int32_t* perm, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
    return ffn_mxq(shape, x, experts, offsets, perm, y, ws, ws_bytes, stream, 8, false);
}

int moe_layer_mx8(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias, float* logits,
                  const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
    return layer_mxq(shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, ws, ws_bytes, stream, 8);
}

size_t moe_workspace_bytes_mx4(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return qrmoe::mxq_carve(*shape, 4).total;
}

size_t moe_layer_mx4_workspace_bytes(const moe_shape* shape) {
    if (check_shape(shape) != MOE_OK) return 0;
    return qrmoe::layer_carve_mxq(*shape, 4).total;
}

int moe_expert_ffn_mx4(const moe_shape* shape, const uint16_t* x, const moe_experts* experts, const int32_t* offsets,
                       const int32_t* perm, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
    return ffn_mxq(shape, x, experts, offsets, perm, y, ws, ws_bytes, stream, 4, false);
}

int moe_layer_mx4(const moe_shape* shape, const uint16_t* x, const float* w_router, const float* bias, float* logits,
                  const moe_experts* experts, int32_t* topk_ids, float* topk_w, float* out, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
    return layer_mxq(shape, x, w_router, bias, logits, experts, topk_ids, topk_w, out, ws, ws_bytes, stream, 4);
}

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: shape outside the supported limits";
        case MOE_ERR_FORMAT: return "MOE_ERR_FORMAT: unknown, mixed or mislaid pack format or layout";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer not aligned as required";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: request not supported";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed";
        case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: a kernel flagged bad device data";
        default: return "unknown moe status";
    }
}

int moe_read_device_status_bits(const void* ws, uint32_t* bits, hipStream_t stream) {
    if (!ws) return MOE_ERR_NULL;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGN;
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, stream) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
    if (bits) *bits = word;
    return word ? MOE_ERR_DEVICE : MOE_OK;
}

int moe_read_device_status(const void* ws, hipStream_t stream) {
    return moe_read_device_status_bits(ws, nullptr, stream);
}

}  // extern "C"
