// Host-side argument validation shared by the entry points (api.cpp) and
// the slot bank (bank.hip).  Every check runs before any HIP call, so a
// rejected call enqueues nothing.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"
#include "workspace.hpp"

namespace qrmoe {
namespace check {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline int check_shape(const moe_shape* s) {
    if (!s) return MOE_ERR_NULL;
    if (s->T < 0 || s->k < 1 || s->E < 1 || s->E > 64 || s->k > s->E) return MOE_ERR_SHAPE;
    if (s->d < 32 || s->f < 32 || s->d % 32 || s->f % 32) return MOE_ERR_SHAPE;
    const long long rows = static_cast<long long>(s->T) * s->k;
    const long long wide = s->d > s->f ? s->d : s->f;
    if (rows * wide >= (1ll << 31)) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Array sizes of one (fmt, layout) matrix; false when the request is invalid.
inline bool qmat_sizes(int fmt, int layout, int slots, int n, int K, size_t* codes, size_t* scales,
                       size_t* mins) {
    *codes = *scales = *mins = 0;
    if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_Q2G32 && fmt != MOE_FMT_Q4G32) return false;
    if (layout != MOE_LAYOUT_ROWS && layout != MOE_LAYOUT_TILES) return false;
    if (slots < 1 || n < 16 || n % 16 || K < 32 || K % 32) return false;
    const size_t rows = static_cast<size_t>(slots) * n;
    const size_t groups = rows * (K / 32);
    if (layout == MOE_LAYOUT_ROWS) {
        *codes = fmt == MOE_FMT_Q2G32 ? rows * (K / 4) : rows * (K / 2);
        *scales = fmt == MOE_FMT_MXFP4 ? groups : groups * 2;
        *mins = fmt == MOE_FMT_MXFP4 ? 0 : groups * 2;
    } else {
        const size_t pieces = static_cast<size_t>(slots) * (n / 16) * ((K + 127) / 128) * 64;
        *codes = pieces * (fmt == MOE_FMT_Q2G32 ? 8 : 16);
        *scales = pieces * (fmt == MOE_FMT_MXFP4 ? 1 : 4);
    }
    return true;
}

// A matrix the expert FFN can read: tile layout, every pointer 16-byte aligned.
inline int check_qmat(const moe_qmat& m, int fmt) {
    if (m.fmt != fmt || m.layout != MOE_LAYOUT_TILES) return MOE_ERR_FORMAT;
    if (!m.codes || !m.scales) return MOE_ERR_NULL;
    if (m.mins) return MOE_ERR_FORMAT;
    if (!aligned(m.codes, 16) || !aligned(m.scales, 16)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

inline int check_experts(const moe_shape& s, const moe_experts* ex) {
    if (!ex) return MOE_ERR_NULL;
    const int fmt = ex->gate.fmt;
    if (fmt != MOE_FMT_MXFP4 && fmt != MOE_FMT_Q2G32 && fmt != MOE_FMT_Q4G32) return MOE_ERR_FORMAT;
    int rc;
    if ((rc = check_qmat(ex->gate, fmt)) != MOE_OK) return rc;
    if ((rc = check_qmat(ex->up, fmt)) != MOE_OK) return rc;
    if ((rc = check_qmat(ex->down, fmt)) != MOE_OK) return rc;
    if (ex->num_slots < 1) return MOE_ERR_SHAPE;
    if (!ex->slot_of_expert && ex->num_slots < s.E) return MOE_ERR_SHAPE;
    if (ex->slot_of_expert && !aligned(ex->slot_of_expert, 4)) return MOE_ERR_ALIGN;
    if (ex->slot_bytes % 256) return MOE_ERR_ALIGN;
    return MOE_OK;
}

inline int check_route_args(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                            const float* logits, const int32_t* ids, const float* w) {
    if (!logits || !ids || !w) return MOE_ERR_NULL;
    if (wr && !x) return MOE_ERR_NULL;
    if (!wr && bias) return MOE_ERR_UNSUPPORTED;
    if ((x && !aligned(x, 16)) || (wr && !aligned(wr, 16)) || !aligned(logits, 16)) return MOE_ERR_ALIGN;
    if ((bias && !aligned(bias, 4)) || !aligned(ids, 4) || !aligned(w, 4)) return MOE_ERR_ALIGN;
    (void)s;
    return MOE_OK;
}

inline int check_dispatch_args(const moe_shape& s, const int32_t* ids, const int32_t* offsets,
                               const int32_t* perm, const int32_t* inv, const void* ws, size_t ws_bytes) {
    if (!ids || !offsets || !perm || !inv || !ws) return MOE_ERR_NULL;
    if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv, 4) || !aligned(ws, 16))
        return MOE_ERR_ALIGN;
    if (ws_bytes < kHeader) return MOE_ERR_WORKSPACE;
    (void)s;
    return MOE_OK;
}

// need: the FFN workspace the call uses (the bf16 FFN's by default; the
// quantised-activation calls pass their own, smaller for MXFP4)
inline int check_ffn_args(const moe_shape& s, const uint16_t* x, const moe_experts* ex, const int32_t* offsets,
                          const int32_t* perm, const float* y, const void* ws, size_t ws_bytes, size_t need = 0) {
    if (!x || !offsets || !perm || !y || !ws) return MOE_ERR_NULL;
    int rc = check_experts(s, ex);
    if (rc != MOE_OK) return rc;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(ws, 16)) return MOE_ERR_ALIGN;
    if (!aligned(offsets, 4) || !aligned(perm, 4)) return MOE_ERR_ALIGN;
    if (ws_bytes < (need ? need : ffn_ws_bytes(s))) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

inline int check_combine_args(const float* y, const int32_t* inv, const float* w, const float* out) {
    if (!y || !inv || !w || !out) return MOE_ERR_NULL;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(inv, 4) || !aligned(w, 4)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace check
}  // namespace qrmoe
