// Workspace sizes and carving, shared by the entry points of api.cpp and the
// slot-bank layer (bank.hip).  Layout: a 256-byte header (device status
// word), act bf16 [rows][f], the ready flags of the single-launch prefill FFN;
// moe_layer then carves offsets, perm [rows], inv [T*k] and y fp32 [rows][d];
// rows = T*k, plus T with a shared expert.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace qrmoe {

constexpr size_t kHeader = 256;

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

// Rows of act, y and perm: the T*k routed pairs, plus T rows of the shared
// expert when there is one.
inline size_t ffn_rows(const moe_shape& s, bool shared) {
    return static_cast<size_t>(s.T) * s.k + (shared ? static_cast<size_t>(s.T) : 0);
}

inline size_t act_bytes(const moe_shape& s, bool shared = false) { return align256(ffn_rows(s, shared) * s.f * 2); }

inline size_t flag_bytes(const moe_shape& s, bool shared = false) {
    return align256(static_cast<size_t>(grouped_flag_count(s, shared)) * 8);
}

// Group sums of the 2-bit / 4-bit grouped FFN (FfnArgs::xsum, ::asum): u32
// [T][d/32] and [rows][f/32], after the flags; none where the grouped path
// is never taken.
inline size_t xsum_bytes(const moe_shape& s) {
    return grouped_shape(s) ? align256(static_cast<size_t>(s.T) * (s.d / 32) * 4) : 0;
}
inline size_t asum_bytes(const moe_shape& s, bool shared = false) {
    return grouped_shape(s) ? align256(ffn_rows(s, shared) * (s.f / 32) * 4) : 0;
}

inline size_t ffn_ws_bytes(const moe_shape& s, bool shared = false) {
    return kHeader + act_bytes(s, shared) + flag_bytes(s, shared) + xsum_bytes(s) + asum_bytes(s, shared);
}

// Byte offsets of the FFN workspace's arrays (0: not present).
struct FfnCarve {
    size_t act, flags, xsum, asum;
};

inline FfnCarve ffn_carve(const moe_shape& s, bool shared = false) {
    FfnCarve c;
    c.act = kHeader;
    const size_t fl = c.act + act_bytes(s, shared);
    c.flags = flag_bytes(s, shared) ? fl : 0;
    const size_t xs = fl + flag_bytes(s, shared);
    c.xsum = xsum_bytes(s) ? xs : 0;
    c.asum = asum_bytes(s, shared) ? xs + xsum_bytes(s) : 0;
    return c;
}

struct LayerCarve {
    size_t offsets, perm, inv, y, total;
};

inline LayerCarve layer_carve(const moe_shape& s, bool shared = false) {
    LayerCarve c;
    const size_t pairs = static_cast<size_t>(s.T) * s.k, rows = ffn_rows(s, shared);
    c.offsets = ffn_ws_bytes(s, shared);
    c.perm = c.offsets + align256(static_cast<size_t>(s.E + 1) * 4);
    c.inv = c.perm + align256(rows * 4);
    c.y = c.inv + align256(pairs * 4);
    c.total = c.y + align256(rows * s.d * 4);
    return c;
}

// MXFP8 or MXFP4 activations (moe_expert_ffn_mx8 / _mx4; bits = 8 or 4):
// header, act codes [R][f * bits / 8], act scales [f/32][R + 128], the ready
// flags, token codes [R][d * bits / 8], token scales [d/32][R + 128]
// (R = T*k).
struct MxqCarve {
    size_t aq, as, flags, xq, xs, total;
    int rpad;
};

inline MxqCarve mxq_carve(const moe_shape& s, int bits) {
    MxqCarve c;
    const size_t R = static_cast<size_t>(s.T) * s.k;
    c.rpad = static_cast<int>(R) + 128;
    c.aq = kHeader;
    c.as = c.aq + align256(R * s.f * bits / 8);
    c.flags = c.as + align256(static_cast<size_t>(s.f / 32) * c.rpad);
    c.xq = c.flags + flag_bytes(s);
    c.xs = c.xq + align256(R * s.d * bits / 8);
    c.total = c.xs + align256(static_cast<size_t>(s.d / 32) * c.rpad);
    return c;
}

// moe_layer_mx8 / _mx4: the FFN workspace above, then offsets, perm, inv and y.
inline LayerCarve layer_carve_mxq(const moe_shape& s, int bits) {
    LayerCarve c;
    const size_t pairs = static_cast<size_t>(s.T) * s.k;
    c.offsets = mxq_carve(s, bits).total;
    c.perm = c.offsets + align256(static_cast<size_t>(s.E + 1) * 4);
    c.inv = c.perm + align256(pairs * 4);
    c.y = c.inv + align256(pairs * 4);
    c.total = c.y + align256(pairs * s.d * 4);
    return c;
}

}  // namespace qrmoe
