// Workspace sizes and carving, shared by the entry points of api.cpp and the
// slot-bank layer (bank.hip).  Layout: a 256-byte header (device status
// word), act bf16 [T*k][f], the ready flags of the single-launch prefill FFN;
// moe_layer then carves offsets, perm, inv and y fp32 [T*k][d].
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace qrmoe {

constexpr size_t kHeader = 256;

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

inline size_t act_bytes(const moe_shape& s) { return align256(static_cast<size_t>(s.T) * s.k * s.f * 2); }

inline size_t flag_bytes(const moe_shape& s) { return align256(static_cast<size_t>(grouped_flag_count(s)) * 8); }

inline size_t ffn_ws_bytes(const moe_shape& s) { return kHeader + act_bytes(s) + flag_bytes(s); }

struct LayerCarve {
    size_t offsets, perm, inv, y, total;
};

inline LayerCarve layer_carve(const moe_shape& s) {
    LayerCarve c;
    const size_t pairs = static_cast<size_t>(s.T) * s.k;
    c.offsets = ffn_ws_bytes(s);
    c.perm = c.offsets + align256(static_cast<size_t>(s.E + 1) * 4);
    c.inv = c.perm + align256(pairs * 4);
    c.y = c.inv + align256(pairs * 4);
    c.total = c.y + align256(pairs * s.d * 4);
    return c;
}

}  // namespace qrmoe
