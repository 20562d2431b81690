// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace qrmoe {

// Everything the expert-FFN kernels read, resolved on the host.
struct FfnArgs {
    int T, d, E, k, f;
    const uint16_t* x;            // bf16 [T][d]
    const int32_t* offsets;       // [E+1]
    const int32_t* perm;          // [T*k]
    const int32_t* slot_of_expert;  // [E] or null
    int num_slots;
    size_t slot_bytes;            // moe_experts.slot_bytes: 0, or the stride of every array's slots (slabs)
    const uint8_t* codes[3];      // gate, up, down: tile layout (MOE_LAYOUT_TILES)
    const uint8_t* scales[3];     // MXFP4: e8m0 byte per piece; Q2: fp16 scale | fp16 min << 16
    uint16_t* act;                // bf16 [T*k][f] (workspace)
    float* y;                     // fp32 [T*k][d]
    uint32_t* status;             // device status word (the workspace header's, or the caller's)
    const uint32_t* header;       // workspace header (poll-limit word), or null: defaults
    // The one-call layer: an expert mapped to MOE_SLOT_SKIP contributes zero
    // (its y rows are zeroed).  Off for moe_expert_ffn, whose callers (the
    // slot bank) fill y over several calls.
    int zero_skipped;
    // moe_layer with k <= 2 on the skinny path only: the gate/up launch
    // zeroes out and the down projection scatter-adds w[p] * y[r] into it
    // instead of writing y, replacing the combine kernel
    const float* topk_w;          // [T*k]
    float* out;                   // [T][d]
    int fuse_combine;
    // moe_layer with T <= 8 and T*k <= 64 only: the gate/up launch routes the
    // batch itself from the logits [T][E] (every workgroup, in LDS); its
    // workgroup 0 writes the routing outputs (same buffers as offsets/perm).
    const float* logits;
    int32_t* ids_out;
    float* w_out;
    int32_t* offsets_out;
    int32_t* perm_out;
    int32_t* inv_out;
    // Ready flags of the single-launch grouped FFN (workspace), one per
    // gate/up unit (grouped_flag_count); null: two launches.
    unsigned long long* flags;
    // Shared expert (moe_layer_shared): one more item whose rows are the T
    // rows after the routed ones, [T*k, T*k + T) in act and y (row T*k + t is
    // token t: the dispatch writes perm[T*k + t] = t*k), with its own pack
    // (one slot) -- computed in the same launches as the routed experts.
    int has_shared;
    const uint8_t* sh_codes[3];
    const uint8_t* sh_scales[3];
    // MXFP8 activations (grouped path, MXFP4 weights): token rows quantised
    // and gathered in sorted-row order, xq u8 [T*k][d] with scale bytes
    // xs [d/32][rpad]; the SwiGLU output aq u8 [T*k][f] with as [f/32][rpad]
    // (rpad = T*k + 128: a padded m-tile reads whole 128-row scale runs).
    const uint8_t* xq;
    const uint8_t* xs;
    uint8_t* aq;
    uint8_t* as;
    int rpad;
    // 2-bit / 4-bit packs on the grouped path: per 32-element group, the sum
    // of a row's input values as two fp16 halves (hi | lo << 16, hi + lo =
    // the fp32 sum to 22 bits): xsum [T][d/32] of the token rows (written by
    // a pass before the FFN launch), asum [rows][f/32] of the act rows
    // (written by the gate/up tiles; workspace).
    uint32_t* xsum;
    uint32_t* asum;
};

hipError_t launch_route(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                        float* logits, int32_t* ids, float* w, hipStream_t st);
// shared: also perm[T*k + t] = t*k for t < T (the shared expert's rows).
hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, int32_t* offsets, int32_t* perm,
                           int32_t* inv, uint32_t* status, hipStream_t st, bool shared = false);
hipError_t launch_ffn(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st);
bool grouped_supported(const moe_shape& s, int fmt);
bool ffn_uses_grouped(const moe_shape& s, int fmt);
// Router logits only (no top-k), by the per-expert row kernel (small T).
hipError_t launch_router_logits(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                                float* logits, hipStream_t st);
// Router logits + top-k + dispatch of a small batch, the last two in one
// workgroup (T <= 16, T*k <= 64).
bool small_route_supported(const moe_shape& s);
hipError_t launch_small_route(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                              float* logits, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                              int32_t* inv, hipStream_t st, bool shared = false);
// moe_layer for small batches: the skinny FFN whose gate/up launch routes the
// batch from a.logits (see FfnArgs).
bool routed_ffn_supported(const moe_shape& s, int fmt);
hipError_t launch_ffn_routed(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st);
hipError_t launch_ffn_grouped(const moe_shape& s, const FfnArgs& a, hipStream_t st);
// The grouped FFN for the 2-bit and 4-bit packs (ffn_grouped_q.hip): the
// token rows' group sums into a.xsum, then one launch of both projections.
hipError_t launch_ffn_grouped_q(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st);
// Shapes that take the grouped path at all (any format): T*k rows enough
// for it and d, f multiples of its tiles.  The workspace then also holds the
// group sums of the 2-bit / 4-bit path.
bool grouped_shape(const moe_shape& s);
// MXFP8 activations: gather + quantise the token rows into a.xq / a.xs, then
// the single-launch grouped FFN on the block-scaled fp4 x fp8 (bits = 8) or
// fp4 x fp4 (bits = 4) matrix cores.
hipError_t launch_ffn_mxq(const moe_shape& s, const FfnArgs& a, int bits, hipStream_t st);
// Ready flags the grouped FFN needs in the workspace (0: none).
int grouped_flag_count(const moe_shape& s, bool shared = false);
// shared: out[t] also adds y[T*k + t] (weight 1) after the routed terms.
hipError_t launch_combine(const moe_shape& s, const float* y, const int32_t* inv, const float* w,
                          float* out, hipStream_t st, bool shared = false);
hipError_t launch_clear_header(uint32_t* header, hipStream_t st);
hipError_t launch_pack(int fmt, const void* src_codes, const void* src_scales, const void* src_mins, void* dst_codes,
                       void* dst_scales, int slots, int n, int K, hipStream_t st);

}  // namespace qrmoe
