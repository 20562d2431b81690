// Re-layout of quantised expert matrices from rows (n x K per slot) into the
// tile layout the expert-FFN kernels stream: 16-row tiles x 128-element K
// steps, each (tile, step) block a contiguous array of 64 pieces in the order
// the lanes of a wave consume them (include/moe.h, enum moe_layout).  A pure
// gather: every code, scale and min is copied bit for bit.  Runs once when
// the weights are loaded.
#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

// Scale word L of the (tile, step) block of a Q2 or Q4 matrix: the block's
// words are row-major, word L = (row L/4, group 4s + L%4), fp16 scale in the
// low half and fp16 min in the high half (0 past the last group).
__device__ __forceinline__ uint32_t q_scale_word(const uint8_t* src_scales, const uint16_t* src_mins, size_t slot,
                                                 int n, int G, int NT, size_t ti, int s, int L) {
    const int srow = static_cast<int>(ti % NT) * 16 + (L >> 2), sg = 4 * s + (L & 3);
    if (sg >= G) return 0u;
    const size_t srow_g = slot * n + srow;
    const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(src_scales);
    return static_cast<uint32_t>(sc16[srow_g * G + sg]) | (static_cast<uint32_t>(src_mins[srow_g * G + sg]) << 16);
}

// One thread per piece.  pieces = slots * (n/16) * S * 64, S = ceil(K/128).
template <int FMT>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src_codes,
                                                   const uint8_t* __restrict__ src_scales,
                                                   const uint16_t* __restrict__ src_mins,
                                                   uint8_t* __restrict__ dst_codes, uint8_t* __restrict__ dst_scales,
                                                   int n, int K, size_t pieces) {
    const int G = K / kGroup;
    const int S = ceil_div(K, 128);
    const int NT = n / 16;
    for (size_t p = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; p < pieces;
         p += static_cast<size_t>(gridDim.x) * blockDim.x) {
        const int L = static_cast<int>(p & 63);
        const size_t blk = p >> 6;                       // (slot * NT + tile) * S + step
        const int s = static_cast<int>(blk % S);
        const size_t ti = blk / S;                       // slot * NT + tile
        const size_t slot = ti / NT;
        const int row = static_cast<int>(ti % NT) * 16 + (L & 15);
        const int g = L >> 4;
        const size_t grow = slot * n + row;
        const int gi = 4 * s + g;                        // group of this piece's scale
        if constexpr (FMT == MOE_FMT_MXFP4) {
            u32x4 c = {0u, 0u, 0u, 0u};
            uint8_t sc = 127;
            if (gi < G) {
                c = *reinterpret_cast<const u32x4*>(src_codes + grow * (K / 2) + static_cast<size_t>(gi) * 16);
                sc = src_scales[grow * G + gi];
            }
            *reinterpret_cast<u32x4*>(dst_codes + p * 16) = c;
            dst_scales[p] = sc;
        } else if constexpr (FMT == MOE_FMT_Q4G32) {
            // elements 8g..8g+7 of each of the step's four groups (bytes 4g
            // .. 4g+3 of the group's sixteen): word j holds group 4s+j, the
            // even elements' nibbles in its low half, the odd ones' in its
            // high half
            u32x4 c = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gj = 4 * s + j;
                const uint32_t b4 = gj < G ? *reinterpret_cast<const uint32_t*>(src_codes + grow * (K / 2) +
                                                                              static_cast<size_t>(gj) * 16 + 4 * g)
                                           : 0u;
                uint32_t w = 0u;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const uint32_t b = (b4 >> (8 * h)) & 0xffu;
                    w |= (b & 0xfu) << (4 * h);
                    w |= (b >> 4) << (16 + 4 * h);
                }
                c[j] = w;
            }
            *reinterpret_cast<u32x4*>(dst_codes + p * 16) = c;
            reinterpret_cast<uint32_t*>(dst_scales)[p] = q_scale_word(src_scales, src_mins, slot, n, G, NT, ti, s, L);
        } else {
            // elements 8g..8g+7 of each of the step's four groups (bytes 2g,
            // 2g+1 of the group's eight), even and odd elements apart
            const uint16_t* row16 = reinterpret_cast<const uint16_t*>(src_codes + grow * (K / 4));
            uint32_t ev[4], od[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int gj = 4 * s + j;
                const uint32_t h = gj < G ? row16[gj * 4 + g] : 0u;   // element 8g+e at bits 2e
                ev[j] = od[j] = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ev[j] |= ((h >> (4 * i)) & 3u) << (2 * i);
                    od[j] |= ((h >> (4 * i + 2)) & 3u) << (2 * i);
                }
            }
            *reinterpret_cast<u32x2*>(dst_codes + p * 8) =
                u32x2{ev[0] | (ev[1] << 8) | (od[0] << 16) | (od[1] << 24),
                      ev[2] | (ev[3] << 8) | (od[2] << 16) | (od[3] << 24)};
            reinterpret_cast<uint32_t*>(dst_scales)[p] = q_scale_word(src_scales, src_mins, slot, n, G, NT, ti, s, L);
        }
    }
}

hipError_t launch_pack(int fmt, const void* src_codes, const void* src_scales, const void* src_mins, void* dst_codes,
                       void* dst_scales, int slots, int n, int K, hipStream_t st) {
    const size_t pieces = static_cast<size_t>(slots) * (n / 16) * ceil_div(K, 128) * 64;
    const size_t want = (pieces + 255) / 256;
    const int blocks = static_cast<int>(want < 65536 ? want : 65536);
    const auto* sc = static_cast<const uint8_t*>(src_codes);
    const auto* ss = static_cast<const uint8_t*>(src_scales);
    const auto* sm = static_cast<const uint16_t*>(src_mins);
    auto* dc = static_cast<uint8_t*>(dst_codes);
    auto* ds = static_cast<uint8_t*>(dst_scales);
    if (fmt == MOE_FMT_MXFP4) pack_kernel<MOE_FMT_MXFP4><<<blocks, 256, 0, st>>>(sc, ss, sm, dc, ds, n, K, pieces);
    else if (fmt == MOE_FMT_Q2G32) pack_kernel<MOE_FMT_Q2G32><<<blocks, 256, 0, st>>>(sc, ss, sm, dc, ds, n, K, pieces);
    else pack_kernel<MOE_FMT_Q4G32><<<blocks, 256, 0, st>>>(sc, ss, sm, dc, ds, n, K, pieces);
    return hipGetLastError();
}

}  // namespace qrmoe
