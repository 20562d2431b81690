// Building blocks of the skinny expert-FFN kernels (few token rows per
// expert): one wave computes a 16 (weight rows) x 16 (token columns) output
// tile over a slice of K on the 16x16x32 bf16 matrix cores, with the weights
// dequantised in registers.
//
// Weights are in the tile layout (include/moe.h, MOE_LAYOUT_TILES): for a
// 16-row tile, K step s (128 elements, four 32-element groups) is a block of
// 64 pieces and lane L of the wave loads piece L, so one load instruction
// reads one contiguous block (1 KB of MXFP4 codes, 512 B of Q2 codes) and
// every cache line it touches is consumed whole.
//  * MXFP4: lane (row = L%16, g = L/16) holds group 4s+g of its row (16 code
//    bytes, one scale).  MFMA j of the step takes elements 8j..8j+7 of that
//    group; the token operand supplies the same elements of its row.
//  * Q2: each MFMA covers ONE group (4s+j), all four lane groups supplying
//    slices of it, because the per-group scale and min must be applied to the
//    group's partial sum.  The tile layout already hands lane (row, g) the
//    codes of elements 8g..8g+7 of each of the four groups.  A = bf16(1 + q/4)
//    is exact (bit pattern 0x3F80 | q<<5); with C = sum (1+q/4) x and
//    xs = sum x (a second MFMA against a ones operand) the group contributes
//        (4*scale)*C + (min - 4*scale)*xs == sum (scale*q + min) x.
//    The offset 1 keeps the cancellation between C and xs small.  The
//    per-(row, group) scale pairs pass through a wave-private LDS area so that
//    each lane finds the four rows its accumulator holds.
#pragma once

#include "common.hpp"

namespace qrmoe {

constexpr int kCap = 4;        // K steps held in registers per chunk
constexpr int kStepK = 128;    // K elements per step of the tile layout

template <int FMT> struct PieceBytes;
template <> struct PieceBytes<MOE_FMT_MXFP4> { static constexpr int codes = 16, scales = 1; };
template <> struct PieceBytes<MOE_FMT_Q2G32> { static constexpr int codes = 8, scales = 4; };

template <int FMT> struct WChunk;
template <> struct WChunk<MOE_FMT_MXFP4> {
    u32x4 c[kCap];        // 32 e2m1 codes of group 4s+g
    uint32_t s[kCap];     // its e8m0 scale byte
};
template <> struct WChunk<MOE_FMT_Q2G32> {
    u32x2 c[kCap];        // elements 8g..8g+7 of groups 4s..4s+3, 2 bytes each
    uint32_t sm[kCap];    // fp16 scale | fp16 min << 16 of (row, group 4s+g)
};

// This lane's piece of step 0 of one 16-row tile of one matrix.
struct WTile {
    const uint8_t* codes;
    const uint8_t* scales;
};

// tile_index = slot * (n/16) + tile; S = K steps of the matrix.
template <int FMT>
__device__ __forceinline__ WTile wtile(const uint8_t* codes, const uint8_t* scales, size_t tile_index, int S,
                                       int lane) {
    const size_t piece = tile_index * S * kWave + lane;
    return WTile{codes + piece * PieceBytes<FMT>::codes, scales + piece * PieceBytes<FMT>::scales};
}

// Loads steps [s0, s0 + kCap) of the tile; steps at or past s1 reload step
// s1 - 1 (step 0 when the range is empty), so every load is issued
// unconditionally and the surplus values are simply not used.
template <int FMT>
__device__ __forceinline__ void load_w(WChunk<FMT>& w, const WTile& t, int s0, int s1) {
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        const size_t s = static_cast<size_t>(max(min(s0 + u, s1 - 1), 0));
        if constexpr (FMT == MOE_FMT_MXFP4) {
            w.c[u] = *reinterpret_cast<const u32x4*>(t.codes + s * kWave * 16);
            w.s[u] = t.scales[s * kWave];
        } else {
            w.c[u] = *reinterpret_cast<const u32x2*>(t.codes + s * kWave * 8);
            w.sm[u] = *reinterpret_cast<const uint32_t*>(t.scales + s * kWave * 4);
        }
    }
}

// Token operand (bf16) of steps [s0, s0 + kCap) for this lane's column:
// brow is a readable row of K elements (a valid row even when the column is
// padding); elements of padding columns and of groups past G read as zero.
template <int FMT>
__device__ __forceinline__ void load_b(u32x4 (&b)[kCap][4], const uint16_t* brow, bool colok, int s0, int G, int g) {
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        const int s = s0 + u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gi = FMT == MOE_FMT_MXFP4 ? 4 * s + g : 4 * s + j;
            const int e0 = FMT == MOE_FMT_MXFP4 ? 8 * j : 8 * g;
            const bool ok = colok && gi < G;
            const u32x4 v = *reinterpret_cast<const u32x4*>(brow + min(gi, G - 1) * kGroup + e0);
            b[u][j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Wave-private LDS area for the Q2 scale pairs of one 16-row tile step.
struct Q2Lds {
    float2 sm[4][16];     // [group in step][row]: (4*scale, min - 4*scale)
};

// acc[m] += W_m(16 rows, steps [0, nsteps) of the chunk) x B(chunk, 16
// columns), for NM matrices that share the token operand.
template <int FMT, int NM>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[NM], const WChunk<FMT> (&w)[NM],
                                          const u32x4 (&b)[kCap][4], int nsteps, Q2Lds* q2 /* [NM], Q2 only */) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        if (u >= nsteps) break;
        if constexpr (FMT == MOE_FMT_MXFP4) {
            float scl[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) scl[m] = e8m0_to_f32(w[m].s[u] & 0xffu);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 bb = bf16x8_from_u32x4(b[u][j]);
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc[m] = mfma16x16x32(mxfp4x8_to_bf16(w[m].c[u][j], scl[m]), bb, acc[m]);
            }
        } else {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const float sf = fp16_to_f32(w[m].sm[u]);
                const float mf = fp16_to_f32(w[m].sm[u] >> 16);
                q2[m].sm[g][row] = make_float2(4.f * sf, fmaf(-4.f, sf, mf));
            }
            __builtin_amdgcn_wave_barrier();
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 bb = bf16x8_from_u32x4(b[u][j]);
                const f32x4 xs = mfma16x16x32(ones, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    const uint32_t c16 = ((j & 2) ? w[m].c[u][1] : w[m].c[u][0]) >> (16 * (j & 1));
                    u32x4 av;   // eight 2-bit codes -> eight bf16(1 + q/4), two per dword
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t c4 = c16 >> (4 * h);
                        av[h] = ((c4 & 3u) << 5) | ((c4 & 0xcu) << 19) | 0x3f803f80u;
                    }
                    const f32x4 cq = mfma16x16x32(bf16x8_from_u32x4(av), bb, f32x4{0.f, 0.f, 0.f, 0.f});
                    const float4* smp = reinterpret_cast<const float4*>(&q2[m].sm[j][4 * g]);
                    const float4 s01 = smp[0], s23 = smp[1];
                    f32x4 ac = acc[m];
                    ac[0] = fmaf(s01.x, cq[0], fmaf(s01.y, xs[0], ac[0]));
                    ac[1] = fmaf(s01.z, cq[1], fmaf(s01.w, xs[1], ac[1]));
                    ac[2] = fmaf(s23.x, cq[2], fmaf(s23.y, xs[2], ac[2]));
                    ac[3] = fmaf(s23.z, cq[3], fmaf(s23.w, xs[3], ac[3]));
                    acc[m] = ac;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

}  // namespace qrmoe
