// Building blocks of the skinny expert-FFN kernels (few token rows per
// expert): one wave computes a 16 (weight rows) x 16 (token rows) output tile
// over a slice of K on the 16x16x32 bf16 matrix cores, with the weights
// dequantised in registers.
//
// K is walked in "steps" of four 32-element groups.  In step s:
//  * MXFP4: lane group g (= lane/16) loads the 16 code bytes of group 4s+g of
//    its weight row (lane%16); MFMA j of the step takes elements 8j..8j+7 of
//    that group, and the token operand supplies the same elements of x.
//  * Q2: each MFMA covers ONE group (4s+j), all four lane groups supplying
//    slices of it, because the per-group scale and min must be applied to the
//    group's partial sum.  A = bf16(1 + q/4) is exact (bit pattern
//    0x3F80 | q<<5); with C = sum (1+q/4) x and xs = sum x (a second MFMA
//    against a ones operand) the group contributes
//        (4*scale)*C + (min - 4*scale)*xs == sum (scale*q + min) x.
//    The offset 1 keeps the cancellation between C and xs small.  Code bytes
//    and per-row (scale, min) are re-laid through a wave-private LDS area so
//    that each lane finds the slice and rows it needs.
#pragma once

#include "common.hpp"

namespace qrmoe {

constexpr int kCap = 4;   // steps held in registers per chunk

template <int FMT> struct WChunk;
template <> struct WChunk<MOE_FMT_MXFP4> {
    u32x4 c[kCap];        // 32 e2m1 codes of group 4s+g
    uint32_t s[kCap];     // its e8m0 scale byte
};
template <> struct WChunk<MOE_FMT_Q2G32> {
    u32x2 c[kCap];        // 32 2-bit codes of group 4s+g
    uint32_t sm[kCap];    // fp16 scale (low half) | fp16 min (high half)
};

// Per-lane row pointers into one matrix pack for weight row n of slot `slot`.
struct WRow {
    const uint8_t* codes;
    const uint8_t* scales;
    const uint16_t* mins;
};

template <int FMT>
__device__ __forceinline__ WRow wrow(const uint8_t* codes, const uint8_t* scales, const uint16_t* mins,
                                     size_t row, int K) {
    const int G = K / kGroup;
    WRow r;
    if constexpr (FMT == MOE_FMT_MXFP4) {
        r.codes = codes + row * (K / 2);
        r.scales = scales + row * G;
        r.mins = nullptr;
    } else {
        r.codes = codes + row * (K / 4);
        r.scales = scales + row * G * 2;
        r.mins = mins + row * G;
    }
    return r;
}

// Loads steps [s0, s0 + kCap) (clipped to s1 and to G groups) of one row.
template <int FMT>
__device__ __forceinline__ void load_w(WChunk<FMT>& w, const WRow& r, int s0, int s1, int G, int g) {
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        const int s = s0 + u;
        const int gl = 4 * s + g;
        const bool ok = s < s1 && gl < G;
        if constexpr (FMT == MOE_FMT_MXFP4) {
            w.c[u] = ok ? *reinterpret_cast<const u32x4*>(r.codes + gl * 16) : u32x4{0u, 0u, 0u, 0u};
            w.s[u] = ok ? r.scales[gl] : 127u;
        } else {
            w.c[u] = ok ? *reinterpret_cast<const u32x2*>(r.codes + gl * 8) : u32x2{0u, 0u};
            const uint32_t sv = ok ? reinterpret_cast<const uint16_t*>(r.scales)[gl] : 0u;
            const uint32_t mv = ok ? r.mins[gl] : 0u;
            w.sm[u] = sv | (mv << 16);
        }
    }
}

// Token operand (bf16) of steps [s0, s0 + kCap) for this lane's token row.
template <int FMT>
__device__ __forceinline__ void load_b(u32x4 (&b)[kCap][4], const uint16_t* brow, bool colok, int s0, int s1,
                                       int G, int g) {
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        const int s = s0 + u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (FMT == MOE_FMT_MXFP4) {
                const int gi = 4 * s + g;
                const bool ok = colok && s < s1 && gi < G;
                b[u][j] = ok ? reinterpret_cast<const u32x4*>(brow + gi * kGroup)[j] : u32x4{0u, 0u, 0u, 0u};
            } else {
                const int gj = 4 * s + j;
                const bool ok = colok && s < s1 && gj < G;
                b[u][j] = ok ? *reinterpret_cast<const u32x4*>(brow + gj * kGroup + 8 * g) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
}

// Wave-private LDS area for the Q2 re-layout of one 16-row tile.
struct Q2Lds {
    u32x2 codes[16][4];   // [row][group in step]
    float2 sm[4][16];     // [group in step][row]: (4*scale, min - 4*scale)
};

// acc[m] += W_m(16 rows, chunk) x B(chunk, 16 tokens), for NM matrices that
// share the token operand.
template <int FMT, int NM>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[NM], const WChunk<FMT> (&w)[NM],
                                          const u32x4 (&b)[kCap][4], Q2Lds* q2 /* [NM], Q2 only */) {
    const int lane = threadIdx.x & 63;
    const int row = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < kCap; ++u) {
        if constexpr (FMT == MOE_FMT_MXFP4) {
            float scl[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) scl[m] = e8m0_to_f32(w[m].s[u]);
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
                q2[m].codes[row][g] = w[m].c[u];
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
                    const u32x2 cw = q2[m].codes[row][j];
                    const uint32_t c16 = ((g & 2) ? cw[1] : cw[0]) >> (16 * (g & 1));
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
