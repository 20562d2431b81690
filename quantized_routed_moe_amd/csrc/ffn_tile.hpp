// Building blocks of the skinny expert-FFN kernels (few token rows per
// expert): one wave computes a 16 (token columns) x 16 (weight rows) output
// tile over a slice of K on the 16x16x32 bf16 matrix cores, with the weights
// dequantised in registers and the token operand read from LDS.  The tokens
// are the MFMA's A operand and the weights its B operand, so lane l receives
// the outputs of weight row l%16 for tokens 4(l/16) .. 4(l/16)+3: every
// per-row quantity (a Q2 group's scale and min) is uniform over a lane's
// four outputs.
//
// Weights are in the tile layout (include/moe.h, MOE_LAYOUT_TILES): for a
// 16-row tile, K step s (128 elements, four 32-element groups) is a block of
// 64 pieces and lane L of the wave loads piece L, so one load instruction
// reads one contiguous block (1 KB of MXFP4 codes, 512 B of Q2 codes) and
// every cache line it touches is consumed whole.
//  * MXFP4: lane (row = L%16, g = L/16) holds group 4s+g of its row (16 code
//    bytes, one scale).  MFMA j of the step takes elements 8j..8j+7 of that
//    group; the token operand supplies the same elements of its row.  The
//    scale bytes of four consecutive steps are 256 contiguous bytes: one
//    dword per lane fetches them all and a lane permute hands each lane its
//    own byte, so a chunk costs one scale load instead of four.
//  * Q2: each MFMA covers ONE group (4s+j), all four lane groups supplying
//    slices of it, because the per-group scale and min must be applied to the
//    group's partial sum.  The tile layout hands lane (row, g) the codes of
//    elements 8g..8g+7 of each of the four groups, even elements and odd
//    elements in separate bytes, so that one shift and one and-or turn a
//    pair of codes into two bf16 values 1 + q/4 (bit pattern 0x3F80 | q<<5,
//    exact).  With C = sum (1+q/4) x and xs = sum x (a second MFMA against a
//    ones operand) the group contributes
//        (4*scale)*C + (min - 4*scale)*xs == sum (scale*q + min) x.
//    The offset 1 keeps the cancellation between C and xs small.  A lane
//    loads the four (scale, min) words of its own row for the step (16
//    contiguous bytes of the row-major scale block).
//  * Q4: as Q2 with 4-bit codes: one word per group, the even elements'
//    nibbles in its low half and the odd ones' in its high half, so one
//    shift and one and-or give bf16(1 + q/16) pairs (0x3F80 | q<<3, exact),
//    and the group contributes (16*scale)*C + (min - 16*scale)*xs.
//
// Token operand: the wave copies the K slice of each real token row of the
// column pass (kCap steps = 512 bf16 = 1 KB per row) straight from global
// memory into its own LDS rows (gfx950 global_load_lds, 16 bytes per lane),
// one instruction per row, and reads the MFMA fragments from there.
// Padding columns read a staged copy of some row and their outputs are never
// stored; MFMA rows and columns do not mix.  Elements past K read a clamped,
// finite address and meet padding weights, which are exactly zero.
#pragma once

#include "common.hpp"

namespace qrmoe {

constexpr int kCap = 4;        // K steps held in registers per chunk
constexpr int kStepK = 128;    // K elements per step of the tile layout
// One staged token row in LDS: kCap steps of bf16 plus 16 bytes, so that the
// rows read by the 16 lanes of one ds_read_b128 phase start in distinct
// 16-byte bank groups (row stride 1040 B = 260 banks = 4 mod 64).
constexpr int kBRowBytes = kCap * kStepK * 2 + 16;

// K steps per register chunk of a format: Q4 holds two (its 16 code bytes
// and 16 scale bytes per step would not fit 128 VGPRs at four); a staged
// token row still spans kCap steps, of which the chunk reads the first.
template <int FMT> constexpr int kCapOf = FMT == MOE_FMT_Q4G32 ? 2 : kCap;

template <int FMT> struct PieceBytes;
template <> struct PieceBytes<MOE_FMT_MXFP4> { static constexpr int codes = 16, scales = 1; };
template <> struct PieceBytes<MOE_FMT_Q2G32> { static constexpr int codes = 8, scales = 4; };
template <> struct PieceBytes<MOE_FMT_Q4G32> { static constexpr int codes = 16, scales = 4; };

template <int FMT> struct WChunk;
template <> struct WChunk<MOE_FMT_MXFP4> {
    u32x4 c[kCap];        // 32 e2m1 codes of group 4s+g
    uint32_t sraw;        // dword `lane` of the chunk's 256 scale bytes
};
template <> struct WChunk<MOE_FMT_Q2G32> {
    u32x2 c[kCap];        // elements 8g..8g+7 of groups 4s..4s+3 (dword t: groups 4s+2t, 4s+2t+1)
    u32x4 sm[kCap];       // fp16 scale | fp16 min << 16 of (row, group 4s+j), j = 0..3
};
template <> struct WChunk<MOE_FMT_Q4G32> {
    u32x4 c[kCapOf<MOE_FMT_Q4G32>];     // elements 8g..8g+7 of groups 4s..4s+3 (dword j: group 4s+j)
    u32x4 sm[kCapOf<MOE_FMT_Q4G32>];    // as Q2
};

// Weight loads per chunk and matrix (code blocks + scale loads).
template <int FMT> constexpr int kWLoads = FMT == MOE_FMT_MXFP4 ? kCap + 1 : 2 * kCapOf<FMT>;

// One 16-row tile of one matrix: this lane's code piece of step 0 and the
// tile's scale block of step 0.
struct WTile {
    const uint8_t* codes;
    const uint8_t* scales;
};

// Tile `tile` of slot `slot` of a matrix of NT tiles and S K steps.  The
// slots of an array lie slot_bytes apart when the pack keeps each expert's
// six arrays in one slab (moe_experts.slot_bytes), else back to back.
template <int FMT>
__device__ __forceinline__ WTile wtile(const uint8_t* codes, const uint8_t* scales, int slot, size_t slot_bytes,
                                       int NT, int tile, int S, int lane) {
    const size_t per_slot = static_cast<size_t>(NT) * S * kWave;     // pieces of one slot
    const size_t cs = slot_bytes ? slot_bytes : per_slot * PieceBytes<FMT>::codes;
    const size_t ss = slot_bytes ? slot_bytes : per_slot * PieceBytes<FMT>::scales;
    const size_t block = static_cast<size_t>(tile) * S * kWave;
    return WTile{codes + slot * cs + (block + lane) * PieceBytes<FMT>::codes,
                 scales + slot * ss + block * PieceBytes<FMT>::scales};
}

// Loads steps [s0, s0 + kCap) of the tile; steps at or past s1 reload step
// s1 - 1 (step 0 when the range is empty), so every load is issued
// unconditionally and the surplus values are simply not used.
template <int FMT>
__device__ __forceinline__ void load_w(WChunk<FMT>& w, const WTile& t, int s0, int s1) {
    const int lane = threadIdx.x & 63;
    if constexpr (FMT == MOE_FMT_MXFP4) {
        // bytes [64 s, 64 s + 64) are the scales of step s; lane L takes the
        // dword holding pieces 4(L%16)..4(L%16)+3 of step s0 + L/16.  Issued
        // first: every step needs it.
        const size_t s = static_cast<size_t>(max(min(s0 + (lane >> 4), s1 - 1), 0));
        w.sraw = *reinterpret_cast<const uint32_t*>(t.scales + s * kWave + 4 * (lane & 15));
    }
#pragma unroll
    for (int u = 0; u < kCapOf<FMT>; ++u) {
        const size_t s = static_cast<size_t>(max(min(s0 + u, s1 - 1), 0));
        if constexpr (FMT == MOE_FMT_MXFP4) {
            w.c[u] = *reinterpret_cast<const u32x4*>(t.codes + s * kWave * 16);
        } else {
            // row-major scale block: the four words of row L%16
            w.sm[u] = *reinterpret_cast<const u32x4*>(t.scales + s * kWave * 4 + 16 * (lane & 15));
            if constexpr (FMT == MOE_FMT_Q4G32) w.c[u] = *reinterpret_cast<const u32x4*>(t.codes + s * kWave * 16);
            else w.c[u] = *reinterpret_cast<const u32x2*>(t.codes + s * kWave * 8);
        }
    }
}

// Scale byte of this lane's piece in step u of the chunk (MXFP4).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t sraw, int u) {
    const int lane = threadIdx.x & 63;
    const uint32_t v = static_cast<uint32_t>(
        __builtin_amdgcn_ds_bpermute((16 * u + (lane >> 2)) << 2, static_cast<int>(sraw)));
    return (v >> (8 * (lane & 3))) & 0xffu;
}

// Copies K elements [e0, e0 + kCap*kStepK) of RB token rows into the wave's
// LDS rows (row c at dst + c * kBRowBytes), one global_load_lds per row.
// Lane i moves elements e0 + 8i .. e0 + 8i + 7, clamped to the last eight
// elements of the row.  `src(c)` is row c's first element; rows past the
// pass's real rows repeat its last one: a fixed number of loads, so every
// wait count after them is known at compile time.
template <int RB, typename Src>
__device__ __forceinline__ void stage_rows(uint8_t* dst, Src src, int e0, int K) {
    const int lane = threadIdx.x & 63;
    const int e = min(e0 + 8 * lane, K - 8);
#pragma unroll
    for (int c = 0; c < RB; ++c)
        __builtin_amdgcn_global_load_lds(src(c) + e, (lds_void*)(dst + c * kBRowBytes), 16, 0, 0);
}

// Independent accumulator chains per matrix: MXFP4 alternates two over the
// MFMAs of a step (their sum is taken at the end), so consecutive dependent
// MFMAs of a wave are two apart; Q2 adds scaled partial sums with VALU
// instructions and keeps one.
template <int FMT> constexpr int kChains = FMT == MOE_FMT_MXFP4 ? 2 : 1;

// acc[.][m] += B(chunk, 16 token columns)^T x W_m(steps [0, nsteps) of the
// chunk, 16 rows), for NM matrices that share the token operand: lane l
// accumulates weight row l%16 for tokens 4(l/16)+i.  `brow` is this lane's
// staged token row (column lane % 16).
template <int FMT, int NM>
__device__ __forceinline__ void mma_chunk(f32x4 (&acc)[kChains<FMT>][NM], const WChunk<FMT> (&w)[NM],
                                          const uint8_t* brow, int nsteps) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
#pragma unroll
    for (int u = 0; u < kCapOf<FMT>; ++u) {
        if (u >= nsteps) break;
        if constexpr (FMT == MOE_FMT_MXFP4) {
            float scl[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) scl[m] = e8m0_to_f32(mx_scale_byte(w[m].sraw, u));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // elements 128u + 32g + 8j .. +7 of the row
                const bf16x8 bb = *reinterpret_cast<const bf16x8*>(brow + 256 * u + 64 * g + 16 * j);
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc[j & 1][m] = mfma16x16x32(bb, mxfp4x8_to_bf16(w[m].c[u][j], scl[m]), acc[j & 1][m]);
            }
        } else {
            // Q2: codes q/4 steps at bits 5-6 of each bf16 half; Q4: q/16 steps at bits 3-6
            constexpr bool q4 = FMT == MOE_FMT_Q4G32;
            constexpr float kStep = q4 ? 16.f : 4.f;      // 1/step of the operand 1 + q/kStep
            const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
            // the code mask in a register: (x & mask) | 0x3f803f80 is then one
            // v_and_or_b32 (gfx950 VOP3 takes no second literal)
            uint32_t qmask = q4 ? 0x00780078u : 0x00600060u;
            asm volatile("" : "+v"(qmask));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // elements 128u + 32j + 8g .. +7 of the row (group 4s+j)
                const bf16x8 bb = *reinterpret_cast<const bf16x8*>(brow + 256 * u + 64 * j + 16 * g);
                const f32x4 xs = mfma16x16x32(bb, ones, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    // Q2: even elements of group j in byte (j&1), odd ones in
                    // byte 2 + (j&1).  Q4: group j is word j, even elements
                    // in its low half, odd ones in its high half.
                    uint32_t cw;
                    if constexpr (q4) cw = w[m].c[u][j];
                    else cw = w[m].c[u][j >> 1];
                    u32x4 av;   // pair h = elements 2h, 2h+1 -> bf16(1 + q/kStep) in the low, high half
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int sh = q4 ? 4 * h - 3 : 8 * (j & 1) + 2 * h - 5;
                        const uint32_t x = sh >= 0 ? cw >> sh : cw << -sh;
                        av[h] = (x & qmask) | 0x3f803f80u;
                    }
                    const f32x4 cq = mfma16x16x32(bb, bf16x8_from_u32x4(av), f32x4{0.f, 0.f, 0.f, 0.f});
                    const uint32_t smw = w[m].sm[u][j];
                    const float fs = kStep * fp16_to_f32(smw);                 // kStep * scale
                    const float fm = fmaf(-kStep, fp16_to_f32(smw), fp16_to_f32(smw >> 16));  // min - kStep * scale
                    f32x4 ac = acc[0][m];
#pragma unroll
                    for (int i = 0; i < 4; ++i) ac[i] = fmaf(fs, cq[i], fmaf(fm, xs[i], ac[i]));
                    acc[0][m] = ac;
                }
            }
        }
    }
}

}  // namespace qrmoe
