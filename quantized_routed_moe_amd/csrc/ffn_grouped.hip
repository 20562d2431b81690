// Expert FFN for many token rows per expert (prefill chunks): a grouped GEMM
// over the token-by-expert permutation on the 32x32x16 bf16 matrix cores
// with fp32 accumulation.  This is the block-sparse routed-expert
// computation of "antirez ds4: DeepSeek Metal inference" (section
// 技术深度解析) at prefill sizes: each activated expert's weights are read
// from HBM once per 128-token tile, inactive experts not at all, and the
// quantised weights are dequantised on the fly.
//
// Workgroup = 8 waves; output tile = 128 token rows x 512 weight rows; K step 64.
//  * MODE 0 (gate/up + SwiGLU): weight rows are gate rows [n0, n0+256) then
//    up rows [n0, n0+256); wave w owns gate and up rows [n0+32w, n0+32w+32),
//    so silu(g)*u is formed in registers and act = bf16_rne(.) is stored.
//  * MODE 1 (down): weight rows [m0, m0+512) of W_d; wave w owns rows
//    [m0+64w, m0+64w+64); y is stored in fp32.
// Every wave covers all 128 token rows (four 32-wide MFMA column tiles); the
// K loop is instantiated for the number of column tiles that hold a valid
// row (1..4), so a partial tile costs MFMA work in proportion to its rows and
// the inner loop has no branches.
//
// Operands in LDS, in a ring of stages filled by direct global -> LDS loads
// (gfx950 global_load_lds, 16 bytes per lane: lane i of an instruction lands
// at the instruction's LDS base + 16 i, from an address of its own choice):
//  * weights: the raw MXFP4 pieces of the tile layout (include/moe.h): a
//    64-element step of a 16-row tile is half of one layout block, 32 pieces
//    of 16 code bytes, contiguous in HBM and copied as is; the 32 scale bytes
//    of each of the 32 tiles with them, all in one 1 KB copy by wave 0 (two
//    16-byte lanes per tile: with 1-, 2- or 4-byte lanes the LDS destination
//    advances 4 bytes per lane, so narrower copies would not be contiguous);
//  * tokens: bf16 rows of 128 B (64 elements) whose 16-byte chunks are stored
//    XOR-swizzled by (row / 2) mod 8 -- each lane fetches the global chunk
//    that belongs at its LDS position.  gfx950's LDS serves 256 B per cycle
//    (16 lanes of a ds_read_b128), and the swizzle puts any 16 consecutive
//    rows at one logical chunk in 16 distinct bank groups.
// A wave dequantises its own A fragment (gfx950 scaled fp4 -> bf16
// conversion) right after reading it.  K is permuted inside a step so that in
// sub-step kk lane half h (= lane/32) takes elements 32h + 8kk .. +8: a lane
// then reads one whole 32-element group (one piece: 16 code bytes, one scale)
// of the weight row and 64 contiguous bytes of the token row per step.
//
// Pipeline: a ring of NST stages (4 to 7: a stage holds only the token rows
// of the unit's live column tiles, so units with few rows keep more weight
// bytes in flight); every wave issues its LDS-bound loads of a stage (two
// weight, up to two token, wave 0 the scales too) NST - 2 or NST - 1 stages
// ahead; the stages go in pairs: before a pair it waits (vmcnt, counting its
// own loads, a compile-time count per wave role) until only the younger
// stages are in flight, and one barrier per pair makes every wave's copies
// visible and frees the previous pair's buffers for the copies of the next
// two stages, issued right after the barrier (MX tokens) or after the first
// stage's fragment reads (bf16 tokens).  No register
// ring and no LDS store pass: the registers go to the accumulators and to the
// B fragments, which are all read at the start of a stage so that their LDS
// latency overlaps the multiplies.  Padding token rows (past the expert's
// last row) load a valid row; their output columns are never stored.
//
// Schedule: work units (expert, m-tile, n-tile) are enumerated with the n-tile
// fastest.  Workgroup ids are dealt round-robin over the 8 XCDs, and there
// are 8 n-tiles at the workload's shape; grouped_unit_index gives each XCD
// G = 4 n-tiles of every fourth m-tile position: consecutive m-tiles of a hot expert reuse the same
// weight tiles from that XCD's L2, an m-tile's token rows are fetched by
// 8/G XCDs, and the heavy units of hot experts are spread evenly over all
// XCDs (handing out contiguous ranges of units per XCD instead put a whole
// hot expert on one XCD and was measured ~1.5x slower).  Units are derived
// from offsets on the device.
#include <type_traits>

#include "chain.hpp"
#include "common.hpp"
#include "grouped_sched.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kGN = 512;        // weight rows per tile
constexpr int kGK = 64;         // K per step
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * 64;
constexpr int kStageW = kGN * 32;            // 32 tiles x 32 pieces x 16 B
constexpr int kStageS = kGN * 2;             // 32 tiles x 32 scale bytes
constexpr int kLdsBytes = 153600;            // the stage ring (of 160 KB per CU)
constexpr int kLdsAlloc = kLdsBytes + 16;    // + one word past the ring (the hand-off verdict)

// Stage ring of a unit whose valid token rows fill NTT 32-row column tiles:
// a stage holds the weights, their scales and only the 32*NTT token rows the
// multiplies read, so units with few rows keep more stages (and bytes) in
// flight: 7 stages for NTT = 1, 6, 5 and 4 for NTT = 4.
// XQ = 8 or 4 (MXFP8 or MXFP4 activations): token rows of 64 E4M3 bytes
// or 32 E2M1 bytes, plus their two blocks' scale bytes for all 128 rows
// (256 bytes); XQ = 0: bf16 token rows.
template <int NTT, int XQ = 0> struct Ring {
    static constexpr int x_bytes = 32 * NTT * (XQ == 8 ? 64 : XQ == 4 ? 32 : 128);  // token rows x 64 elements
    static constexpr int stage = kStageW + kStageS + x_bytes + (XQ ? 256 : 0);
    static constexpr int count = kLdsBytes / stage;
    static_assert(count >= 4 && count <= 8, "ring depth");
};

// Waits until at most r (<= R) stages of L loads each are still in flight.
template <int L, int R>
__device__ __forceinline__ void wait_stages(int r) {
    if constexpr (R == 0) {
        wait_vmcnt<0>();
    } else {
        if (r >= R) wait_vmcnt<R * L>();
        else wait_stages<L, R - 1>(r);
    }
}

// Byte offset of 16-byte chunk `chunk` (0..7) of token row `row` (128 B) in
// the token tile (see the swizzle above).
__device__ __forceinline__ int xswz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
// The same for E4M3 token rows (64 B, chunks 0..3): chunk ^ (row / 4) mod 4
// puts 16 consecutive rows at one logical chunk in 16 distinct bank groups.
__device__ __forceinline__ int xswz8(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }
// And for E2M1 token rows (32 B, chunks 0..1): chunk ^ (row / 8) mod 2.
__device__ __forceinline__ int xswz4(int row, int chunk) { return row * 32 + ((chunk ^ ((row >> 3) & 1)) << 4); }

// One work unit (see Schedule above) on the workgroup's LDS ring `lds`.
// CHAIN (both projections in one launch): a gate/up unit stores act with
// device-scope stores and then raises flag `unit`; a down unit first waits
// for the flags of every gate/up unit of its m-tile, then reads act with
// device-scope loads (chain.hpp).
template <int MODE, bool CHAIN, int XQ = 0>
__device__ __forceinline__ void grouped_unit(const FfnArgs& a, int unit, unsigned long long tag, uint8_t* lds) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int NT = MODE == 0 ? a.f / (kGN / 2) : a.d / kGN;
    const int S = K / kGK;

    GroupedUnit gu;
    unit = grouped_unit_index<4>(unit, NT);
    if (!grouped_unit_of<kFullPerPartMx>(a, unit, NT, lane, gu)) return;
    const int e = gu.e, mti = gu.mti, nt = gu.nt, r_base = gu.r_base, nvalid = gu.nvalid, slot = gu.slot;
    const bool sh = gu.sh;
    // element-wise selects: choosing between the two pointer arrays would
    // put the kernel argument block in scratch memory
    auto wcodes = [&](int mat) { return sh ? a.sh_codes[mat] : a.codes[mat]; };
    auto wscales = [&](int mat) { return sh ? a.sh_scales[mat] : a.scales[mat]; };
    // y rows [r_base, r_base + nvalid) x this unit's weight rows, all set to v
    auto fill_y = [&](float v) {
        for (int i = tid; i < nvalid * kGN; i += kGThreads)
            a.y[static_cast<size_t>(r_base + i / kGN) * a.d + nt * kGN + i % kGN] = v;
    };
    if (!sh && (slot < 0 || slot >= a.num_slots)) {
        // MOE_SLOT_SKIP: left out of this call -- its y rows are untouched
        // (the slot bank fills y over several calls), or zero when the
        // one-call layer runs (a skipped expert then contributes nothing)
        const bool skip = slot == MOE_SLOT_SKIP;
        if (!skip && tid == 0 && nt == 0 && mti == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1 && (!skip || a.zero_skipped)) fill_y(0.f);
        if (CHAIN && MODE == 0) raise_flag(a.flags + unit, tag);   // its act is never read
        return;
    }
    if constexpr (CHAIN && MODE == 1) {
        // units are numbered m-tile-major in both projections, so the gate/up
        // units of this m-tile are flags [m-tile * NT0, + NT0).  A wait that
        // gives up leaves act unknown: the unit then writes NaN into its y
        // rows instead of a product of stale act rows, and raises
        // MOE_DEV_CHAIN_TIMEOUT.
        // the verdict goes through a word past the stage ring of the
        // workgroup's one LDS array: a __shared__ variable of its own made
        // the compiler wait for every global -> LDS copy in flight (vmcnt(0))
        // before each stage's LDS reads, which it cannot tell apart from it
        int* chain_ok = reinterpret_cast<int*>(lds + kLdsBytes);
        const int NT0 = a.f / (kGN / 2);
        if (wave == 0) {
            const bool ok =
                wait_flags(a.flags + static_cast<size_t>(unit / NT) * NT0, NT0, tag, chain_poll_limit(a.header));
            if (lane == 0) {
                *chain_ok = ok;
                if (!ok) raise_status(a.status, MOE_DEV_CHAIN_TIMEOUT);
            }
        }
        __syncthreads();
        if (!*chain_ok) {
            fill_y(__builtin_nanf(""));
            return;
        }
    }

    // ---- load roles of this lane (per stage: 2 weight and 2 token
    // instructions per wave, and one scale instruction by wave 0)
    auto tile_base = [&](int tt, int& mat) {     // layout block of workgroup tile tt (0..31) within its slot
        mat = 2;
        int tile = nt * (kGN / 16) + tt;
        if (MODE == 0) {
            mat = tt < kGN / 32 ? 0 : 1;
            tile = nt * (kGN / 32) + (tt & (kGN / 32 - 1));
        }
        return static_cast<size_t>(tile) * (K / 128);
    };
    // first byte of the slot in the codes and scales arrays: slabs of
    // slot_bytes (moe_experts.slot_bytes), else the arrays' own slot sizes
    const size_t slot_blocks = static_cast<size_t>(N / 16) * (K / 128);
    const size_t slot_c = static_cast<size_t>(slot) * (a.slot_bytes ? a.slot_bytes : slot_blocks * 64 * 16);
    const size_t slot_s = static_cast<size_t>(slot) * (a.slot_bytes ? a.slot_bytes : slot_blocks * 64);
    const uint8_t* wsrc[2];      // piece (lane & 31) of tile 4w + 2i + (lane >> 5), step 0
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int mat;
        const size_t blk = tile_base(4 * wave + 2 * i + (lane >> 5), mat);
        wsrc[i] = wcodes(mat) + slot_c + blk * 64 * 16 + (lane & 31) * 16;
    }
    const uint8_t* ssrc;         // wave 0: scale bytes 16 (lane & 1) .. +16 of tile lane >> 1
    {
        int mat;
        const size_t blk = tile_base(lane >> 1, mat);
        ssrc = wscales(mat) + slot_s + blk * 64 + 16 * (lane & 1);
    }
    const uint16_t* xsrc[2];     // token row 16w + 8i + (lane >> 3), global chunk for LDS chunk lane & 7
    const uint8_t* qsrc = nullptr;   // XQ = 8: E4M3 token row 16w + (lane >> 2), global chunk for LDS chunk lane & 3;
                                     // XQ = 4: E2M1 token row 32w + (lane >> 1), global chunk for LDS chunk lane & 1
    const uint8_t* qssrc = nullptr;  // XQ, wave 1, lanes 0..15: scale bytes of rows r_base + 16 (lane & 7) .. +16, block lane >> 3
    if constexpr (XQ == 8) {
        const int row = 16 * wave + (lane >> 2);
        const int rr = r_base + (row < nvalid ? row : 0);
        qsrc = (MODE == 0 ? a.xq + static_cast<size_t>(rr) * a.d : a.aq + static_cast<size_t>(rr) * a.f) +
               (((lane & 3) ^ ((row >> 2) & 3)) << 4);
        qssrc = (MODE == 0 ? a.xs : a.as) + static_cast<size_t>(lane >> 3 & 1) * a.rpad + r_base + 16 * (lane & 7);
    } else if constexpr (XQ == 4) {
        const int row = 32 * wave + (lane >> 1);
        const int rr = r_base + (row < nvalid ? row : 0);
        qsrc = (MODE == 0 ? a.xq + static_cast<size_t>(rr) * (a.d / 2) : a.aq + static_cast<size_t>(rr) * (a.f / 2)) +
               (((lane & 1) ^ ((row >> 3) & 1)) << 4);
        qssrc = (MODE == 0 ? a.xs : a.as) + static_cast<size_t>(lane >> 3 & 1) * a.rpad + r_base + 16 * (lane & 7);
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = 16 * wave + 8 * i + (lane >> 3);
            const int rr = r_base + (row < nvalid ? row : 0);
            const uint16_t* rowp = MODE == 0 ? a.x + static_cast<size_t>(a.perm[rr] / a.k) * a.d
                                             : a.act + static_cast<size_t>(rr) * a.f;
            xsrc[i] = rowp + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
        }
    }
    // Token rows at or past 32 * (live column tiles) are never read: the waves
    // that own them (rows 16w .. 16w+15) copy no token rows at all.
    const int ntt = __builtin_amdgcn_readfirstlane(ceil_div(nvalid, 32));
    const bool x_live = XQ == 4 ? wave < ntt : 16 * wave < 32 * ntt;   // E2M1: a wave copies 32 rows
    // stage s of a ring of NST stages of SB bytes -> LDS buffer s % NST
    auto issue = [&](int s, auto nst_c, auto sb_c) {
        constexpr int NST = decltype(nst_c)::value, SB = decltype(sb_c)::value;
        uint8_t* base = lds + (s % NST) * SB;
        const size_t half = static_cast<size_t>(s >> 1) * 1024 + (s & 1) * 512;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_global_load_lds(wsrc[i] + half, (lds_void*)(base + (4 * wave + 2 * i) * 512), 16, 0, 0);
        if (wave == 0)     // all 32 tiles' scale bytes of the stage: one 1 KB copy
            __builtin_amdgcn_global_load_lds(ssrc + (s >> 1) * 64 + (s & 1) * 32,
                                             (lds_void*)(base + kStageW), 16, 0, 0);
        if constexpr (XQ) {
            constexpr int XB = SB - kStageW - kStageS - 256;        // token rows of the stage
            if (x_live)         // 1 KB: 16 E4M3 rows or 32 E2M1 rows
                __builtin_amdgcn_global_load_lds(qsrc + s * (kGK * XQ / 8), (lds_void*)(base + kStageW + kStageS + 1024 * wave),
                                                 16, 0, CHAIN && MODE == 1 ? kAuxDevice : 0);
            if (wave == 1 && lane < 16)   // both K blocks' scale bytes of all 128 rows
                __builtin_amdgcn_global_load_lds(qssrc + static_cast<size_t>(2 * s) * a.rpad,
                                                 (lds_void*)(base + kStageW + kStageS + XB), 16, 0,
                                                 CHAIN && MODE == 1 ? kAuxDevice : 0);
        } else if (x_live) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                __builtin_amdgcn_global_load_lds(xsrc[i] + s * kGK,
                                                 (lds_void*)(base + kStageW + kStageS + (16 * wave + 8 * i) * 128), 16, 0,
                                                 CHAIN && MODE == 1 ? kAuxDevice : 0);
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;
    const int rt0 = MODE == 0 ? 32 * wave : 64 * wave;
    const int rt1 = MODE == 0 ? kGN / 2 + 32 * wave : 64 * wave + 32;
    const int r32 = lane & 31, h = lane >> 5;
    // LDS piece index of weight row rt + r32, local group h
    const int pc0 = (rt0 / 16 + (r32 >> 4)) * 32 + 16 * h + (r32 & 15);
    const int pc1 = (rt1 / 16 + (r32 >> 4)) * 32 + 16 * h + (r32 & 15);

    auto kloop = [&](auto ntt_c) {
        constexpr int NTT = decltype(ntt_c)::value;
        constexpr int NST = Ring<NTT, XQ>::count, SB = Ring<NTT, XQ>::stage;
        const auto nst_c = std::integral_constant<int, NST>{};
        const auto sb_c = std::integral_constant<int, SB>{};
        for (int s = 0; s < NST - 2 && s < S; ++s) issue(s, nst_c, sb_c);
        auto stage = [&](int s, auto l_c, auto m_c) {
            constexpr int L = decltype(l_c)::value;
            // One barrier per pair of stages: M = 1 is the pair's first stage,
            // M = 2 its second.  The pair's wait leaves NST - 4 stages in
            // flight (each wave counts its own loads, L per stage: its role's
            // count, see run below); after the barrier every wave's copies of
            // both stages are visible and every wave is done with the
            // previous pair, whose buffers stages s + NST - 2 and s + NST - 1
            // take: MX tokens issue their copies right after the barrier,
            // bf16 tokens after the first stage's fragment reads.  Against
            // one barrier per stage: bf16 FFN call -1.3 to -1.5 % (two
            // boxes), MXFP8 -1.7 %, MXFP4 -2.6 % (alternating runs).
            constexpr int M = decltype(m_c)::value;
            if constexpr (M == 1) {
                const int younger = min(S - 1, s + NST - 3) - min(s + 1, S - 1);
                if (younger == NST - 4) wait_vmcnt<L * (NST - 4)>();
                else wait_stages<L, NST - 4>(younger);
                __builtin_amdgcn_s_barrier();
                if constexpr (XQ != 0) {
                    if (s + NST - 2 < S) issue(s + NST - 2, nst_c, sb_c);
                    if (s + NST - 1 < S) issue(s + NST - 1, nst_c, sb_c);
                }
            }
            const uint8_t* wb = lds + (s % NST) * SB;
            const uint8_t* sb = wb + kStageW;
            const uint8_t* xb = sb + kStageS;
            // weight operand first, then the token fragments and the
            // weight conversions one sub-step ahead of the multiplies that
            // use them (the scheduling barriers keep the compiler from
            // sinking each read next to its use, which exposed the full LDS
            // latency on every MFMA pair)
            const u32x4 c0 = *reinterpret_cast<const u32x4*>(wb + pc0 * 16);
            const u32x4 c1 = *reinterpret_cast<const u32x4*>(wb + pc1 * 16);
            const uint32_t sc0 = sb[pc0], sc1 = sb[pc1];
            if constexpr (XQ == 4) {
                // fp4 x fp4: the token fragment is chunk h (K block h) of
                // the E2M1 row, with that block's scale byte
                const uint8_t* xsb = xb + 32 * NTT * 32;
                u32x4 b[NTT];
                int bs[NTT];
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    b[t] = *reinterpret_cast<const u32x4*>(xb + xswz4(32 * t + r32, h));
                    bs[t] = xsb[128 * h + 32 * t + r32];
                }
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    acc[0][t] = mfma_scale_fp4_fp4(c0, b[t], acc[0][t], static_cast<int>(sc0), bs[t]);
                    acc[1][t] = mfma_scale_fp4_fp4(c1, b[t], acc[1][t], static_cast<int>(sc1), bs[t]);
                }
                return;
            } else if constexpr (XQ == 8) {
                // one block-scaled 32x32x64 product per (weight tile, column
                // tile): the pieces and their E8M0 bytes go in as they are,
                // the token fragment is chunks h and 2 + h of the E4M3 row
                const uint8_t* xsb = xb + 32 * NTT * 64;
                i32x8 b[NTT];
                int bs[NTT];
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    const u32x4 lo = *reinterpret_cast<const u32x4*>(xb + xswz8(32 * t + r32, h));
                    const u32x4 hi = *reinterpret_cast<const u32x4*>(xb + xswz8(32 * t + r32, 2 + h));
                    b[t] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                                 static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                                 static_cast<int>(hi[2]), static_cast<int>(hi[3])};
                    bs[t] = xsb[128 * h + 32 * t + r32];
                }
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    acc[0][t] = mfma_scale_fp4_fp8(c0, b[t], acc[0][t], static_cast<int>(sc0), bs[t]);
                    acc[1][t] = mfma_scale_fp4_fp8(c1, b[t], acc[1][t], static_cast<int>(sc1), bs[t]);
                }
                return;
            }
            u32x4 bcur[NTT], bnext[NTT];
#pragma unroll
            for (int t = 0; t < NTT; ++t) bcur[t] = *reinterpret_cast<const u32x4*>(xb + xswz(32 * t + r32, 4 * h));
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (M == 1) {
                if (s + NST - 2 < S) issue(s + NST - 2, nst_c, sb_c);
                if (s + NST - 1 < S) issue(s + NST - 1, nst_c, sb_c);
            }
            __builtin_amdgcn_sched_barrier(0);
            const float s0 = e8m0_to_f32(sc0);
            const float s1 = e8m0_to_f32(sc1);
            bf16x8 a0 = mxfp4x8_to_bf16(c0[0], s0);
            bf16x8 a1 = mxfp4x8_to_bf16(c1[0], s1);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                __builtin_amdgcn_sched_barrier(0);
                if (kk < 3) {
#pragma unroll
                    for (int t = 0; t < NTT; ++t)
                        bnext[t] = *reinterpret_cast<const u32x4*>(xb + xswz(32 * t + r32, 4 * h + kk + 1));
                }
                bf16x8 n0 = a0, n1 = a1;
                if (kk < 3) {
                    n0 = mxfp4x8_to_bf16(c0[kk + 1], s0);
                    n1 = mxfp4x8_to_bf16(c1[kk + 1], s1);
                }
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    const bf16x8 b = bf16x8_from_u32x4(bcur[t]);
                    acc[0][t] = mfma32x32x16(a0, b, acc[0][t]);
                    acc[1][t] = mfma32x32x16(a1, b, acc[1][t]);
                }
                // sub-step kk + 1's conversions and token reads placed between
                // sub-step kk's products (one conversion, and while any remain
                // one token read, after each product), so a wave keeps
                // issuing them while its own products run on the matrix core
                if (kk < 3) {
#pragma unroll
                    for (int q = 0; q < 2 * NTT; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        if (q < 8) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
                        if (q < NTT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                a0 = n0;
                a1 = n1;
#pragma unroll
                for (int t = 0; t < NTT; ++t) bcur[t] = bnext[t];
            }
        };
        // The loads per stage of this wave's role are a compile-time count,
        // so the steady-state wait is one instruction and not a tree of
        // scalar branches every stage.  bf16: wave 0 copies the scale bytes
        // (+1), waves holding live token rows copy two rows of 1 KB (+2).
        // MXFP8: waves 0 and 1 always hold live rows (one copy), wave 1 the
        // token scale bytes too.  MXFP4: wave 0 always holds live rows, wave 1
        // copies the token scale bytes.
        auto run = [&](auto l_c) {
            for (int s = 0; s < S; s += 2) {
                stage(s, l_c, std::integral_constant<int, 1>{});
                if (s + 1 < S) stage(s + 1, l_c, std::integral_constant<int, 2>{});
            }
        };
        if constexpr (XQ == 0) {
            if (wave == 0) {
                if (x_live) run(std::integral_constant<int, 5>{});
                else run(std::integral_constant<int, 3>{});
            } else {
                if (x_live) run(std::integral_constant<int, 4>{});
                else run(std::integral_constant<int, 2>{});
            }
        } else if constexpr (XQ == 8) {
            if (wave <= 1) run(std::integral_constant<int, 4>{});
            else if (x_live) run(std::integral_constant<int, 3>{});
            else run(std::integral_constant<int, 2>{});
        } else {
            if (wave == 0 || (wave == 1 && x_live)) run(std::integral_constant<int, 4>{});
            else if (wave == 1 || x_live) run(std::integral_constant<int, 3>{});
            else run(std::integral_constant<int, 2>{});
        }
    };

    switch (ntt) {
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        default: kloop(std::integral_constant<int, 4>{}); break;
    }

    // ---- epilogue.  Lane l holds, for element i, weight row
    // 8*(i/4) + 4*(l/32) + i%4 of the 32-row tile and token row l%32.
    if constexpr (XQ == 4 && MODE == 0) {
        // act to MXFP4: a wave's 32 gate rows of one token are one block of
        // 32 act columns, 16 values in lane l and 16 in lane l ^ 32; the
        // block's 16 code bytes are written as two 8-byte halves, lane l
        // (h = 0) the first, lane l ^ 32 the second, after one exchange
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t >= ntt) continue;
            float v[16];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[i] = silu_mul(acc[0][t][i], acc[1][t][i]);
                amax = fmaxf(amax, fabsf(v[i]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int sbyte = mx4_scale_byte(amax);
            // columns 8q + 4h .. +3 of the block: nibbles of bytes 4q + 2h, 4q + 2h + 1
            uint32_t half[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sh = 127 - sbyte;
                half[q] = e2m1_rne_sat(ldexpf(v[4 * q], sh)) | (e2m1_rne_sat(ldexpf(v[4 * q + 1], sh)) << 4) |
                          (e2m1_rne_sat(ldexpf(v[4 * q + 2], sh)) << 8) | (e2m1_rne_sat(ldexpf(v[4 * q + 3], sh)) << 12);
            }
            const uint32_t send = h ? (half[0] | (half[1] << 16)) : (half[2] | (half[3] << 16));
            const uint32_t recv = static_cast<uint32_t>(__shfl_xor(static_cast<int>(send), 32));
            const int j = 32 * t + r32;
            if (j >= nvalid) continue;
            const uint32_t w0 = h ? ((recv & 0xFFFFu) | (half[2] << 16)) : (half[0] | (recv << 16));
            const uint32_t w1 = h ? ((recv >> 16) | (half[3] << 16)) : (half[1] | (recv & 0xFFFF0000u));
            const size_t r = static_cast<size_t>(r_base + j);
            unsigned long long* dst = reinterpret_cast<unsigned long long*>(
                a.aq + r * (a.f / 2) + (nt * (kGN / 2) + 32 * wave) / 2 + 8 * h);
            const unsigned long long word = static_cast<unsigned long long>(w0) | (static_cast<unsigned long long>(w1) << 32);
            if constexpr (CHAIN) __hip_atomic_store(dst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = word;
            if (h == 0) {
                uint8_t* ds = a.as + static_cast<size_t>(nt * (kGN / 64) + wave) * a.rpad + r;
                if constexpr (CHAIN) __hip_atomic_store(ds, static_cast<uint8_t>(sbyte), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else *ds = static_cast<uint8_t>(sbyte);
            }
        }
        if constexpr (CHAIN) raise_flag(a.flags + unit, tag);
        return;
    }
    if constexpr (XQ == 8 && MODE == 0) {
        // act to MXFP8: a wave's 32 gate rows of one token are one block of
        // 32 act columns, 16 values in lane l and 16 in lane l ^ 32
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t >= ntt) continue;
            float v[16];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                v[i] = silu_mul(acc[0][t][i], acc[1][t][i]);
                amax = fmaxf(amax, fabsf(v[i]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            const int j = 32 * t + r32;
            if (j >= nvalid) continue;
            const int sbyte = mx8_scale_byte(amax);
            const size_t r = static_cast<size_t>(r_base + j);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int sh = 127 - sbyte;
                const uint32_t word = e4m3x4_rne_sat(ldexpf(v[4 * q], sh), ldexpf(v[4 * q + 1], sh),
                                                     ldexpf(v[4 * q + 2], sh), ldexpf(v[4 * q + 3], sh));
                uint32_t* dst = reinterpret_cast<uint32_t*>(a.aq + r * a.f + nt * (kGN / 2) + 32 * wave + 8 * q + 4 * h);
                if constexpr (CHAIN) __hip_atomic_store(dst, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else *dst = word;
            }
            if (h == 0) {
                uint8_t* ds = a.as + static_cast<size_t>(nt * (kGN / 64) + wave) * a.rpad + r;
                if constexpr (CHAIN) __hip_atomic_store(ds, static_cast<uint8_t>(sbyte), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else *ds = static_cast<uint8_t>(sbyte);
            }
        }
        if constexpr (CHAIN) raise_flag(a.flags + unit, tag);
        return;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int j = 32 * t + r32;
        if (t >= ntt || j >= nvalid) continue;
        const size_t r = static_cast<size_t>(r_base + j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = 8 * q + 4 * h;              // first of 4 consecutive rows
            if constexpr (MODE == 0) {
                uint32_t pk[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint16_t lo = f32_to_bf16_rne(silu_mul(acc[0][t][4 * q + 2 * hh], acc[1][t][4 * q + 2 * hh]));
                    const uint16_t hi = f32_to_bf16_rne(silu_mul(acc[0][t][4 * q + 2 * hh + 1], acc[1][t][4 * q + 2 * hh + 1]));
                    pk[hh] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
                }
                const int n = nt * (kGN / 2) + 32 * wave + nl;
                if constexpr (CHAIN) {
                    __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.act + r * a.f + n),
                                       static_cast<unsigned long long>(pk[0]) | (static_cast<unsigned long long>(pk[1]) << 32),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    *reinterpret_cast<u32x2*>(a.act + r * a.f + n) = u32x2{pk[0], pk[1]};
                }
            } else {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int mrow = nt * kGN + 64 * wave + 32 * m + nl;
                    *reinterpret_cast<float4*>(a.y + r * a.d + mrow) =
                        make_float4(acc[m][t][4 * q], acc[m][t][4 * q + 1], acc[m][t][4 * q + 2], acc[m][t][4 * q + 3]);
                }
            }
        }
    }
    if constexpr (CHAIN && MODE == 0) raise_flag(a.flags + unit, tag);
}

template <int MODE>
__global__ __launch_bounds__(kGThreads) void ffn_grouped_kernel(FfnArgs a) {
    __shared__ __align__(16) uint8_t lds[kLdsAlloc];
    grouped_unit<MODE, false>(a, blockIdx.x, 0, lds);
}

__global__ void zero_tail_rows_kernel(FfnArgs a) { zero_tail_rows(a, blockIdx.x, gridDim.x); }

// Both projections in one launch: workgroups [0, ub0) are the gate/up units,
// [ub0, ub0 + ub1) the down units (each waits for its m-tile's gate/up
// units, chain.hpp), the last one zeroes the y rows past offsets[E].  The
// down units thus fill the CUs that the gate/up launch's last, uneven units
// leave idle, instead of waiting for all of them behind a kernel boundary.
template <int XQ>
__global__ __launch_bounds__(kGThreads) void ffn_grouped_chained_kernel(FfnArgs a, int ub0, int ub1) {
    __shared__ __align__(16) uint8_t lds[kLdsAlloc];
    const unsigned long long tag = chain_tag();
    const int b = blockIdx.x;
    if (b < ub0) grouped_unit<0, true, XQ>(a, b, tag, lds);
    else if (b < ub0 + ub1) grouped_unit<1, true, XQ>(a, b - ub0, tag, lds);
    else zero_tail_rows(a, 0, 1);
}

bool grouped_supported(const moe_shape& s, int fmt) {
    return (fmt == MOE_FMT_MXFP4 || fmt == MOE_FMT_Q2G32 || fmt == MOE_FMT_Q4G32) && s.f % (kGN / 2) == 0 &&
           s.d % kGN == 0;
}

static int max_mtiles(const moe_shape& s, bool shared) {
    const int pairs = s.T * s.k;
    const int m = ceil_div(pairs, kGM) + (s.E < pairs ? s.E : pairs) + (shared ? ceil_div(s.T, kGM) : 0);
    return (m + kPosBlockMax - 1) / kPosBlockMax * kPosBlockMax;   // whole blocks of grouped_unit_index
}

int grouped_flag_count(const moe_shape& s, bool shared) {
    return s.f % (kGN / 2) == 0 ? max_mtiles(s, shared) * (s.f / (kGN / 2)) : 0;
}

hipError_t launch_ffn_grouped(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    const int units0 = max_mtiles(s, a.has_shared) * (s.f / (kGN / 2));
    const int units1 = max_mtiles(s, a.has_shared) * (s.d / kGN);
    if (a.flags) {
        ffn_grouped_chained_kernel<0><<<units0 + units1 + 1, kGThreads, 0, st>>>(a, units0, units1);
        return hipGetLastError();
    }
    ffn_grouped_kernel<0><<<units0, kGThreads, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_grouped_kernel<1><<<units1, kGThreads, 0, st>>>(a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    zero_tail_rows_kernel<<<64, 256, 0, st>>>(a);
    return hipGetLastError();
}

// MXFP8 (BITS = 8) or MXFP4 (BITS = 4) token rows in sorted-row order: row
// r is token perm[r] / k; one thread per block of 32 elements (E8M0 scale
// of the block maximum; E4M3 elements rounded to nearest even and
// saturated at 448, or E2M1 elements rounded to nearest even and clamped
// at 6, two per byte, the even element in the low nibble).  xs is
// block-major, [d/32][rpad], so an m-tile's scale bytes of one block are
// contiguous.  256 threads per workgroup.
template <int BITS>
__global__ __launch_bounds__(256) void mxq_gather_quant_kernel(const uint16_t* __restrict__ x,
                                                             const int32_t* __restrict__ perm, int k, int d, int R,
                                                             int rpad, uint8_t* __restrict__ xq,
                                                             uint8_t* __restrict__ xs) {
    // a workgroup takes 16 rows x 16 blocks, lane i row i % 16 and block
    // i / 16: the 16 lanes of one block write its 16 scale bytes (block-major
    // xs) as one contiguous run, and a wave still reads and writes whole
    // 128-byte runs of each of its 16 rows
    const int nb = d / 32, nbt = (nb + 15) / 16;
    const int r = static_cast<int>(blockIdx.x / nbt) * 16 + static_cast<int>(threadIdx.x & 15);
    const int b = static_cast<int>(blockIdx.x % nbt) * 16 + static_cast<int>(threadIdx.x >> 4);
    if (r >= R || b >= nb) return;
    const int t = perm[r] / k;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * d + 32 * b);
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 w = src[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
            v[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
    if constexpr (BITS == 8) {
        const int sbyte = mx8_scale_byte(amax);
        u32x4 out[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int sh = 127 - sbyte;
                const float* vv = v + 16 * c + 4 * e;
                out[c][e] = e4m3x4_rne_sat(ldexpf(vv[0], sh), ldexpf(vv[1], sh), ldexpf(vv[2], sh), ldexpf(vv[3], sh));
            }
        u32x4* dst = reinterpret_cast<u32x4*>(xq + static_cast<size_t>(r) * d + 32 * b);
        dst[0] = out[0];
        dst[1] = out[1];
        xs[static_cast<size_t>(b) * rpad + r] = static_cast<uint8_t>(sbyte);
    } else {
        const int sbyte = mx4_scale_byte(amax);
        const int sh = 127 - sbyte;
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t w = 0;
#pragma unroll
            for (int n = 0; n < 8; ++n) w |= e2m1_rne_sat(ldexpf(v[8 * e + n], sh)) << (4 * n);
            out[e] = w;
        }
        *reinterpret_cast<u32x4*>(xq + static_cast<size_t>(r) * (d / 2) + 16 * b) = out;
        xs[static_cast<size_t>(b) * rpad + r] = static_cast<uint8_t>(sbyte);
    }
}

hipError_t launch_ffn_mxq(const moe_shape& s, const FfnArgs& a, int bits, hipStream_t st) {
    const int R = s.T * s.k;
    const unsigned grid = static_cast<unsigned>(ceil_div(R, 16)) * static_cast<unsigned>(ceil_div(s.d / 32, 16));
    uint8_t* xq = const_cast<uint8_t*>(a.xq);
    uint8_t* xs = const_cast<uint8_t*>(a.xs);
    if (bits == 8) mxq_gather_quant_kernel<8><<<grid, 256, 0, st>>>(a.x, a.perm, s.k, s.d, R, a.rpad, xq, xs);
    else mxq_gather_quant_kernel<4><<<grid, 256, 0, st>>>(a.x, a.perm, s.k, s.d, R, a.rpad, xq, xs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int units0 = max_mtiles(s, false) * (s.f / (kGN / 2));
    const int units1 = max_mtiles(s, false) * (s.d / kGN);
    if (bits == 8) ffn_grouped_chained_kernel<8><<<units0 + units1 + 1, kGThreads, 0, st>>>(a, units0, units1);
    else ffn_grouped_chained_kernel<4><<<units0 + units1 + 1, kGThreads, 0, st>>>(a, units0, units1);
    return hipGetLastError();
}

}  // namespace qrmoe
