// Work units of the single-launch grouped expert FFN (prefill chunks): which
// expert, 128-row m-tile and n-tile a workgroup computes.  Shared by the
// MXFP4 kernel (ffn_grouped.hip) and the 2-bit / 4-bit kernel
// (ffn_grouped_q.hip), so that both deal the work out the same way.
//
// Full 128-row m-tiles (expert-major; matrix-core bound) and partial m-tiles
// (at most one per expert, by decreasing row count, ties to the lower expert
// id; bound by streaming their weight tile; increasing order measured 6 %
// slower for MXFP4 and 17 % for the 2-bit pack) are dealt in groups of
// kFullPerPart (a template argument) full m-tiles and one partial while both
// kinds remain, then the
// rest in the same orders, n-tile fastest within an m-tile.  So HBM
// streaming overlaps the matrix-core work from the start, and the smallest
// partial m-tiles fill the end of the launch.  A shared expert's m-tiles
// (rows [T*k, T*k + T)) come first.  Units are derived from offsets on the
// device; every lane of the calling wave gets the same answer.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kGM = 128;        // token rows per m-tile
// Dispatch order: kFullPerPart full m-tiles per partial m-tile while both
// remain.  At the prefill workload (24 full, 44 partial m-tiles), measured per
// FFN call with the XCD mapping below: the MXFP4 launch is fastest at 2 (1
// is 8-18 % slower, 3 and 4 are 1-4 % slower, for bf16, MXFP8 and MXFP4
// tokens alike); the 2-bit and 4-bit launch, whose full m-tiles take longer,
// at 4 or more (2: +9-10 %, 3: +7 %; 4, 8 and all full m-tiles first within
// 0.5 % of each other).
constexpr int kFullPerPartMx = 2;
constexpr int kFullPerPartQ = 4;

struct GroupedUnit {
    int e;          // expert (E: the shared expert)
    int mti;        // m-tile of the expert
    int nt;         // n-tile
    int r_base;     // first sorted row of the m-tile
    int nvalid;     // its rows (1..128)
    int slot;       // the expert's slot (slot_of_expert), unchecked
    bool sh;        // the shared expert
};

// Unit `unit` of a projection with NT n-tiles; false past the last unit.
template <int kFullPerPart>
__device__ __forceinline__ bool grouped_unit_of(const FfnArgs& a, int unit, int NT, int lane, GroupedUnit& u) {
    int cnt = 0;
    if (lane < a.E) cnt = a.offsets[lane + 1] - a.offsets[lane];
    const int full = cnt / kGM;          // full m-tiles of expert `lane`
    const int rem = cnt % kGM;           // rows of its partial m-tile (0: none)
    int incl = full;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    const int n_full = lane_value(incl, 63);
    const uint64_t has_part = __ballot(rem > 0);
    const int n_sh = a.has_shared ? ceil_div(a.T, kGM) : 0;
    const int total_units = (n_sh + n_full + __popcll(has_part)) * NT;
    if (unit >= total_units) return false;
    int e, mti, nt;
    // m-tile position p -> shared m-tile, full m-tile qi or partial m-tile qi
    const int n_part = __popcll(has_part);
    const int p = unit / NT - n_sh;
    nt = unit % NT;
    const int groups = min(n_full / kFullPerPart, n_part);
    bool is_full;
    int qi;
    if (p < 0) {
        e = a.E;
        mti = p + n_sh;
        is_full = true;
        qi = 0;
    } else if (p < groups * (kFullPerPart + 1)) {
        const int gg = p / (kFullPerPart + 1), rr = p % (kFullPerPart + 1);
        is_full = rr < kFullPerPart;
        qi = is_full ? gg * kFullPerPart + rr : gg;
    } else {
        const int p2 = p - groups * (kFullPerPart + 1), rf = n_full - groups * kFullPerPart;
        is_full = p2 < rf;
        qi = is_full ? groups * kFullPerPart + p2 : groups + (p2 - rf);
    }
    if (p < 0) {
        // shared m-tile: e and mti set above
    } else if (is_full) {
        const int q = qi;
        const int excl = incl - full;
        const uint64_t below = __ballot(full > 0 && excl <= q);
        e = 63 - __clzll(static_cast<long long>(below));
        mti = q - lane_value(excl, e);
    } else {
        const int q = qi;
        int rank = 0;                    // partial tiles longer than this lane's, or as long with a lower id
        for (int j = 0; j < 64; ++j) {
            const int rj = lane_value(rem, j);
            rank += (rj > rem) || (rj == rem && j < lane);
        }
        const uint64_t hit = __ballot(rem > 0 && rank == q);
        e = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        mti = lane_value(full, e);
    }
    u.sh = e == a.E;
    u.e = e;
    u.mti = mti;
    u.nt = nt;
    u.r_base = (u.sh ? a.T * a.k : a.offsets[e]) + mti * kGM;
    u.nvalid = min(kGM, (u.sh ? a.T * a.k + a.T : a.offsets[e + 1]) - u.r_base);
    u.slot = u.sh ? 0 : a.slot_of_expert ? a.slot_of_expert[e] : e;
    return true;
}

// Unit of workgroup `wg` of a projection with NT n-tiles.  Workgroups are
// dealt round-robin over the 8 XCDs, and every XCD keeps the weight tiles
// and token rows it reads in its own L2.  With NT = 8, G consecutive m-tile
// positions share the 8 XCDs: XCD x takes n-tiles G(x % (8/G)) .. +G-1 of
// position Gj + x / (8/G).  An m-tile's token rows are then fetched by 8/G
// XCDs instead of 8, and a weight tile of an expert with several m-tiles by
// up to G.  Measured per FFN call at the 2048-token prefill chunk against
// G = 1: bf16 tokens -1.6 % at G = 2 (G = 4 and 8 within noise of G = 1);
// MXFP8 tokens -2.5 / -4.3 / -4.4 % at G = 2 / 4 / 8, MXFP4 tokens -3 % at
// G = 4; 2-bit packs -1.2 / -4.3 / -4.8 %, 4-bit packs unchanged at G = 2
// and 4.  After the K-loop scheduling changes of the MXFP4 kernel, bf16
// tokens measured G = 4 1.0 % faster than G = 2 and G = 1 0.6 % slower
// (three alternating runs, one box); every launch now takes G = 4.  The
// launches round their m-tile count up to a multiple of
// kPosBlockMax, so every block of positions is whole.
constexpr int kPosBlockMax = 4;
template <int G>
__device__ __forceinline__ int grouped_unit_index(int wg, int NT) {
    static_assert(G == 1 || G == 2 || G == 4, "positions per block");
    if (NT != 8 || G == 1) return wg;
    constexpr int XG = 8 / G;
    const int j = wg / (8 * G), h = (wg >> 3) % G, x = wg & 7;
    return 8 * (G * j + x / XG) + G * (x % XG) + h;
}

// Zeroes the y rows past offsets[E] (pairs with an invalid expert id); block
// `blk` of `nblk` takes every nblk-th float4.
__device__ __forceinline__ void zero_tail_rows(const FfnArgs& a, int blk, int nblk) {
    const int r_lo = a.offsets[a.E], r_hi = a.T * a.k;
    const int n4 = a.d / 4;
    float4* base = reinterpret_cast<float4*>(a.y + static_cast<size_t>(r_lo) * a.d);
    const long long total = static_cast<long long>(r_hi - r_lo) * n4;
    for (long long i = blk * static_cast<long long>(blockDim.x) + threadIdx.x; i < total;
         i += static_cast<long long>(nblk) * blockDim.x)
        base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace qrmoe
