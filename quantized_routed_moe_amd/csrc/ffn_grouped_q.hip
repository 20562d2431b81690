// Expert FFN for many token rows per expert (prefill chunks) with the 2-bit
// and 4-bit group-asymmetric packs (w = scale * q + min per 32-element group,
// "DwarfStar 4 (ds4) | Mac Studio 原生部署 DeepSeek V4 Flash 完整指南",
// section 性能实测参考: q2 and q4 prefill): a grouped GEMM over the
// token-by-expert permutation, both projections in one launch, on the units
// and schedule of the MXFP4 kernel (grouped_sched.hpp, chain.hpp).
//
// Arithmetic.  A bf16 operand cannot hold scale * q + min exactly, so the
// weight operand is bf16(1 + q/K) (K = 4 for 2-bit, 16 for 4-bit codes;
// exact, bit pattern 0x3F80 | q << 5 or q << 3) and per group g of 32 K
// elements
//     sum_k w_k x_k = (K*scale) * C_g + (min - K*scale) * X_g,
//     C_g = sum_k (1 + q_k/K) x_k,   X_g = sum_k x_k.
// C_g is one 16x16x32 bf16 product per group (K = 32 is exactly one group),
// scaled into the accumulator by the lane's own K*scale: the tokens are the
// MFMA's A operand and the weights its B operand, so a lane's four outputs
// share one weight row.  The second term is itself a product over groups:
// X_g is kept as two fp16 halves (hi + lo, the fp32 sum to 22 bits) and
// min and -K*scale are exact fp16, so one 16x16x16 fp16 product per 4 groups
// adds (X_hi + X_lo)(min - K*scale) for all four, with every product exact
// and fp32 accumulation.  X_g comes precomputed: for the token rows from a
// pass before the launch (xsum_kernel), for the act rows from the gate/up
// tiles, which sum their own bf16 outputs per group before raising their
// flags.
//
// Workgroup = 8 waves; unit = 128 token rows x 512 weight rows; K step 128
// (one block of the tile layout: four groups).  Wave w owns four 16-row
// weight tiles: MODE 0 gate rows [32w, 32w + 32) and the same up rows (so
// silu(g) * u pairs in registers), MODE 1 down rows [64w, 64w + 64); every
// wave covers all the unit's 16-row token tiles.
//
// Operands in LDS, a ring of stages filled by direct global -> LDS loads
// (16 bytes per lane), every wave issuing the same number per stage:
//  * weights: the tile layout's blocks as stored (512 B per 16-row tile and
//    step for 2-bit codes, 1 KB for 4-bit), lane l of a wave reading piece l
//    of a block -- exactly the B operand of a 16x16x32 product (row l%16,
//    elements 8(l/16) .. +8 of each group); the (scale | min << 16) words,
//    16 rows x 4 groups per block;
//  * tokens: bf16 rows of 256 B whose 16-byte chunks are stored XOR-swizzled
//    by row mod 16, so the 16 rows a ds_read_b128 phase reads at one logical
//    chunk fall in 16 distinct bank groups;
//  * the rows' group sums (4 words per row and step).
// The ring holds 32, 64 or 128 token rows (the unit's live 16-row tiles
// rounded up), so units with few rows keep more stages in flight.
#include <type_traits>

#include "chain.hpp"
#include "common.hpp"
#include "grouped_sched.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kQN = 512;                  // weight rows per unit
constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * 64;
constexpr int kQLds = 153600;             // the stage ring (of 160 KB per CU)
constexpr int kQLdsAlloc = kQLds + 16;    // + one word past the ring (the hand-off verdict)

template <int FMT> constexpr int kQBlock = FMT == MOE_FMT_Q4G32 ? 1024 : 512;   // code bytes per tile and step
template <int FMT> constexpr float kQStep = FMT == MOE_FMT_Q4G32 ? 16.f : 4.f;  // operand 1 + q / kQStep

// Stage of a ring for NR staged token rows.
template <int FMT, int NR> struct QRing {
    static constexpr int wc = 0;                                  // codes: 32 tiles
    static constexpr int ws = wc + 32 * kQBlock<FMT>;             // scale words: 32 tiles x 256 B
    static constexpr int xr = ws + 32 * 256;                      // token rows: NR x 256 B
    static constexpr int xs = xr + NR * 256;                      // group sums: NR x 16 B
    static constexpr int stage = xs + NR * 16;
    static constexpr int count = kQLds / stage;
    // loads per wave and stage: codes, scales, token rows, group sums
    static constexpr int loads = 32 * kQBlock<FMT> / 1024 / kQWaves + 1 + NR / 32 + 1;
    static_assert(count >= 2 && count <= 8, "ring depth");
};

template <int L, int R>
__device__ __forceinline__ void q_wait_stages(int r) {
    if constexpr (R == 0) {
        wait_vmcnt<0>();
    } else {
        if (r >= R) wait_vmcnt<R * L>();
        else q_wait_stages<L, R - 1>(r);
    }
}

// Two fp16 halves of an fp32 value: hi = fp16(v), lo = fp16(v - hi).
__device__ __forceinline__ uint32_t f16_pair(float v) {
    const _Float16 hi = static_cast<_Float16>(v);
    const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) << 16);
}

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// D = A(16x16) * B(16x16) + C, fp16 inputs, fp32 accumulate: lane l supplies
// A[l%16][4(l/16) + 0..3] and B[4(l/16) + 0..3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x16_f16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// The weight operand of group g from this lane's piece: eight bf16
// 1 + q/K, element pairs (2h, 2h + 1) in dword h.  2-bit: dword g/2 holds
// the group's even elements in byte g%2 and its odd ones in byte 2 + g%2;
// 4-bit: dword g, even elements' nibbles in the low half, odd in the high.
template <int FMT>
__device__ __forceinline__ bf16x8 q_operand(const u32x4& code, int g, uint32_t qmask) {
    u32x4 av;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        uint32_t x;
        if constexpr (FMT == MOE_FMT_Q4G32) {
            const int sh = 4 * h - 3;
            const uint32_t cw = code[g];
            x = sh >= 0 ? cw >> sh : cw << -sh;
        } else {
            const int sh = 8 * (g & 1) + 2 * h - 5;
            const uint32_t cw = code[g >> 1];
            x = sh >= 0 ? cw >> sh : cw << -sh;
        }
        av[h] = (x & qmask) | 0x3f803f80u;
    }
    return bf16x8_from_u32x4(av);
}

// One work unit on the workgroup's LDS ring (see ffn_grouped.hip for the
// CHAIN hand-off: gate/up units store act and its group sums with
// device-scope stores, then raise flag `unit`; a down unit waits for its
// m-tile's flags, then reads them with device-scope loads).
template <int FMT, int MODE, bool CHAIN>
__device__ __forceinline__ void grouped_q_unit(const FfnArgs& a, int unit, unsigned long long tag, uint8_t* lds) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int NT = MODE == 0 ? a.f / (kQN / 2) : a.d / kQN;
    const int S = K / 128;
    const int G = K / 32;                  // groups per row

    GroupedUnit gu;
    unit = grouped_unit_index<4>(unit, NT);
    if (!grouped_unit_of<kFullPerPartQ>(a, unit, NT, lane, gu)) return;
    const int nt = gu.nt, r_base = gu.r_base, nvalid = gu.nvalid, slot = gu.slot;
    const bool sh = gu.sh;
    auto wcodes = [&](int mat) { return sh ? a.sh_codes[mat] : a.codes[mat]; };
    auto wscales = [&](int mat) { return sh ? a.sh_scales[mat] : a.scales[mat]; };
    auto fill_y = [&](float v) {
        for (int i = tid; i < nvalid * kQN; i += kQThreads)
            a.y[static_cast<size_t>(r_base + i / kQN) * a.d + nt * kQN + i % kQN] = v;
    };
    if (!sh && (slot < 0 || slot >= a.num_slots)) {
        // MOE_SLOT_SKIP: y rows untouched (moe_expert_ffn) or zero (the
        // one-call layers); any other bad slot: zero and MOE_DEV_BAD_SLOT
        const bool skip = slot == MOE_SLOT_SKIP;
        if (!skip && tid == 0 && nt == 0 && gu.mti == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1 && (!skip || a.zero_skipped)) fill_y(0.f);
        if (CHAIN && MODE == 0) raise_flag(a.flags + unit, tag);   // its act is never read
        return;
    }
    if constexpr (CHAIN && MODE == 1) {
        int* chain_ok = reinterpret_cast<int*>(lds + kQLds);
        const int NT0 = a.f / (kQN / 2);
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

    // ---- load roles.  Layout tile of workgroup tile tt (0..31) within its
    // slot: MODE 0 tiles 0..15 are the gate rows of n-tile nt, 16..31 its up
    // rows; MODE 1 the 32 down tiles of the n-tile.
    auto tile_of = [&](int tt, int& mat) {
        mat = 2;
        int tile = nt * (kQN / 16) + tt;
        if (MODE == 0) {
            mat = tt < 16 ? 0 : 1;
            tile = nt * 16 + (tt & 15);
        }
        return tile;
    };
    const size_t slot_blocks = static_cast<size_t>(N / 16) * S;
    const size_t slot_c = static_cast<size_t>(slot) * (a.slot_bytes ? a.slot_bytes : slot_blocks * kQBlock<FMT>);
    const size_t slot_s = static_cast<size_t>(slot) * (a.slot_bytes ? a.slot_bytes : slot_blocks * 256);
    constexpr int kCL = 32 * kQBlock<FMT> / 1024 / kQWaves;      // code loads per wave (2 or 4)
    const uint8_t* csrc[kCL];
#pragma unroll
    for (int i = 0; i < kCL; ++i) {
        // 1 KB per load: 2-bit, tiles 4w + 2i + (lane >> 5); 4-bit, tile 4w + i
        const int tt = FMT == MOE_FMT_Q4G32 ? 4 * wave + i : 4 * wave + 2 * i + (lane >> 5);
        const int off = FMT == MOE_FMT_Q4G32 ? 16 * lane : 16 * (lane & 31);
        int mat;
        const size_t tile = tile_of(tt, mat);
        csrc[i] = wcodes(mat) + slot_c + tile * S * kQBlock<FMT> + off;
    }
    const uint8_t* ssrc;         // scale words: tile 4w + (lane >> 4), row lane & 15
    {
        int mat;
        const size_t tile = tile_of(4 * wave + (lane >> 4), mat);
        ssrc = wscales(mat) + slot_s + tile * S * 256 + 16 * (lane & 15);
    }

    const int ntt = __builtin_amdgcn_readfirstlane(ceil_div(nvalid, 16));   // live 16-row token tiles
    // rows of token row r (< nvalid, else a valid row) and of its group sums
    auto row_src = [&](int row) {
        const int rr = r_base + (row < nvalid ? row : 0);
        return MODE == 0 ? a.x + static_cast<size_t>(a.perm[rr] / a.k) * a.d : a.act + static_cast<size_t>(rr) * a.f;
    };
    auto sum_src = [&](int row) {
        const int rr = r_base + (row < nvalid ? row : 0);
        return MODE == 0 ? a.xsum + static_cast<size_t>(a.perm[rr] / a.k) * G
                         : a.asum + static_cast<size_t>(rr) * G;
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wave's four weight tiles in the stage (workgroup tile index)
    auto wtile = [&](int m) { return MODE == 0 ? (m < 2 ? 2 * wave + m : 16 + 2 * wave + (m - 2)) : 4 * wave + m; };
    uint32_t qmask = FMT == MOE_FMT_Q4G32 ? 0x00780078u : 0x00600060u;
    asm volatile("" : "+v"(qmask));   // one v_and_or_b32 per pair (VOP3 takes no second literal)

    auto run = [&](auto nr_c, auto ntt_c) {
        constexpr int NR = decltype(nr_c)::value, NTT = decltype(ntt_c)::value;
        using R = QRing<FMT, NR>;
        constexpr int NST = R::count, SB = R::stage;
        constexpr int kRows = NR / 32;                       // token-row loads per wave (4 rows each)
        const uint16_t* xsrc[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const int row = (wave * kRows + j) * 4 + (lane >> 4);
            const int gch = (lane & 15) ^ (row & 15);          // global chunk for this lane's LDS chunk
            xsrc[j] = row_src(row) + gch * 8;
        }
        const int srow = wave * (NR / 8) + lane;               // group-sum row of this lane (lane < NR / 8)
        const uint32_t* gsrc = sum_src(lane < NR / 8 ? srow : 0);
        auto issue = [&](int s) {
            uint8_t* base = lds + (s % NST) * SB;
#pragma unroll
            for (int i = 0; i < kCL; ++i)
                __builtin_amdgcn_global_load_lds(csrc[i] + static_cast<size_t>(s) * kQBlock<FMT>,
                                                 (lds_void*)(base + R::wc + 4 * wave * kQBlock<FMT> + 1024 * i), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(ssrc + static_cast<size_t>(s) * 256,
                                             (lds_void*)(base + R::ws + 4 * wave * 256), 16, 0, 0);
#pragma unroll
            for (int j = 0; j < kRows; ++j)
                __builtin_amdgcn_global_load_lds(xsrc[j] + s * 128, (lds_void*)(base + R::xr + (wave * kRows + j) * 1024),
                                                 16, 0, CHAIN && MODE == 1 ? kAuxDevice : 0);
            if (lane < NR / 8)
                __builtin_amdgcn_global_load_lds(gsrc + s * 4, (lds_void*)(base + R::xs + wave * (NR / 8) * 16), 16, 0,
                                                 CHAIN && MODE == 1 ? kAuxDevice : 0);
        };
        for (int s = 0; s < NST - 1 && s < S; ++s) issue(s);
        for (int s = 0; s < S; ++s) {
            q_wait_stages<R::loads, NST - 2>(min(NST - 2, S - 1 - s));
            __builtin_amdgcn_s_barrier();
            const uint8_t* b = lds + (s % NST) * SB;
            // this lane's pieces and scale words of the four weight tiles
            u32x4 code[4], smw[4];
            uint32_t mw[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint8_t* cb = b + R::wc + wtile(m) * kQBlock<FMT>;
                if constexpr (FMT == MOE_FMT_Q4G32) {
                    code[m] = *reinterpret_cast<const u32x4*>(cb + 16 * lane);
                } else {
                    const u32x2 c2 = *reinterpret_cast<const u32x2*>(cb + 8 * lane);
                    code[m] = u32x4{c2[0], c2[1], 0u, 0u};
                }
                const uint8_t* sb = b + R::ws + wtile(m) * 256 + 16 * (lane & 15);
                smw[m] = *reinterpret_cast<const u32x4*>(sb);
                mw[m] = *reinterpret_cast<const uint32_t*>(sb + 4 * (lane >> 4));   // group lane / 16 (the min term)
            }
            // the next stage's copies go out after this stage's fragment
            // reads, so the reads are not queued behind them
            __builtin_amdgcn_sched_barrier(0);
            if (s + NST - 1 < S) issue(s + NST - 1);
            __builtin_amdgcn_sched_barrier(0);
            // min term: A' = (X_hi, X_lo, X_hi, X_lo) of the token row's group
            // lane / 16, B' = (min, min, -K scale, -K scale) of the weight row's
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t mn = mw[m] >> 16;
                const _Float16 nks = static_cast<_Float16>(-kQStep<FMT> * fp16_to_f32(mw[m]));
                const uint32_t k16 = __builtin_bit_cast(uint16_t, nks);
                const u32x2 bm = {mn | (mn << 16), k16 | (k16 << 16)};
#pragma unroll
                for (int t = 0; t < NTT; ++t) {
                    const uint32_t xs = *reinterpret_cast<const uint32_t*>(b + R::xs + (16 * t + (lane & 15)) * 16 +
                                                                             4 * (lane >> 4));
                    acc[m][t] = mfma16x16x16_f16(u32x2{xs, xs}, bm, acc[m][t]);
                }
            }
            // Per group: the products of token tile t are issued while the
            // scaling of tile t - 1's products into the accumulators runs, so
            // the matrix core and the vector ALU work side by side (the
            // scheduling groups pin the pattern: one product, then the four
            // multiply-adds of the previous tile's product with the same
            // weight tile), and the token fragment of tile t + 1 is read
            // from LDS one tile ahead.
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x8 wop[4];
                float ks[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    wop[m] = q_operand<FMT>(code[m], g, qmask);
                    ks[m] = kQStep<FMT> * fp16_to_f32(smw[m][g]);
                }
                auto xfrag = [&](int t) {
                    return *reinterpret_cast<const bf16x8*>(b + R::xr + (16 * t + (lane & 15)) * 256 +
                                                            (((4 * g + (lane >> 4)) ^ (lane & 15)) << 4));
                };
                bf16x8 xa = xfrag(0);
                f32x4 cp[4];
#pragma unroll
                for (int t = 0; t <= NTT; ++t) {
                    bf16x8 xn = xa;
                    if (t + 1 < NTT) xn = xfrag(t + 1);
                    f32x4 cc[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        if (t < NTT) cc[m] = mfma16x16x32(xa, wop[m], f32x4{0.f, 0.f, 0.f, 0.f});
                        if (t > 0) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[m][t - 1][i] = fmaf(ks[m], cp[m][i], acc[m][t - 1][i]);
                        }
                        if (t < NTT && t > 0) {
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one product
                            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four multiply-adds
                        }
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m) cp[m] = cc[m];
                    xa = xn;
                }
            }
        }
    };
    // staged rows: the live 16-row tiles rounded up to 32, 64 or 128 rows
    if (ntt <= 2) {
        if (ntt == 1) run(std::integral_constant<int, 32>{}, std::integral_constant<int, 1>{});
        else run(std::integral_constant<int, 32>{}, std::integral_constant<int, 2>{});
    } else if (ntt <= 4) {
        run(std::integral_constant<int, 64>{}, std::integral_constant<int, 4>{});
    } else {
        run(std::integral_constant<int, 128>{}, std::integral_constant<int, 8>{});
    }

    // ---- epilogue.  Lane l holds, for element i of acc[m][t], token row
    // 16t + 4(l/16) + i and weight row l%16 of the wave's tile m.
    const int q4 = lane >> 4, col = lane & 15;
    if constexpr (MODE == 0) {
        // act = bf16(silu(gate) * up); the wave's 32 act columns are one
        // group of the down projection: their sum per row (of the bf16
        // values, in a fixed order: the two tiles, then a butterfly over the
        // 16 columns) goes to asum
        const int grp = nt * ((kQN / 2) / 32) + wave;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= ntt) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 16 * t + 4 * q4 + i;
                float sum = 0.f;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const uint16_t v = f32_to_bf16_rne(silu_mul(acc[m][t][i], acc[m + 2][t][i]));
                    sum += bf16_to_f32(v);
                    if (j < nvalid) {
                        uint16_t* dst = a.act + static_cast<size_t>(r_base + j) * a.f + nt * (kQN / 2) + 32 * wave +
                                        16 * m + col;
                        if constexpr (CHAIN) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else *dst = v;
                    }
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o);
                if (col == 0 && j < nvalid) {
                    uint32_t* dst = a.asum + static_cast<size_t>(r_base + j) * (a.f / 32) + grp;
                    const uint32_t pair = f16_pair(sum);
                    if constexpr (CHAIN) __hip_atomic_store(dst, pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else *dst = pair;
                }
            }
        }
        if constexpr (CHAIN) raise_flag(a.flags + unit, tag);
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= ntt) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 16 * t + 4 * q4 + i;
                if (j >= nvalid) continue;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    a.y[static_cast<size_t>(r_base + j) * a.d + nt * kQN + 64 * wave + 16 * m + col] = acc[m][t][i];
            }
        }
    }
}

// Both projections in one launch (as ffn_grouped_chained_kernel): gate/up
// units [0, ub0), down units [ub0, ub0 + ub1), then the y tail rows.
template <int FMT>
__global__ __launch_bounds__(kQThreads) void ffn_grouped_q_kernel(FfnArgs a, int ub0, int ub1) {
    __shared__ __align__(16) uint8_t lds[kQLdsAlloc];
    const unsigned long long tag = chain_tag();
    const int b = blockIdx.x;
    if (b < ub0) grouped_q_unit<FMT, 0, true>(a, b, tag, lds);
    else if (b < ub0 + ub1) grouped_q_unit<FMT, 1, true>(a, b - ub0, tag, lds);
    else zero_tail_rows(a, 0, 1);
}

// xsum[t][g] = the sum of x[t][32g .. 32g + 32) (fp32, in element order), as
// two fp16 halves; one thread per (token, group).
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, uint32_t* __restrict__ xsum, int T,
                                                   int d) {
    const int G = d / 32;
    const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<long long>(T) * G) return;
    const int t = static_cast<int>(i / G), g = static_cast<int>(i % G);
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * d + 32 * g);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 w = src[c];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s += bf16lo(w[e]);
            s += bf16hi(w[e]);
        }
    }
    xsum[i] = f16_pair(s);
}

static int q_max_mtiles(const moe_shape& s, bool shared) {
    const int pairs = s.T * s.k;
    const int m = ceil_div(pairs, kGM) + (s.E < pairs ? s.E : pairs) + (shared ? ceil_div(s.T, kGM) : 0);
    return (m + kPosBlockMax - 1) / kPosBlockMax * kPosBlockMax;   // whole blocks of grouped_unit_index
}

hipError_t launch_ffn_grouped_q(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    if (!a.flags || !a.xsum || !a.asum) return hipErrorInvalidValue;
    const long long n = static_cast<long long>(s.T) * (s.d / 32);
    xsum_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(a.x, a.xsum, s.T, s.d);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int units0 = q_max_mtiles(s, a.has_shared) * (s.f / (kQN / 2));
    const int units1 = q_max_mtiles(s, a.has_shared) * (s.d / kQN);
    if (fmt == MOE_FMT_Q4G32)
        ffn_grouped_q_kernel<MOE_FMT_Q4G32><<<units0 + units1 + 1, kQThreads, 0, st>>>(a, units0, units1);
    else
        ffn_grouped_q_kernel<MOE_FMT_Q2G32><<<units0 + units1 + 1, kQThreads, 0, st>>>(a, units0, units1);
    return hipGetLastError();
}

}  // namespace qrmoe
