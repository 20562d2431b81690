// Expert FFN for few token rows per expert (decode, speculative verify,
// short batches).  Each activated expert's quantised weights are streamed
// from HBM once and dequantised in registers ("antirez ds4: DeepSeek Metal
// inference", section 技术深度解析: the block-sparse routed-expert kernel loads
// only the activated experts' weights and dequantises them on the fly).
//
// The active expert of a work item is found on the device from offsets[E+1];
// there is no host round trip.
//
// Weights come in the tile layout, so every weight load of a wave reads one
// contiguous 16-row x 128-element block (1 KB of MXFP4 codes).
//
// Two launches: gate/up + SwiGLU (act to the workspace), then down (y).  A
// single persistent kernel with a grid barrier between the projections was
// measured slower on MI355X: a cooperative launch alone costs ~20 us and a
// 256-workgroup barrier 8-14 us, more than the whole down projection.
#include "common.hpp"
#include "ffn_tile.hpp"
#include "kernels.hpp"
#include "topk_dev.hpp"

namespace qrmoe {

// Waves per workgroup (K split): gate/up K = d, down K = f.  With d = 4096 /
// f = 2048 every wave holds its whole K slice (4 steps) in registers, so all
// of a workgroup's weight loads are in flight at once.
constexpr int kGateUpWaves = 8;
constexpr int kDownWaves = 4;

// The `ai`-th active expert (in id order) of offsets[E+1], its sorted rows
// [r0, r1) and its pack slot, from one load per lane (lane e reads
// offsets[e], offsets[e+1] and slot_of_expert[e]) and wave shuffles.  Every
// lane of the wave receives the result; e = -1 when fewer than ai+1 experts
// are active.
struct Item {
    int e, r0, r1, slot;
};

__device__ __forceinline__ Item pick_item(int lo, int hi, int sl, int ai) {
    const int lane = threadIdx.x & 63;
    const uint64_t mask = __ballot(hi > lo);
    const uint64_t below = mask & ((1ull << lane) - 1ull);
    const uint64_t hit = __ballot(((mask >> lane) & 1ull) && __popcll(below) == ai);
    Item it;
    it.e = hit ? __ffsll(static_cast<unsigned long long>(hit)) - 1 : -1;
    const int src = it.e < 0 ? 0 : it.e;
    it.r0 = lane_value(lo, src);
    it.r1 = lane_value(hi, src);
    it.slot = lane_value(sl, src);
    return it;
}

__device__ __forceinline__ Item find_item(const FfnArgs& a, int ai) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = 0, sl = lane;
    if (lane < a.E) {
        lo = a.offsets[lane];
        hi = a.offsets[lane + 1];
        if (a.slot_of_expert) sl = a.slot_of_expert[lane];
    }
    return pick_item(lo, hi, sl, ai);
}

// Item ai of the launch.  SH (a shared expert; separate instantiations, so
// the kernels without one are unchanged): item 0 is the shared expert (e = E,
// rows [T*k, T*k + T), slot 0 of its own pack) and item ai > 0 the (ai-1)-th
// active routed expert.
template <bool SH>
__device__ __forceinline__ Item item_at(const FfnArgs& a, int ai) {
    if constexpr (SH) {
        if (ai == 0) return Item{a.E, a.T * a.k, a.T * a.k + a.T, 0};
        --ai;
    }
    return find_item(a, ai);
}

// Pack of an item: the shared expert's own, or the routed experts'.
template <bool SH>
__device__ __forceinline__ const uint8_t* item_codes(const FfnArgs& a, const Item& it, int mat) {
    if constexpr (SH) return it.e == a.E ? a.sh_codes[mat] : a.codes[mat];
    return a.codes[mat];
}
template <bool SH>
__device__ __forceinline__ const uint8_t* item_scales(const FfnArgs& a, const Item& it, int mat) {
    if constexpr (SH) return it.e == a.E ? a.sh_scales[mat] : a.scales[mat];
    return a.scales[mat];
}

// Zero y rows [r0, r1) x [n0, n0+16) (down tiles of an expert whose slot is invalid).
__device__ __forceinline__ void zero_y_tile(const FfnArgs& a, int n0, int r0, int r1) {
    for (int i = threadIdx.x; i < (r1 - r0) * 16; i += blockDim.x)
        a.y[static_cast<size_t>(r0 + i / 16) * a.d + n0 + i % 16] = 0.f;
}

// Rows past offsets[E] (pairs with an invalid expert id) read as zero.
__device__ __forceinline__ void zero_y_tail(const FfnArgs& a) {
    const int r_lo = a.offsets[a.E], r_hi = a.T * a.k;
    const int n4 = a.d / 4;
    float4* base = reinterpret_cast<float4*>(a.y + static_cast<size_t>(r_lo) * a.d);
    for (long long i = threadIdx.x; i < static_cast<long long>(r_hi - r_lo) * n4; i += blockDim.x)
        base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Work item = (active expert, tile of 16 weight rows); block = KW waves that
// split the K steps; their partial tiles are summed in LDS in wave order.
//  MODE 0: gate and up + SwiGLU -> act (bf16).  MODE 1: down -> y (fp32), or
//          with fuse_combine the weighted scatter-add into out instead.
// The expert's sorted rows are taken RB at a time (a column pass): column c
// of a pass is sorted row c0 + c; MODE 0 stages x[perm[r]/k], MODE 1 act[r]
// (ffn_tile.hpp).  The weights of a wave's K slice stay in registers across
// the passes when the slice fits one chunk.
//
// Load order: vmcnt retires loads in issue order.  When the token rows'
// addresses need no global load (the down projection reads act[r]; PERM_LDS)
// the token rows are staged first (small and cached), so the multiplies of
// the first steps start as soon as those steps' weights arrive.  Otherwise
// the weights go first and the row indices (perm) are read behind them.
// (Taking the T <= 16 tokens themselves as the columns, which drops that
// index load, measured no faster at T = 1 and slower at T = 5 and 16, where
// most columns then load token rows the expert does not own.)
//
// `it` is the item's expert, rows and slot, `n0` its first weight row; `perm`
// is the sorted-row -> pair map (global, or with PERM_LDS the workgroup's own
// LDS copy).
template <int FMT, int MODE, int KW, int RB, bool PERM_LDS, bool SH>
__device__ __forceinline__ void skinny_body(const FfnArgs& a, const Item& it, int n0, const int32_t* perm) {
    constexpr int NM = MODE == 0 ? 2 : 1;
    // Per wave: RB staged token rows; after the pass's multiplies the same
    // bytes hold the wave's partial tiles for the reduction.
    constexpr int kRegion = RB * kBRowBytes > NM * kWave * 16 ? RB * kBRowBytes : NM * kWave * 16;
    __shared__ __align__(16) uint8_t region[KW][kRegion];
    __shared__ int row_tok[RB];     // fused combine: token of the row
    __shared__ float row_w[RB];     // fused combine: routing weight of the row
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int S = ceil_div(K, kStepK), NT = N / 16;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: K-slice branches stay scalar
    const int col = lane & 15;
    const int s_beg = (S * wave) / KW, s_end = (S * (wave + 1)) / KW;
    const int nk = ceil_div(s_end - s_beg, kCapOf<FMT>);
    const bool fused = MODE == 1 && a.fuse_combine;
    uint8_t* mine = region[wave];
    const uint8_t* brow = mine + (col < RB ? col : RB - 1) * kBRowBytes;
    constexpr bool b_first = MODE == 1;

    WTile wt[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int mat = MODE == 0 ? m : 2;
        wt[m] = wtile<FMT>(item_codes<SH>(a, it, mat), item_scales<SH>(a, it, mat), it.slot, a.slot_bytes, NT,
                           n0 / 16, S, lane);
    }
    WChunk<FMT> w[NM];
    f32x4 acc[kChains<FMT>][NM];
    int pr = 0;             // MODE 0: pair of this lane's column in the current pass
    int tokc[RB];           // fused combine: token and routing weight of each column
    float wc[RB];

    // MODE 0: pair of column `col` of the pass at c0 (a valid row for every
    // lane), issued before the weights so that waiting for it never waits
    // for them.
    auto load_pr = [&](int c0) {
        if constexpr (MODE == 0) pr = perm[min(c0 + col, it.r1 - 1)];
    };
    // Fused combine: token and weight of each column, by scalar loads
    // (wave-uniform addresses), issued once the pass's vector loads are in
    // flight; the scalar counter is independent of the vector one.
    auto load_fused = [&](int c0) {
        if constexpr (MODE == 1) {
            if (!fused) return;
            typedef const __attribute__((address_space(4))) int32_t* cint;
            typedef const __attribute__((address_space(4))) float* cfloat;
            int p[RB];
#pragma unroll
            for (int c = 0; c < RB; ++c) p[c] = ((cint)perm)[min(c0 + c, it.r1 - 1)];
#pragma unroll
            for (int c = 0; c < RB; ++c) {
                wc[c] = ((cfloat)a.topk_w)[p[c]];
                tokc[c] = p[c] / a.k;
            }
        }
    };
    // Issues the loads of chunk kc of the pass at c0 (the weights too when
    // `weights`) and waits until the staged token rows have landed.
    auto issue = [&](int c0, int kc, bool weights) {
        const int nreal = min(RB, it.r1 - c0);
        const int s0 = s_beg + kc * kCapOf<FMT>;
        // staged row c: sorted row min(c0 + c, r1 - 1) (pr is clamped alike)
        auto src_row = [&](int c) -> const uint16_t* {
            if constexpr (MODE == 0) return a.x + static_cast<size_t>(lane_value(pr, c) / a.k) * a.d;
            else return a.act + static_cast<size_t>(c0 + min(c, nreal - 1)) * a.f;
        };
        if constexpr (b_first) {
            stage_rows<RB>(mine, src_row, s0 * kStepK, K);
            // keep the weight loads behind the staged rows
            __builtin_amdgcn_sched_barrier(0);
            if (weights) {
#pragma unroll
                for (int m = 0; m < NM; ++m) load_w<FMT>(w[m], wt[m], s0, s_end);
                // the staged rows are older than every load issued after them
                wait_vmcnt<NM * kWLoads<FMT>>();
            } else {
                wait_vmcnt<0>();
            }
        } else {
            if (weights) {
#pragma unroll
                for (int m = 0; m < NM; ++m) load_w<FMT>(w[m], wt[m], s0, s_end);
            }
            // keep the row addresses (a wait for perm) below the weight loads
            __builtin_amdgcn_sched_barrier(0);
            stage_rows<RB>(mine, src_row, s0 * kStepK, K);
            wait_vmcnt<0>();
        }
    };
    auto multiply = [&](int kc) {
        mma_chunk<FMT, NM>(acc, w, brow, min(kCapOf<FMT>, s_end - (s_beg + kc * kCapOf<FMT>)));
    };
    // Sums the waves' partial tiles of the pass at c0 in wave order and
    // stores its columns.
    auto finish = [&](int c0) {
        const int nreal = min(RB, it.r1 - c0);
        // each wave's own multiplies are done: its staged rows are free
        f32x4* red = reinterpret_cast<f32x4*>(mine);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            f32x4 v = acc[0][m];
#pragma unroll
            for (int c = 1; c < kChains<FMT>; ++c) v += acc[c][m];
            red[m * kWave + lane] = v;
        }
        if (fused && wave == 0 && lane == 0) {
#pragma unroll
            for (int c = 0; c < RB; ++c) {
                row_tok[c] = tokc[c];
                row_w[c] = wc[c];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < nreal * 16; idx += KW * kWave) {
            // column cc, weight row nn: lane nn + 16 (cc / 4), element cc % 4
            const int cc = idx >> 4, nn = idx & 15;
            const int src = nn + 16 * (cc >> 2), i = cc & 3;
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float sum = reinterpret_cast<const f32x4*>(region[0])[m * kWave + src][i];
#pragma unroll
                for (int ww = 1; ww < KW; ++ww) sum += reinterpret_cast<const f32x4*>(region[ww])[m * kWave + src][i];
                v[m] = sum;
            }
            const size_t rr = static_cast<size_t>(c0 + cc);
            const int n = n0 + nn;
            if constexpr (MODE == 0) {
                a.act[rr * a.f + n] = f32_to_bf16_rne(silu_mul(v[0], v[NM - 1]));
            } else if (fused) {
                // scatter-add of the weighted expert output; with at most two
                // addends on a zeroed out the sum does not depend on their
                // order (it equals the combine kernel's)
                atomicAdd(a.out + static_cast<size_t>(row_tok[cc]) * a.d + n, __fmul_rn(row_w[cc], v[0]));
            } else {
                a.y[rr * a.d + n] = v[0];
            }
        }
        // the next pass overwrites the partial tiles
        if (c0 + RB < it.r1) __syncthreads();
    };
    auto zero_acc = [&] {
#pragma unroll
        for (int c = 0; c < kChains<FMT>; ++c)
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    // First pass, first chunk: straight-line loads and multiplies, so the
    // waits before the multiplies count exactly the loads in flight.
    load_pr(it.r0);
    issue(it.r0, 0, true);
    load_fused(it.r0);
    zero_acc();
    multiply(0);
    for (int kc = 1; kc < nk; ++kc) {
        issue(it.r0, kc, true);
        multiply(kc);
    }
    finish(it.r0);
    // Later passes (more rows than RB): the weights stay in registers when
    // the K slice is one chunk.
    for (int c0 = it.r0 + RB; c0 < it.r1; c0 += RB) {
        load_pr(c0);
        issue(c0, 0, nk > 1);
        load_fused(c0);
        zero_acc();
        multiply(0);
        for (int kc = 1; kc < nk; ++kc) {
            issue(c0, kc, true);
            multiply(kc);
        }
        finish(c0);
    }
}

// An item whose expert is left out of the call (MOE_SLOT_SKIP) writes
// nothing, except that in the one-call layer (zero_skipped) its y rows read
// as zero (with the fused combine it simply adds nothing); one whose slot is
// otherwise invalid is skipped too, but its y rows read as zero and
// MOE_DEV_BAD_SLOT is raised.
template <int FMT, int MODE, int KW, int RB, bool PERM_LDS = false, bool SH = false>
__device__ __forceinline__ void run_item(const FfnArgs& a, const Item& it, int n0, const int32_t* perm) {
    if (it.e < 0) return;
    if (it.slot == MOE_SLOT_SKIP) {
        if (MODE == 1 && a.zero_skipped && !a.fuse_combine) zero_y_tile(a, n0, it.r0, it.r1);
        return;
    }
    if ((!SH || it.e < a.E) && (it.slot < 0 || it.slot >= a.num_slots)) {
        if (threadIdx.x == 0 && n0 == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) zero_y_tile(a, n0, it.r0, it.r1);
        return;
    }
    skinny_body<FMT, MODE, KW, RB, PERM_LDS, SH>(a, it, n0, perm);
}

// Every workgroup zeroes its share of out (the fused combine's scatter-add
// target), after its item.
__device__ __forceinline__ void zero_out_share(const FfnArgs& a) {
    const int total = a.T * a.d / 4;
    const int chunk = ceil_div(total, static_cast<int>(gridDim.x));
    const int end = min(total, (static_cast<int>(blockIdx.x) + 1) * chunk);
    float4* o4 = reinterpret_cast<float4*>(a.out);
    for (int i = static_cast<int>(blockIdx.x) * chunk + static_cast<int>(threadIdx.x); i < end;
         i += static_cast<int>(blockDim.x))
        o4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Down-weight prefetch: workgroups appended to the gate/up launch copy the
// down tiles of the active experts through the cache hierarchy into a
// scratch LDS buffer (the copies are discarded), so that the down launch,
// one latency-bound round of workgroups, finds its weights in L2 instead of
// HBM.  Down item i (active expert i / (d/16), tile i % (d/16)) runs as
// workgroup i of the down launch, on XCD i % 8; prefetch workgroup j of
// n_pf takes the items i = j (mod n_pf), and with n_pf and the gate/up
// grid both multiples of 8 it runs on the same XCD, whose L2 the down
// workgroup reads.  `item_of(ai)` gives the ai-th active expert.
//
// Used only when the gate/up items and the prefetch workgroups are resident
// together (decode): 128 workgroups measured +2.9 % decode layer throughput
// (64: -2.7 %, 256: +1.4 %); at 5 and 16 tokens, where the gate/up launch
// already fills the chip, the prefetch cost 11-16 %.
constexpr int kDownPrefetchWGs = 128;
// Gate/up workgroups resident at once: two 8-wave workgroups per CU at <= 128
// VGPRs, 256 CUs.
constexpr int kResidentGateUpWGs = 512;

template <int FMT, bool SH, typename ItemOf>
__device__ __forceinline__ void prefetch_down(const FfnArgs& a, int j, int n_pf, ItemOf item_of, uint8_t* scratch) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int NTd = a.d / 16, S = ceil_div(a.f, kStepK);
    const int code_bytes = S * kWave * PieceBytes<FMT>::codes;      // one tile's codes, contiguous
    const int scale_bytes = S * kWave * PieceBytes<FMT>::scales;    // and its scales
    for (int q = wave;; q += blockDim.x / kWave) {
        const int i = j + n_pf * q;
        const int ai = i / NTd, t = i % NTd;
        const Item it = item_of(ai);
        if (it.e < 0) break;                  // past the active experts (ai grows with q)
        if ((!SH || it.e < a.E) && (it.slot < 0 || it.slot >= a.num_slots)) continue;
        const WTile tl = wtile<FMT>(item_codes<SH>(a, it, 2), item_scales<SH>(a, it, 2), it.slot, a.slot_bytes, NTd, t,
                                    S, 0);
        const uint8_t* c = tl.codes;
        const uint8_t* sc = tl.scales;
        // 1 KB per instruction, lanes past the end re-read the last 16 bytes
        for (int o = 0; o < code_bytes; o += 1024)
            __builtin_amdgcn_global_load_lds(c + min(o + 16 * lane, code_bytes - 16), (lds_void*)scratch, 16, 0, 0);
        for (int o = 0; o < scale_bytes; o += 1024)
            __builtin_amdgcn_global_load_lds(sc + min(o + 16 * lane, scale_bytes - 16), (lds_void*)scratch, 16, 0, 0);
    }
    wait_vmcnt<0>();
}

// The last workgroup of the down launch zeroes the y rows past offsets[E];
// with the fused combine the gate/up launch zeroes out.  Gate/up workgroups
// past the items prefetch down weights.
template <int FMT, int MODE, int KW, int RB, bool SH>
__global__ __launch_bounds__(KW * 64) __attribute__((amdgpu_waves_per_eu(4))) void ffn_skinny_kernel(FfnArgs a) {
    if (MODE == 1 && blockIdx.x == gridDim.x - 1) {
        zero_y_tail(a);
        return;
    }
    const int NT = (MODE == 0 ? a.f : a.d) / 16;
    if (MODE == 0) {
        const int g_items = (min(a.E, a.T * a.k) + (SH ? 1 : 0)) * NT;
        if (static_cast<int>(blockIdx.x) >= g_items) {
            __shared__ __align__(16) uint8_t pf[KW][1024];
            prefetch_down<FMT, SH>(a, blockIdx.x - g_items, gridDim.x - g_items,
                                   [&](int ai) { return item_at<SH>(a, ai); }, pf[threadIdx.x >> 6]);
            if (a.fuse_combine) zero_out_share(a);
            return;
        }
    }
    run_item<FMT, MODE, KW, RB, false, SH>(a, item_at<SH>(a, blockIdx.x / NT), (blockIdx.x % NT) * 16, a.perm);
    if (MODE == 0 && a.fuse_combine) zero_out_share(a);
}

// ------------------------------------------------------------ routed gate/up

// Gate/up launch of moe_layer for small batches: every workgroup routes the
// whole batch from the logits itself (top-k by one wave per token, then the
// one-wave counting sort: a few hundred instructions), so no routing launch
// and no read of routing results from HBM precede its weight loads.
// Workgroup 0 also writes ids, w, offsets, perm and inv after its own item,
// and every workgroup zeroes its share of `out` for the down launch's
// scatter-add.  Arithmetic as topk_kernel and the dispatch
// kernel, so every output is identical.
template <int FMT, int RB, bool SH>
__global__ __launch_bounds__(kGateUpWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void ffn_gate_up_routed_kernel(FfnArgs a) {
    __shared__ SmallRouting r;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, E = a.E, k = a.k, n = a.T * a.k;
    int sl = lane;      // slot of expert `lane`, read before the routing is known
    if (lane < E && a.slot_of_expert) sl = a.slot_of_expert[lane];
    if (wave < T) topk_wave(a.logits + static_cast<size_t>(wave) * E, r.ids + wave * k, r.w + wave * k, E, k);
    __syncthreads();
    if (wave == 0) wave_dispatch(r, n, E);
    if constexpr (SH) {                 // the shared expert's rows: row n + t is token t
        __syncthreads();
        if (tid < T) r.perm[n + tid] = tid * k;
    }
    __syncthreads();
    int lo = 0, hi = 0;
    if (lane < E) {
        lo = r.offsets[lane];
        hi = r.offsets[lane + 1];
    }
    const int NT = a.f / 16;
    const int g_items = (min(E, n) + (SH ? 1 : 0)) * NT;
    // item ai: with a shared expert, item 0 is it (rows [n, n + T), slot 0 of its pack)
    auto item_of = [&](int ai) {
        if constexpr (SH) {
            if (ai == 0) return Item{E, n, n + T, 0};
            --ai;
        }
        return pick_item(lo, hi, sl, ai);
    };
    if (static_cast<int>(blockIdx.x) >= g_items) {
        __shared__ __align__(16) uint8_t pf[kGateUpWaves][1024];
        prefetch_down<FMT, SH>(a, blockIdx.x - g_items, gridDim.x - g_items, item_of, pf[wave]);
    } else {
        run_item<FMT, 0, kGateUpWaves, RB, true, SH>(a, item_of(blockIdx.x / NT), (blockIdx.x % NT) * 16, r.perm);
    }
    // after the item: no stores ahead of its loads (the down launch is the
    // first reader of these)
    if (blockIdx.x == 0) {
        for (int i = tid; i < n; i += blockDim.x) {
            a.ids_out[i] = r.ids[i];
            a.w_out[i] = r.w[i];
            a.perm_out[i] = r.perm[i];
            a.inv_out[i] = r.inv[i];
        }
        for (int i = tid; i <= E; i += blockDim.x) a.offsets_out[i] = r.offsets[i];
        if (SH && tid < T) a.perm_out[n + tid] = r.perm[n + tid];
    }
    if (a.fuse_combine) zero_out_share(a);
}

// ------------------------------------------------------------ launch

// Token rows staged per column pass.  An expert owns at most T rows when a
// token's k ids are distinct (more only with repeated ids, which take extra
// passes), so RB follows T; 16 rows of 1 KB per wave fill most of the LDS.
// From 5 to 8 tokens an expert mostly owns a few rows: four staged rows,
// and a second pass (the weights stay in registers) for an expert with
// more, measured 2.5 % faster per verify step (T = 5) than eight; at 16
// tokens four rows measured 4.5 % slower per FFN call than eight.
static int staged_rows(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 8 ? 4 : T <= 16 ? 8 : 16; }

template <int FMT, int RB, bool SH>
static hipError_t launch_two_sh(const moe_shape& s, const FfnArgs& a, hipStream_t st, bool routed) {
    const int umax = (s.E < s.T * s.k ? s.E : s.T * s.k) + (SH ? 1 : 0);
    const int g_items = umax * (s.f / 16);
    const int g_up = g_items + (g_items + kDownPrefetchWGs <= kResidentGateUpWGs ? kDownPrefetchWGs : 0);
    if (routed) {
        if constexpr (RB <= kGateUpWaves)
            ffn_gate_up_routed_kernel<FMT, RB, SH><<<g_up, kGateUpWaves * 64, 0, st>>>(a);
    } else {
        ffn_skinny_kernel<FMT, 0, kGateUpWaves, RB, SH><<<g_up, kGateUpWaves * 64, 0, st>>>(a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_skinny_kernel<FMT, 1, kDownWaves, RB, SH><<<umax * (s.d / 16) + 1, kDownWaves * 64, 0, st>>>(a);
    return hipGetLastError();
}

template <int FMT, int RB>
static hipError_t launch_two_rb(const moe_shape& s, const FfnArgs& a, hipStream_t st, bool routed) {
    return a.has_shared ? launch_two_sh<FMT, RB, true>(s, a, st, routed) : launch_two_sh<FMT, RB, false>(s, a, st, routed);
}

template <int FMT>
static hipError_t launch_two(const moe_shape& s, const FfnArgs& a, hipStream_t st, bool routed) {
    switch (staged_rows(s.T)) {
        case 1: return launch_two_rb<FMT, 1>(s, a, st, routed);
        case 2: return launch_two_rb<FMT, 2>(s, a, st, routed);
        case 4: return launch_two_rb<FMT, 4>(s, a, st, routed);
        case 8: return launch_two_rb<FMT, 8>(s, a, st, routed);
        default: return launch_two_rb<FMT, 16>(s, a, st, routed);
    }
}

// Token rows (T*k) from which the LDS-tiled grouped GEMM takes over.
constexpr int kGroupedMinRows = 256;

bool ffn_uses_grouped(const moe_shape& s, int fmt) {
    return s.T * s.k >= kGroupedMinRows && grouped_supported(s, fmt);
}

bool grouped_shape(const moe_shape& s) {
    return s.T * s.k >= kGroupedMinRows && grouped_supported(s, MOE_FMT_MXFP4);
}

bool routed_ffn_supported(const moe_shape& s, int fmt) {
    // one workgroup per (expert, tile) item, each routing the whole batch:
    // past a few tokens the items of inactive experts (which still route
    // before they find out) cost more than the separate routing launches
    return s.T <= kGateUpWaves && s.T * s.k <= kRoutedMaxPairs && !ffn_uses_grouped(s, fmt);
}

static hipError_t launch_two_fmt(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st, bool routed) {
    switch (fmt) {
        case MOE_FMT_MXFP4: return launch_two<MOE_FMT_MXFP4>(s, a, st, routed);
        case MOE_FMT_Q2G32: return launch_two<MOE_FMT_Q2G32>(s, a, st, routed);
        default: return launch_two<MOE_FMT_Q4G32>(s, a, st, routed);
    }
}

hipError_t launch_ffn_routed(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    return launch_two_fmt(s, fmt, a, st, true);
}

hipError_t launch_ffn(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    if (ffn_uses_grouped(s, fmt))
        return fmt == MOE_FMT_MXFP4 ? launch_ffn_grouped(s, a, st) : launch_ffn_grouped_q(s, fmt, a, st);
    return launch_two_fmt(s, fmt, a, st, false);
}

}  // namespace qrmoe
