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
// Column c of a 16-row column tile is sorted row c0 + c: MODE 0 reads
// x[perm[r]/k], MODE 1 reads act[r]; padding columns read a valid row and
// are zeroed.  Loads are ordered so that nothing waits on the weight stream
// before the multiply: vmcnt retires loads in issue order, so the row index
// an address needs (perm) is loaded before the weights.  (Taking the T <= 16
// tokens themselves as the columns, which drops that index load, measured no
// faster at T = 1 and slower at T = 5 and 16, where most columns then load
// token rows the expert does not own.)
//
// `it` is the item's expert, rows and slot, `n0` its first weight row; `perm`
// is the sorted-row -> pair map (global, or with PERM_LDS the workgroup's own
// LDS copy).  When the token rows' addresses need no global load (the down
// projection reads act[r]; PERM_LDS) the token operand is loaded first: it
// is small and cached, and with it in place the multiplies of the first
// steps start as soon as those steps' weights arrive.
template <int FMT, int MODE, int KW, bool PERM_LDS>
__device__ __forceinline__ void skinny_body(const FfnArgs& a, const Item& it, int n0, const int32_t* perm) {
    constexpr int NM = MODE == 0 ? 2 : 1;
    __shared__ __align__(16) f32x4 red[KW][NM][kWave];
    __shared__ __align__(16) Q2Lds q2[FMT == MOE_FMT_Q2G32 ? KW * NM : 1];
    __shared__ int row_tok[16];     // fused combine: token of the row
    __shared__ float row_w[16];     // fused combine: routing weight of the row
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int G = K / kGroup, S = ceil_div(K, kStepK), NT = N / 16;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, g = lane >> 4;
    const int s_beg = (S * wave) / KW, s_end = (S * (wave + 1)) / KW;
    const int nk = ceil_div(s_end - s_beg, kCap);
    const bool fused = MODE == 1 && a.fuse_combine;

    // Row index of the first column tile, loaded ahead of the weights.
    int r = it.r0 + row;
    bool colok = r < it.r1;
    int pr = colok && (MODE == 0 || fused) ? perm[r] : 0;
    constexpr bool b_first = MODE == 1 || PERM_LDS;
    const uint16_t* brow = nullptr;
    u32x4 bv[kCap][4];
    if constexpr (b_first) {
        brow = MODE == 0 ? a.x + static_cast<size_t>(pr / a.k) * a.d
                         : a.act + static_cast<size_t>(colok ? r : it.r0) * a.f;
        load_b<FMT>(bv, brow, colok, s_beg, G, g);
        __builtin_amdgcn_sched_barrier(0);
    }

    WTile wt[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int mat = MODE == 0 ? m : 2;
        wt[m] = wtile<FMT>(a.codes[mat], a.scales[mat], static_cast<size_t>(it.slot) * NT + n0 / 16, S, lane);
    }
    // Unconditional (a wave with no K steps loads step 0 and ignores it): a
    // load under a branch makes the wait for `pr` below cover the weights too.
    WChunk<FMT> w[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) load_w<FMT>(w[m], wt[m], s_beg, s_end);
    if constexpr (!b_first) {
        // keep the use of `pr` (a global load: its wait) below the weight loads
        __builtin_amdgcn_sched_barrier(0);
        brow = a.x + static_cast<size_t>(pr / a.k) * a.d;
        load_b<FMT>(bv, brow, colok, s_beg, G, g);
    }
    float wr = fused && colok ? a.topk_w[pr] : 0.f;   // queued behind the weights

    const int ncol = ceil_div(it.r1 - it.r0, 16);
    for (int ct = 0; ct < ncol; ++ct) {
        const int c0 = it.r0 + 16 * ct;
        if (ct > 0) {
            r = c0 + row;
            colok = r < it.r1;
            pr = colok && (MODE == 0 || fused) ? perm[r] : 0;
            brow = MODE == 0 ? a.x + static_cast<size_t>(pr / a.k) * a.d
                             : a.act + static_cast<size_t>(colok ? r : it.r0) * a.f;
            wr = fused && colok ? a.topk_w[pr] : 0.f;
        }
        f32x4 acc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kc = 0; kc < nk; ++kc) {
            const int s0 = s_beg + kc * kCap;
            if (kc > 0 || ct > 0) {
                if (nk > 1) {
#pragma unroll
                    for (int m = 0; m < NM; ++m) load_w<FMT>(w[m], wt[m], s0, s_end);
                }
                load_b<FMT>(bv, brow, colok, s0, G, g);
            }
            mma_chunk<FMT, NM>(acc, w, bv, min(kCap, s_end - s0), q2 + wave * NM);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) red[wave][m][lane] = acc[m];
        if (fused && wave == 0 && lane < 16) {
            row_tok[lane] = pr / a.k;
            row_w[lane] = wr;
        }
        __syncthreads();
        const int R = min(16, it.r1 - c0);
        for (int idx = tid; idx < R * 16; idx += KW * kWave) {
            const int cc = idx >> 4, nn = idx & 15;
            const int src = cc + 16 * (nn >> 2), i = nn & 3;
            float v[NM];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                float sum = red[0][m][src][i];
#pragma unroll
                for (int ww = 1; ww < KW; ++ww) sum += red[ww][m][src][i];
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
        __syncthreads();
    }
}

// An item whose expert has no valid slot is skipped: its y rows read as zero
// and MOE_DEV_BAD_SLOT is raised.
template <int FMT, int MODE, int KW, bool PERM_LDS = false>
__device__ __forceinline__ void run_item(const FfnArgs& a, const Item& it, int n0, const int32_t* perm) {
    if (it.e < 0) return;
    if (it.slot < 0 || it.slot >= a.num_slots) {
        if (threadIdx.x == 0 && n0 == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) zero_y_tile(a, n0, it.r0, it.r1);
        return;
    }
    skinny_body<FMT, MODE, KW, PERM_LDS>(a, it, n0, perm);
}

// The last workgroup of the down launch zeroes the y rows past offsets[E].
template <int FMT, int MODE, int KW>
__global__ __launch_bounds__(KW * 64) void ffn_skinny_kernel(FfnArgs a) {
    if (MODE == 1 && blockIdx.x == gridDim.x - 1) {
        zero_y_tail(a);
        return;
    }
    const int NT = (MODE == 0 ? a.f : a.d) / 16;
    run_item<FMT, MODE, KW>(a, find_item(a, blockIdx.x / NT), (blockIdx.x % NT) * 16, a.perm);
}

// ------------------------------------------------------------ routed gate/up

// Routing of a batch of at most kRoutedMaxPairs pairs, held in LDS.
constexpr int kRoutedMaxPairs = 64;
struct SmallRouting {
    int32_t ids[kRoutedMaxPairs];
    float w[kRoutedMaxPairs];
    int32_t perm[kRoutedMaxPairs];
    int32_t inv[kRoutedMaxPairs];
    int32_t offsets[kMaxExperts + 1];
};

// Stable counting sort of n <= 64 pairs by expert id, by one wave: pair p
// (lane p) goes to row (pairs with a smaller id) + (pairs with its id and a
// smaller index); offsets[x] = pairs with an id below x.  The same
// permutation as the dispatch kernel's for valid ids.
__device__ __forceinline__ void wave_dispatch(SmallRouting& r, int n, int E) {
    const int lane = threadIdx.x & 63;
    const int e = lane < n ? r.ids[lane] : 0x7fffffff;
    int before = 0, tie = 0, below_lane = 0;
    for (int q = 0; q < n; ++q) {
        const int eq = lane_value(e, q);
        before += eq < e;
        tie += (eq == e) & (q < lane);
        below_lane += eq < lane;
    }
    if (lane < n) {
        r.perm[before + tie] = lane;
        r.inv[lane] = before + tie;
    }
    if (lane < E) r.offsets[lane] = below_lane;
    if (lane == 0) r.offsets[E] = n;
}

// Gate/up launch of moe_layer for small batches: every workgroup routes the
// whole batch from the logits itself (top-k by one wave per token, then the
// one-wave counting sort: a few hundred instructions), so no routing launch
// and no read of routing results from HBM precede its weight loads.
// Workgroup 0 also writes ids, w, offsets, perm and inv and zeroes `out` for
// the down launch's scatter-add.  Arithmetic as topk_kernel and the dispatch
// kernel, so every output is identical.
template <int FMT>
__global__ __launch_bounds__(kGateUpWaves * 64) void ffn_gate_up_routed_kernel(FfnArgs a) {
    __shared__ SmallRouting r;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int T = a.T, E = a.E, k = a.k, n = a.T * a.k;
    int sl = lane;      // slot of expert `lane`, read before the routing is known
    if (lane < E && a.slot_of_expert) sl = a.slot_of_expert[lane];
    if (wave < T) topk_wave(a.logits + static_cast<size_t>(wave) * E, r.ids + wave * k, r.w + wave * k, E, k);
    __syncthreads();
    if (wave == 0) wave_dispatch(r, n, E);
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int i = tid; i < n; i += blockDim.x) {
            a.ids_out[i] = r.ids[i];
            a.w_out[i] = r.w[i];
            a.perm_out[i] = r.perm[i];
            a.inv_out[i] = r.inv[i];
        }
        for (int i = tid; i <= E; i += blockDim.x) a.offsets_out[i] = r.offsets[i];
        if (a.fuse_combine) {
            float4* o4 = reinterpret_cast<float4*>(a.out);
            for (int i = tid; i < T * a.d / 4; i += blockDim.x) o4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    int lo = 0, hi = 0;
    if (lane < E) {
        lo = r.offsets[lane];
        hi = r.offsets[lane + 1];
    }
    const int NT = a.f / 16;
    run_item<FMT, 0, kGateUpWaves, true>(a, pick_item(lo, hi, sl, blockIdx.x / NT), (blockIdx.x % NT) * 16, r.perm);
}

// ------------------------------------------------------------ launch


template <int FMT>
static hipError_t launch_two(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    const int umax = s.E < s.T * s.k ? s.E : s.T * s.k;
    ffn_skinny_kernel<FMT, 0, kGateUpWaves><<<umax * (s.f / 16), kGateUpWaves * 64, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_skinny_kernel<FMT, 1, kDownWaves><<<umax * (s.d / 16) + 1, kDownWaves * 64, 0, st>>>(a);
    return hipGetLastError();
}

// Token rows (T*k) from which the LDS-tiled grouped GEMM takes over.
constexpr int kGroupedMinRows = 256;

bool ffn_uses_grouped(const moe_shape& s, int fmt) {
    return s.T * s.k >= kGroupedMinRows && grouped_supported(s, fmt);
}

bool routed_ffn_supported(const moe_shape& s, int fmt) {
    return s.T <= kGateUpWaves && s.T * s.k <= kRoutedMaxPairs && !ffn_uses_grouped(s, fmt);
}

template <int FMT>
static hipError_t launch_two_routed(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    const int umax = s.E < s.T * s.k ? s.E : s.T * s.k;
    ffn_gate_up_routed_kernel<FMT><<<umax * (s.f / 16), kGateUpWaves * 64, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_skinny_kernel<FMT, 1, kDownWaves><<<umax * (s.d / 16) + 1, kDownWaves * 64, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_ffn_routed(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    return fmt == MOE_FMT_MXFP4 ? launch_two_routed<MOE_FMT_MXFP4>(s, a, st) : launch_two_routed<MOE_FMT_Q2G32>(s, a, st);
}

hipError_t launch_ffn(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    if (ffn_uses_grouped(s, fmt)) return launch_ffn_grouped(s, a, st);
    return fmt == MOE_FMT_MXFP4 ? launch_two<MOE_FMT_MXFP4>(s, a, st) : launch_two<MOE_FMT_Q2G32>(s, a, st);
}

}  // namespace qrmoe
