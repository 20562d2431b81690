// Expert FFN for few token rows per expert (decode, speculative verify,
// short batches).  Each activated expert's quantised weights are streamed
// from HBM once and dequantised in registers ("antirez ds4: DeepSeek Metal
// inference", section 技术深度解析: the block-sparse routed-expert kernel loads
// only the activated experts' weights and dequantises them on the fly).
//
// Work item = (active expert, tile of 16 weight rows); the waves of a
// workgroup split K and their partial tiles are summed in LDS in a fixed wave
// order (deterministic).  The active expert of an item is found on the device
// from offsets[E+1]; there is no host round trip.
//
// Two launches: gate/up + SwiGLU (act to the workspace), then down (y).  A
// single persistent kernel with a grid barrier between the projections was
// measured slower on MI355X: a cooperative launch alone costs ~20 us and a
// 256-workgroup barrier 8-14 us, more than the whole down projection.
#include "common.hpp"
#include "ffn_tile.hpp"
#include "kernels.hpp"

namespace qrmoe {

template <int MODE>
struct ModeDims {
    static constexpr int NM = MODE == 0 ? 2 : 1;
};

// One work item: 16 weight rows starting at n0 of expert slot `slot`, all of
// the expert's token rows [r0, r1).  Wave w of KW handles K steps
// [S*w/KW, S*(w+1)/KW).  `pre` (when has_pre) holds this wave's first weight
// chunk, loaded earlier.
template <int FMT, int MODE, int KW>
__device__ __forceinline__ void run_item(const FfnArgs& a, int slot, int n0, int r0, int r1,
                                         f32x4 (*red)[ModeDims<MODE>::NM][kWave], Q2Lds* q2,
                                         const WChunk<FMT> (&pre)[ModeDims<MODE>::NM], bool has_pre) {
    constexpr int NM = ModeDims<MODE>::NM;
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int G = K / kGroup;
    const int S = ceil_div(G, 4);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int row = lane & 15, g = lane >> 4;
    const int s_beg = (S * wave) / KW, s_end = (S * (wave + 1)) / KW;
    const int nk = ceil_div(s_end - s_beg, kCap);

    WRow wr[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int mat = MODE == 0 ? m : 2;
        wr[m] = wrow<FMT>(a.codes[mat], a.scales[mat], a.mins[mat], static_cast<size_t>(slot) * N + n0 + row, K);
    }
    WChunk<FMT> w[NM];
    if (nk == 1) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (has_pre) w[m] = pre[m];
            else load_w<FMT>(w[m], wr[m], s_beg, s_end, G, g);
        }
    }
    for (int c0 = r0; c0 < r1; c0 += 16) {
        const int r = c0 + row;
        const bool colok = r < r1;
        const uint16_t* brow;
        if (MODE == 0) brow = a.x + static_cast<size_t>(colok ? a.perm[r] / a.k : 0) * a.d;
        else brow = a.act + static_cast<size_t>(colok ? r : 0) * a.f;
        f32x4 acc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kc = 0; kc < nk; ++kc) {
            const int s0 = s_beg + kc * kCap;
            if (nk > 1) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    if (has_pre && kc == 0 && c0 == r0) w[m] = pre[m];
                    else load_w<FMT>(w[m], wr[m], s0, s_end, G, g);
                }
            }
            u32x4 bv[kCap][4];
            load_b<FMT>(bv, brow, colok, s0, s_end, G, g);
            mma_chunk<FMT, NM>(acc, w, bv, q2 + wave * NM);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) red[wave][m][lane] = acc[m];
        __syncthreads();
        for (int idx = tid; idx < 16 * 16; idx += KW * kWave) {
            const int col = idx >> 4, nn = idx & 15;
            const int src = col + 16 * (nn >> 2), i = nn & 3;
            const int rr = c0 + col;
            if (rr < r1) {
                float v[NM];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    float s = red[0][m][src][i];
#pragma unroll
                    for (int ww = 1; ww < KW; ++ww) s += red[ww][m][src][i];
                    v[m] = s;
                }
                const int n = n0 + nn;
                if constexpr (MODE == 0) {
                    a.act[static_cast<size_t>(rr) * a.f + n] = f32_to_bf16_rne(silu_mul(v[0], v[NM - 1]));
                } else {
                    a.y[static_cast<size_t>(rr) * a.d + n] = v[0];
                    if (a.fuse_combine) {
                        // scatter-add of the weighted expert output; with at
                        // most two addends on a zeroed out the sum does not
                        // depend on their order (it equals the combine kernel's)
                        const int p = a.perm[rr];
                        atomicAdd(a.out + static_cast<size_t>(p / a.k) * a.d + n, __fmul_rn(a.topk_w[p], v[0]));
                    }
                }
            }
        }
        __syncthreads();
    }
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

struct ItemRef {
    int e, slot, r0, r1, n0;
    bool slot_ok;
};

// Work item `item` of a projection with `ntiles` 16-row tiles per expert.
__device__ __forceinline__ ItemRef item_ref(const FfnArgs& a, int item, int ntiles) {
    ItemRef it;
    const int ai = item / ntiles;
    it.n0 = (item % ntiles) * 16;
    it.e = nth_active_expert(a.offsets, a.E, ai);
    it.r0 = it.r1 = it.slot = 0;
    it.slot_ok = false;
    if (it.e < 0) return it;
    it.r0 = a.offsets[it.e];
    it.r1 = a.offsets[it.e + 1];
    it.slot = a.slot_of_expert ? a.slot_of_expert[it.e] : it.e;
    it.slot_ok = it.slot >= 0 && it.slot < a.num_slots;
    return it;
}

__device__ __forceinline__ int active_count(const int32_t* offsets, int E) {
    const int lane = threadIdx.x & 63;
    const int cnt = lane < E ? offsets[lane + 1] - offsets[lane] : 0;
    return __popcll(__ballot(cnt > 0));
}

// ------------------------------------------------------------ two launches

template <int FMT, int MODE, int KW>
__global__ __launch_bounds__(KW * 64) void ffn_skinny_kernel(FfnArgs a) {
    constexpr int NM = ModeDims<MODE>::NM;
    __shared__ __align__(16) f32x4 red[KW][NM][kWave];
    __shared__ __align__(16) Q2Lds q2[FMT == MOE_FMT_Q2G32 ? KW * NM : 1];
    if (MODE == 1 && blockIdx.x == gridDim.x - 1) {
        zero_y_tail(a);
        return;
    }
    const int ntiles = (MODE == 0 ? a.f : a.d) / 16;
    const ItemRef it = item_ref(a, blockIdx.x, ntiles);
    if (it.e < 0) return;
    if (!it.slot_ok) {
        if (threadIdx.x == 0 && it.n0 == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) zero_y_tile(a, it.n0, it.r0, it.r1);
        return;
    }
    WChunk<FMT> none[NM];
    run_item<FMT, MODE, KW>(a, it.slot, it.n0, it.r0, it.r1, red, q2, none, false);
}

// ------------------------------------------------------------ launch

// Waves per workgroup (K split): gate/up K = d, down K = f.  With d = 4096 /
// f = 2048 every wave holds its whole K slice (4 steps) in registers, so all
// of a workgroup's weight loads are in flight at once.
constexpr int kGateUpWaves = 8;
constexpr int kDownWaves = 4;

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

hipError_t launch_ffn(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    if (ffn_uses_grouped(s, fmt)) return launch_ffn_grouped(s, a, st);
    return fmt == MOE_FMT_MXFP4 ? launch_two<MOE_FMT_MXFP4>(s, a, st) : launch_two<MOE_FMT_Q2G32>(s, a, st);
}

}  // namespace qrmoe
