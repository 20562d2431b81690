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
// Every wave covers all 128 token rows (four 32-wide MFMA column tiles); a
// column tile holding only padding rows (past the expert's last row) is
// skipped, so a partial tile costs MFMA work in proportion to its rows.
//
// Operands in LDS: the weight tile stays in its raw MXFP4 form, exactly as
// the tile layout stores it (include/moe.h, MOE_LAYOUT_TILES): a 64-element
// K step of a 16-row tile is half of one layout block, 32 pieces of 16 code
// bytes + 32 scale bytes, contiguous in HBM, so each thread copies whole
// pieces and each wave load instruction reads full cache lines.  A wave
// dequantises its own A fragment (gfx950 scaled fp4 -> bf16 conversion)
// right after reading it; the 64 lanes of that read cover two pieces arrays
// of 512 contiguous bytes (no bank conflicts).  The token tile is bf16 with
// its 16-byte chunks XOR-swizzled by (row / 2 mod 8) (see xswz).  K is permuted inside a
// step so that in sub-step kk lane half h (= lane/32) takes elements
// 32h + 8kk .. +8: a lane then reads one whole 32-element group (one piece:
// 16 code bytes, one scale) of the weight row and 64 contiguous bytes of the
// token row per step.
//
// Pipeline: global loads run four K steps ahead into a 4-slot register ring;
// after step s is multiplied, the slot of step s+1 is written to the other
// LDS buffer.  Every load is issued unconditionally (past-the-end steps
// reload the last step, padding token rows reload row 0 and are zeroed when
// written to LDS) and the loop is unrolled by the ring depth, so the compiler
// can wait for exactly the step it needs (s_waitcnt vmcnt(N)) instead of
// draining every prefetch.
//
// Schedule: work units (expert, m-tile, n-tile) are enumerated with the n-tile
// fastest and unit = workgroup id.  Workgroup ids are dealt round-robin over
// the 8 XCDs, and there are 8 n-tiles at the workload's shape, so an XCD
// works through one n-tile of every m-tile: consecutive m-tiles of a hot
// expert reuse the same weight tile from that XCD's L2, and the heavy units
// of hot experts are spread evenly over all XCDs (handing out contiguous
// ranges of units per XCD instead put a whole hot expert on one XCD and was
// measured ~1.5x slower).  Units are derived from offsets on the device.
#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kGM = 128;        // token rows per tile
constexpr int kGN = 512;        // weight rows per tile
constexpr int kGK = 64;         // K per step
constexpr int kGWaves = 8;
constexpr int kGThreads = kGWaves * 64;

struct GSlot {
    u32x4 w[2];     // pieces p and 16+p of this thread's tile for the step
    uint32_t sc;    // the scale bytes of pieces 2p and 2p+1
    u32x4 x[2];     // 32 bytes of this thread's token row quarter
};

// Byte offset of 16-byte chunk `chunk` (0..7) of token row `row` (128 B) in
// the token tile.  gfx950's LDS serves 256 B per cycle (64 four-byte banks),
// i.e. one ds_read_b128 phase is 16 lanes; XOR-ing the chunk with
// (row / 2) % 8 puts any 16 consecutive rows at the same logical chunk into
// 16 distinct bank groups (row parity picks the half of the 256 B, the
// swizzled chunk the 16 B within it).  (The XOR with row % 8, right for
// 128 B per cycle, left a 2-way conflict on every read: rows r and r+8.)
__device__ __forceinline__ int xswz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

template <int MODE>
__global__ __launch_bounds__(kGThreads) void ffn_grouped_kernel(FfnArgs a) {
    __shared__ __align__(16) uint8_t wl[2][kGN * 32];   // codes [tile][piece][16 B]
    __shared__ __align__(16) uint8_t sl[2][kGN * 2];    // e8m0 [tile][piece]
    __shared__ __align__(16) uint8_t xl[2][kGM * 128];  // bf16 tokens [row][64], swizzled

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int NT = MODE == 0 ? a.f / (kGN / 2) : a.d / kGN;
    const int S = K / kGK;

    // ---- schedule: expert / m-tile / n-tile of this workgroup
    int cnt = 0;
    if (lane < a.E) cnt = a.offsets[lane + 1] - a.offsets[lane];
    const int mt = ceil_div(cnt, kGM);
    int incl = mt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    const int total_units = __shfl(incl, 63) * NT;
    const int unit = blockIdx.x;
    if (unit >= total_units) return;
    const int excl = incl - mt;
    const uint64_t below = __ballot(mt > 0 && excl * NT <= unit);
    const int e = 63 - __clzll(static_cast<long long>(below));
    const int e_excl = __shfl(excl, e), e_mt = __shfl(mt, e);
    const int local = unit - e_excl * NT;
    const int mti = local / NT, nt = local % NT;
    const int r_base = a.offsets[e] + mti * kGM;
    const int nvalid = min(kGM, a.offsets[e + 1] - r_base);
    const int slot = a.slot_of_expert ? a.slot_of_expert[e] : e;
    if (slot < 0 || slot >= a.num_slots) {
        if (tid == 0 && nt == 0 && mti == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) {
            for (int i = tid; i < nvalid * kGN; i += kGThreads)
                a.y[static_cast<size_t>(r_base + i / kGN) * a.d + nt * kGN + i % kGN] = 0.f;
        }
        return;
    }

    // ---- per-thread load roles: pieces p and 16+p (p = tid%16) of 16-row
    // tile tid/16 of the workgroup's 32; token row tid/4, quarter tid%4 (16
    // bf16) of the step's 64 K elements.
    const int wt = tid >> 4, wp = tid & 15;
    const uint8_t* wcodes;
    const uint8_t* wscales;
    {
        int mat = 2, tile = nt * (kGN / 16) + wt;
        if (MODE == 0) {
            mat = wt < kGN / 32 ? 0 : 1;
            tile = nt * (kGN / 32) + (wt & (kGN / 32 - 1));
        }
        const size_t blk = (static_cast<size_t>(slot) * (N / 16) + tile) * (K / 128);
        wcodes = a.codes[mat] + blk * 64 * 16 + wp * 16;
        wscales = a.scales[mat] + blk * 64 + 2 * wp;
    }
    const int xj = tid >> 2, xq = tid & 3;
    const bool xok = xj < nvalid;
    const uint16_t* xrow;    // padding rows read row 0 (always valid) and store zeros
    if (MODE == 0) xrow = a.x + static_cast<size_t>(xok ? a.perm[r_base + xj] / a.k : 0) * a.d;
    else xrow = a.act + static_cast<size_t>(xok ? r_base + xj : r_base) * a.f;

    // step s of 64 elements = half s%2 of layout block s/2 (pieces 32*(s%2) ..)
    auto gload = [&](GSlot& g, int s) {
        s = min(s, S - 1);
        const size_t half = static_cast<size_t>(s >> 1) * 64 + 32 * (s & 1);
        const u32x4* cp = reinterpret_cast<const u32x4*>(wcodes + half * 16);
        g.w[0] = cp[0];
        g.w[1] = cp[16];
        g.sc = *reinterpret_cast<const uint16_t*>(wscales + half);
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + s * kGK + xq * 16);
        g.x[0] = xp[0];
        g.x[1] = xp[1];
    };
    auto lstore = [&](int buf, const GSlot& g) {
        u32x4* wd = reinterpret_cast<u32x4*>(wl[buf] + wt * 512 + wp * 16);
        wd[0] = g.w[0];
        wd[16] = g.w[1];
        *reinterpret_cast<uint16_t*>(&sl[buf][wt * 32 + 2 * wp]) = static_cast<uint16_t>(g.sc);
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(xl[buf] + xswz(xj, 2 * xq)) = xok ? g.x[0] : z;
        *reinterpret_cast<u32x4*>(xl[buf] + xswz(xj, 2 * xq + 1)) = xok ? g.x[1] : z;
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;
    // uniform in the workgroup: scalar branches on the column tiles below
    const int ntt = __builtin_amdgcn_readfirstlane(ceil_div(nvalid, 32));
    const int rt0 = MODE == 0 ? 32 * wave : 64 * wave;
    const int rt1 = MODE == 0 ? kGN / 2 + 32 * wave : 64 * wave + 32;
    const int r32 = lane & 31, h = lane >> 5;

    // LDS piece index of weight row rt + r32, local group h
    const int pc0 = (rt0 / 16 + (r32 >> 4)) * 32 + 16 * h + (r32 & 15);
    const int pc1 = (rt1 / 16 + (r32 >> 4)) * 32 + 16 * h + (r32 & 15);
    auto compute = [&](int buf) {
        const uint8_t* wb = wl[buf];
        const u32x4 c0 = *reinterpret_cast<const u32x4*>(wb + pc0 * 16);
        const u32x4 c1 = *reinterpret_cast<const u32x4*>(wb + pc1 * 16);
        const float s0 = e8m0_to_f32(sl[buf][pc0]);
        const float s1 = e8m0_to_f32(sl[buf][pc1]);
        const uint8_t* xb = xl[buf];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 a0 = mxfp4x8_to_bf16(c0[kk], s0);
            const bf16x8 a1 = mxfp4x8_to_bf16(c1[kk], s1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t < ntt) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(xb + xswz(32 * t + r32, 4 * h + kk));
                    acc[0][t] = mfma32x32x16(a0, b, acc[0][t]);
                    acc[1][t] = mfma32x32x16(a1, b, acc[1][t]);
                }
            }
        }
    };

    // Iteration s: multiply LDS buffer s%2, write ring slot (s+1)%4 (step s+1,
    // loaded four iterations earlier) into LDS buffer (s+1)%2, then refill
    // ring slot s%4 with step s+4.  S is a multiple of 4.
    GSlot g0, g1, g2, g3;
    gload(g0, 0);
    gload(g1, 1);
    gload(g2, 2);
    gload(g3, 3);
    lstore(0, g0);
    __syncthreads();
    auto iter = [&](int s, GSlot& mine, GSlot& next, int buf) {
        compute(buf);
        lstore(buf ^ 1, next);
        gload(mine, s + 4);
        __syncthreads();
    };
    for (int s = 0; s < S; s += 4) {
        iter(s, g0, g1, 0);
        iter(s + 1, g1, g2, 1);
        iter(s + 2, g2, g3, 0);
        iter(s + 3, g3, g0, 1);
    }

    // ---- epilogue.  Lane l holds, for element i, weight row
    // 8*(i/4) + 4*(l/32) + i%4 of the 32-row tile and token row l%32.
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
                *reinterpret_cast<u32x2*>(a.act + r * a.f + n) = u32x2{pk[0], pk[1]};
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
}

__global__ void zero_tail_rows_kernel(FfnArgs a) {
    const int r_lo = a.offsets[a.E], r_hi = a.T * a.k;
    const int n4 = a.d / 4;
    float4* base = reinterpret_cast<float4*>(a.y + static_cast<size_t>(r_lo) * a.d);
    const long long total = static_cast<long long>(r_hi - r_lo) * n4;
    for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < total;
         i += static_cast<long long>(gridDim.x) * blockDim.x)
        base[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

bool grouped_supported(const moe_shape& s, int fmt) {
    return fmt == MOE_FMT_MXFP4 && s.f % (kGN / 2) == 0 && s.d % kGN == 0;
}

hipError_t launch_ffn_grouped(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    const int pairs = s.T * s.k;
    const int max_mtiles = ceil_div(pairs, kGM) + (s.E < pairs ? s.E : pairs);
    const int units0 = max_mtiles * (s.f / (kGN / 2));
    const int units1 = max_mtiles * (s.d / kGN);
    ffn_grouped_kernel<0><<<units0, kGThreads, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_grouped_kernel<1><<<units1, kGThreads, 0, st>>>(a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    zero_tail_rows_kernel<<<64, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace qrmoe
