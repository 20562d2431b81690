// Expert FFN for many token rows per expert (prefill chunks): a grouped GEMM
// over the token-by-expert permutation.  MXFP4 weight tiles are dequantised
// to bf16 into LDS once per workgroup and reused by 128 token rows on the
// 32x32x16 bf16 matrix cores, with fp32 accumulation.  This is the
// block-sparse routed-expert computation of "antirez ds4: DeepSeek Metal
// inference" (section 技术深度解析) at prefill sizes: each activated expert's
// weights are read from HBM once per 128-token tile, inactive experts not at
// all.
//
// Workgroup = 4 waves, output tile = 128 token rows x 256 weight rows, K step 64:
//  * MODE 0 (gate/up + SwiGLU): weight rows are gate rows [n0, n0+128) then
//    up rows [n0, n0+128); wave w owns gate and up rows [n0+32w, n0+32w+32),
//    so silu(g)*u is formed in registers and act = bf16_rne(.) is stored.
//  * MODE 1 (down): weight rows [m0, m0+256) of W_d; wave w owns rows
//    [m0+64w, m0+64w+64); y is stored in fp32.
// Every wave covers all 128 token rows (four 32-wide MFMA column tiles); a
// column tile that holds only padding rows (past the expert's last row) is
// skipped, so a partial tile costs MFMA work in proportion to its rows.
//
// Pipeline: global loads run two K steps ahead into registers; the
// registers of step s+1 are dequantised into the other LDS buffer while
// step s is multiplied.  LDS rows are 128 bytes (64 bf16) with the 16-byte
// chunks XOR-swizzled by (row mod 8), so the 32 rows an MFMA operand read
// touches fall in distinct banks.
//
// Schedule: work units (expert, n-tile, m-tile) are enumerated with the m-tile
// fastest; consecutive units, which share a weight tile, go to the same XCD
// (workgroup ids are dealt round-robin over the 8 XCDs, so unit =
// xcd * units_per_xcd + id / 8).  Units are derived from offsets on the device.
#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kGM = 128;        // token rows per tile
constexpr int kGN = 256;        // weight rows per tile
constexpr int kGK = 64;         // K per step
constexpr int kGThreads = 256;
constexpr int kXcds = 8;

struct GStage {
    u32x4 w[2];     // 32 code bytes of this thread's weight row (two groups)
    uint32_t sc;    // their two e8m0 scales
    u32x4 x[4];     // 64 bytes of this thread's token row
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int MODE>
__global__ __launch_bounds__(kGThreads) void ffn_grouped_kernel(FfnArgs a) {
    __shared__ __align__(16) uint8_t wl[2][kGN * 128];
    __shared__ __align__(16) uint8_t xl[2][kGM * 128];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = MODE == 0 ? a.f : a.d;              // output columns of the projection
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
    const int per_xcd = ceil_div(total_units, kXcds);
    const int loc = blockIdx.x / kXcds;
    const int unit = (blockIdx.x % kXcds) * per_xcd + loc;
    if (loc >= per_xcd || unit >= total_units) return;
    const int excl = incl - mt;
    const uint64_t below = __ballot(mt > 0 && excl * NT <= unit);
    const int e = 63 - __clzll(static_cast<long long>(below));
    const int e_excl = __shfl(excl, e), e_mt = __shfl(mt, e);
    const int local = unit - e_excl * NT;
    const int nt = local / e_mt, mti = local % e_mt;
    const int r_base = a.offsets[e] + mti * kGM;
    const int nvalid = min(kGM, a.offsets[e + 1] - r_base);
    int slot = a.slot_of_expert ? a.slot_of_expert[e] : e;
    if (slot < 0 || slot >= a.num_slots) {
        if (tid == 0 && nt == 0 && mti == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) {
            for (int i = tid; i < nvalid * kGN; i += kGThreads)
                a.y[static_cast<size_t>(r_base + i / kGN) * a.d + nt * kGN + i % kGN] = 0.f;
        }
        return;
    }

    // ---- per-thread load roles
    // weight row `tid` of the 256-row tile
    const uint8_t* wcodes;
    const uint8_t* wscales;
    {
        int mat = 2, row = nt * kGN + tid;
        if (MODE == 0) {
            mat = tid < 128 ? 0 : 1;
            row = nt * 128 + (tid & 127);
        }
        const size_t grow = static_cast<size_t>(slot) * N + row;
        wcodes = a.codes[mat] + grow * (K / 2);
        wscales = a.scales[mat] + grow * (K / 32);
    }
    // token row j = tid / 2, half h = tid % 2 of the 128-byte K chunk
    const int xj = tid >> 1, xh = tid & 1;
    const bool xok = xj < nvalid;
    const uint16_t* xrow;
    if (MODE == 0) xrow = a.x + static_cast<size_t>(xok ? a.perm[r_base + xj] / a.k : 0) * a.d;
    else xrow = a.act + static_cast<size_t>(xok ? r_base + xj : 0) * a.f;

    auto gload = [&](GStage& st, int s) {
        const u32x4* cp = reinterpret_cast<const u32x4*>(wcodes + s * (kGK / 2));
        st.w[0] = cp[0];
        st.w[1] = cp[1];
        st.sc = *reinterpret_cast<const uint16_t*>(wscales + s * 2);
        const u32x4* xp = reinterpret_cast<const u32x4*>(xrow + s * kGK + xh * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) st.x[i] = xok ? xp[i] : u32x4{0u, 0u, 0u, 0u};
    };
    auto lstore = [&](int buf, const GStage& st) {
        uint8_t* wdst = wl[buf];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
            const float scl = e8m0_to_f32((st.sc >> (8 * gi)) & 0xffu);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bf16x8 v = mxfp4x8_to_bf16(st.w[gi][q], scl);
                *reinterpret_cast<bf16x8*>(wdst + swz(tid, gi * 4 + q)) = v;
            }
        }
        uint8_t* xdst = xl[buf];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(xdst + swz(xj, xh * 4 + i)) = st.x[i];
    };

    // ---- accumulators: [row tile][token tile]
    f32x16 acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;
    const int ntt = ceil_div(nvalid, 32);          // token tiles holding real rows
    // weight-tile rows of this wave's two 32-row MFMA tiles
    const int rt0 = MODE == 0 ? 32 * wave : 64 * wave;
    const int rt1 = MODE == 0 ? 128 + 32 * wave : 64 * wave + 32;

    // One K step: prefetch step s+2 into `mine`, multiply from LDS buffer
    // `cur`, dequantise step s+1 (held in `other`) into the other buffer.
    auto body = [&](int s, int cur, GStage& mine, GStage& other) {
        if (s + 2 < S) gload(mine, s + 2);
        const uint8_t* wb = wl[cur];
        const uint8_t* xb = xl[cur];
        const int r32 = lane & 31;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int chunk = 2 * kk + (lane >> 5);
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(wb + swz(rt0 + r32, chunk));
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(wb + swz(rt1 + r32, chunk));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t < ntt) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(xb + swz(32 * t + r32, chunk));
                    acc[0][t] = mfma32x32x16(a0, b, acc[0][t]);
                    acc[1][t] = mfma32x32x16(a1, b, acc[1][t]);
                }
            }
        }
        if (s + 1 < S) lstore(cur ^ 1, other);
        __syncthreads();
    };

    GStage st0, st1;
    gload(st0, 0);
    if (S > 1) gload(st1, 1);
    lstore(0, st0);
    __syncthreads();
    for (int s = 0; s < S; s += 2) {
        body(s, 0, st0, st1);
        if (s + 1 < S) body(s + 1, 1, st1, st0);
    }

    // ---- epilogue.  Lane l holds, for element i, weight row
    // 8*(i/4) + 4*(l/32) + i%4 of the 32-row tile and token row l%32.
    const int c32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int j = 32 * t + c32;
        if (t >= ntt || j >= nvalid) continue;
        const size_t r = static_cast<size_t>(r_base + j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = 8 * q + 4 * half;           // first of 4 consecutive rows
            if constexpr (MODE == 0) {
                uint32_t pk[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint16_t lo = f32_to_bf16_rne(silu_mul(acc[0][t][4 * q + 2 * h], acc[1][t][4 * q + 2 * h]));
                    const uint16_t hi = f32_to_bf16_rne(silu_mul(acc[0][t][4 * q + 2 * h + 1], acc[1][t][4 * q + 2 * h + 1]));
                    pk[h] = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
                }
                const int n = nt * 128 + 32 * wave + nl;
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
    return fmt == MOE_FMT_MXFP4 && s.f % 128 == 0 && s.d % kGN == 0 && s.d % kGK == 0 && s.f % kGK == 0;
}

hipError_t launch_ffn_grouped(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    const int pairs = s.T * s.k;
    const int max_mtiles = ceil_div(pairs, kGM) + (s.E < pairs ? s.E : pairs);
    const int units0 = max_mtiles * (s.f / 128);
    const int units1 = max_mtiles * (s.d / kGN);
    ffn_grouped_kernel<0><<<kXcds * ceil_div(units0, kXcds), kGThreads, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_grouped_kernel<1><<<kXcds * ceil_div(units1, kXcds), kGThreads, 0, st>>>(a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    zero_tail_rows_kernel<<<64, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace qrmoe
