// Router logits and top-k selection with renormalised softmax weights.
//
// The router scores every token against every expert in full float32
// precision (the ds4 guide, section "避坑指南", reports that quantised routers
// collapse quality); the top-k experts per token are kept ("antirez ds4:
// DeepSeek Metal inference", section 技术深度解析: top-2 of 64).
//
// Kernels:
//   router_rows_kernel  small T: one workgroup per expert streams W_r[e] once
//                       and dots it with every token (T <= kRowsMaxT).
//   router_mfma_kernel  large T: 32 tokens x 16 experts per workgroup, eight
//                       waves splitting K; float32 scores from three bf16
//                       parts of W_r on the bf16 matrix cores.
//   topk_kernel         one wave64 per token, lane = expert.
#include "common.hpp"
#include "kernels.hpp"
#include "topk_dev.hpp"

namespace qrmoe {

constexpr int kRowsMaxT = 8;
constexpr int kRowsThreads = 512;

// logits[t][e] for t in [t0, t0 + nt) of one expert (nt = min(NT, T - t0)),
// by one workgroup of kRowsThreads threads.  Thread i handles elements
// 8*i .. 8*i+7 of each 8*512-element chunk of d (one chunk at d = 4096: one
// round of loads); the loads of all NT token rows are issued together (rows
// past nt repeat the last one; their sums are never stored), so a batch of
// tokens costs one load latency, not one per token.  The partial sums are
// reduced in a fixed order within each wave (DPP shifts and broadcasts,
// wave_sum_f32), then across the waves in wave order.
template <int NT>
__device__ __forceinline__ void router_rows_block(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                  const float* __restrict__ bias, float* __restrict__ logits,
                                                  int e, int t0, int T, int d, int E) {
    const int nt = min(NT, T - t0);
    const float* wrow = wr + static_cast<size_t>(e) * d;
    const uint16_t* xrow[NT];
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        xrow[j] = x + static_cast<size_t>(t0 + min(j, nt - 1)) * d;
        acc[j] = 0.f;
    }
#pragma unroll 2
    for (int i = threadIdx.x * 8; i < d; i += kRowsThreads * 8) {
        const float4 w0 = *reinterpret_cast<const float4*>(wrow + i);
        const float4 w1 = *reinterpret_cast<const float4*>(wrow + i + 4);
        u32x4 xv[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) xv[j] = *reinterpret_cast<const u32x4*>(xrow[j] + i);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            float s = acc[j];
            s = fmaf(bf16lo(xv[j][0]), w0.x, s);
            s = fmaf(bf16hi(xv[j][0]), w0.y, s);
            s = fmaf(bf16lo(xv[j][1]), w0.z, s);
            s = fmaf(bf16hi(xv[j][1]), w0.w, s);
            s = fmaf(bf16lo(xv[j][2]), w1.x, s);
            s = fmaf(bf16hi(xv[j][2]), w1.y, s);
            s = fmaf(bf16lo(xv[j][3]), w1.z, s);
            s = fmaf(bf16hi(xv[j][3]), w1.w, s);
            acc[j] = s;
        }
    }
    __shared__ float part[kRowsThreads / kWave][kRowsMaxT];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const float s = wave_sum_f32(acc[j]);
        if (lane == 0) part[wave][j] = s;
    }
    __syncthreads();
    if (threadIdx.x < nt) {
        const int j = threadIdx.x;
        float s = part[0][j];
#pragma unroll
        for (int w = 1; w < kRowsThreads / kWave; ++w) s += part[w][j];
        if (bias) s += bias[e];
        logits[static_cast<size_t>(t0 + j) * E + e] = s;
    }
}

template <int NT>
__global__ __launch_bounds__(kRowsThreads) void router_rows_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
    router_rows_block<NT>(x, wr, bias, logits, blockIdx.x, blockIdx.y * NT, T, d, E);
}

// Large-T router.  Workgroup = 8 waves = 32 tokens x 16 experts, one
// workgroup per CU at T = 2048, E = 64; the waves split K eight ways and their
// partial tiles are summed in LDS in wave order.
//
// The scores stay float32 but run on the bf16 matrix cores: x is bf16
// already, and each W_r element is split in registers into three bf16 parts
// hi + mid + lo (hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid);
// each subtraction is exact in fp32 and each part takes the next 8
// significant bits, so the parts sum to w within 2^-24 relative).  A bf16 x
// bf16 product is exact in fp32, so x * w is formed exactly as three
// products and only the fp32 accumulation of the 16x16x32 MFMAs rounds --
// the accuracy of a float32 dot product at three bf16 MFMAs per K step of 32
// instead of eight fp32 16x16x4 ones (a sixteenth of the bf16 rate each).
//
// In a K step of 32, lane group g (= lane / 16) supplies elements 8g .. 8g+7
// of its token row (one 16-byte load) and of its expert row (two), so the
// MFMA operands come straight from the loads.  Loads run one batch of
// kRouterBatch steps ahead of the multiplies (two register sets); they are
// unconditional (addresses clamped, values masked), so each batch's loads
// are in flight together.
constexpr int kRouterWaves = 8;
constexpr int kRouterBatch = 4;
constexpr int kRouterTokens = 32;
constexpr int kRouterStep = 32;

// Splits eight floats into three bf16x8 parts whose sum is the floats to
// within 2^-24 relative (see above), two elements per packed conversion
// (round to nearest even).
__device__ __forceinline__ void split3_bf16(const float4& a, const float4& b, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    u32x4 ph, pm, pl;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x2 w{v[2 * p], v[2 * p + 1]};
        const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf16x2));
        const f32x2 r1{w[0] - __uint_as_float(h << 16), w[1] - __uint_as_float(h & 0xffff0000u)};
        const uint32_t m = __builtin_bit_cast(uint32_t, __builtin_convertvector(r1, bf16x2));
        const f32x2 r2{r1[0] - __uint_as_float(m << 16), r1[1] - __uint_as_float(m & 0xffff0000u)};
        ph[p] = h;
        pm[p] = m;
        pl[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
    }
    hi = bf16x8_from_u32x4(ph);
    mid = bf16x8_from_u32x4(pm);
    lo = bf16x8_from_u32x4(pl);
}

__global__ __launch_bounds__(kRouterWaves * 64) void router_mfma_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
    __shared__ __align__(16) f32x4 red[kRouterWaves][2][kWave];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kRouterTokens, e0 = blockIdx.y * 16;
    const int row = lane & 15, g = lane >> 4;
    const int ex = e0 + row;
    const bool ex_ok = ex < E;
    const uint16_t* xr[2];
    bool tok_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tok = t0 + 16 * h + row;
        tok_ok[h] = tok < T;
        xr[h] = x + static_cast<size_t>(tok_ok[h] ? tok : 0) * d + 8 * g;
    }
    const float* wrow = wr + static_cast<size_t>(ex_ok ? ex : 0) * d + 8 * g;
    const int S = d / kRouterStep;
    const int s_beg = (S * wave) / kRouterWaves, s_end = (S * (wave + 1)) / kRouterWaves;
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float4 wv[2][kRouterBatch][2];
    u32x4 xv[2][kRouterBatch][2];
    auto load = [&](int buf, int sb) {
#pragma unroll
        for (int u = 0; u < kRouterBatch; ++u) {
            const int s = max(min(sb + u, s_end - 1), 0);
            wv[buf][u][0] = *reinterpret_cast<const float4*>(wrow + kRouterStep * s);
            wv[buf][u][1] = *reinterpret_cast<const float4*>(wrow + kRouterStep * s + 4);
#pragma unroll
            for (int h = 0; h < 2; ++h) xv[buf][u][h] = *reinterpret_cast<const u32x4*>(xr[h] + kRouterStep * s);
        }
    };
    auto mul = [&](int buf, int sb) {
#pragma unroll
        for (int u = 0; u < kRouterBatch; ++u) {
            // Only the token operand is masked, on steps past the slice: a
            // reloaded step then adds x = 0 times a finite weight.  Lanes
            // of tokens >= T or experts >= E read clamped rows; their
            // output rows and columns are never stored.
            const bool ok = sb + u < s_end;
            bf16x8 hi, mid, lo;
            split3_bf16(wv[buf][u][0], wv[buf][u][1], hi, mid, lo);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8 xx = ok ? bf16x8_from_u32x4(xv[buf][u][h]) : bf16x8_zero();
                // A = x (16 tokens x 32), B = W_r^T (32 x 16 experts)
                acc[h] = mfma16x16x32(xx, hi, acc[h]);
                acc[h] = mfma16x16x32(xx, mid, acc[h]);
                acc[h] = mfma16x16x32(xx, lo, acc[h]);
            }
        }
    };
    // two register sets: batch b + 1 loads while batch b multiplies (the
    // loop is unrolled by two so that every set index is a constant).  The
    // loop body holds no load under a branch, so the compiler's waits before
    // each batch's products count only the loads ahead of it; a batch load
    // under a branch made them wait for the next batch too (prefill router
    // 314.8 -> 312.7 us per layer step, four alternating runs, one box)
    load(0, s_beg);
    int sb = s_beg;
    for (; sb + 2 * kRouterBatch < s_end; sb += 2 * kRouterBatch) {
        load(1, sb + kRouterBatch);
        mul(0, sb);
        load(0, sb + 2 * kRouterBatch);
        mul(1, sb + kRouterBatch);
    }
    if (sb + kRouterBatch < s_end) {
        load(1, sb + kRouterBatch);
        mul(0, sb);
        mul(1, sb + kRouterBatch);
    } else if (sb < s_end) {
        mul(0, sb);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) red[wave][h][lane] = acc[h];
    __syncthreads();
    // acc[h][i] of lane l = C[token 16h + 4(l/16) + i][expert l%16]
    for (int idx = threadIdx.x; idx < 2 * 256; idx += kRouterWaves * 64) {
        const int h = idx >> 8, l = (idx >> 2) & 63, i = idx & 3;
        float v = red[0][h][l][i];
#pragma unroll
        for (int w = 1; w < kRouterWaves; ++w) v += red[w][h][l][i];
        const int t = t0 + 16 * h + 4 * (l >> 4) + i, e = e0 + (l & 15);
        if (t < T && e < E) logits[static_cast<size_t>(t) * E + e] = v + (bias ? bias[e] : 0.f);
    }
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w, int T, int E, int k) {
    const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave(logits + static_cast<size_t>(t) * E, ids + static_cast<size_t>(t) * k,
              w + static_cast<size_t>(t) * k, E, k);
}

// Top-k and dispatch of a small batch (T <= kSmallRouteT tokens, T*k <=
// kRoutedMaxPairs pairs) in one workgroup: one wave per token for the top-k,
// then the one-wave stable counting sort in LDS.  The arithmetic of
// topk_kernel and of the dispatch kernel (whose permutation the counting sort
// reproduces for valid ids, and top-k ids are always valid), so every output
// is identical; one launch instead of two.
constexpr int kSmallRouteT = 16;

__global__ __launch_bounds__(kSmallRouteT * 64) void small_route_kernel(
    const float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv, int T, int E, int k,
    int shared) {
    __shared__ SmallRouting r;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int n = T * k;
    if (wave < T) topk_wave(logits + static_cast<size_t>(wave) * E, r.ids + wave * k, r.w + wave * k, E, k);
    __syncthreads();
    if (wave == 0) wave_dispatch(r, n, E);
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
        ids[i] = r.ids[i];
        w[i] = r.w[i];
        perm[i] = r.perm[i];
        inv[i] = r.inv[i];
    }
    for (int i = tid; i <= E; i += blockDim.x) offsets[i] = r.offsets[i];
    if (shared && tid < T) perm[n + tid] = tid * k;       // the shared expert's rows
}

bool small_route_supported(const moe_shape& s) { return s.T <= kSmallRouteT && s.T * s.k <= kRoutedMaxPairs; }

hipError_t launch_small_route(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                              float* logits, int32_t* ids, float* w, int32_t* offsets, int32_t* perm,
                              int32_t* inv, hipStream_t st, bool shared) {
    if (wr) {
        const hipError_t err = launch_router_logits(s, x, wr, bias, logits, st);
        if (err != hipSuccess) return err;
    }
    small_route_kernel<<<1, kSmallRouteT * 64, 0, st>>>(logits, ids, w, offsets, perm, inv, s.T, s.E, s.k,
                                                        shared ? 1 : 0);
    return hipGetLastError();
}

template <int NT>
static void launch_rows(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias, float* logits,
                        hipStream_t st) {
    router_rows_kernel<NT><<<dim3(s.E, ceil_div(s.T, NT)), kRowsThreads, 0, st>>>(x, wr, bias, logits, s.T, s.d, s.E);
}

hipError_t launch_router_logits(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                                float* logits, hipStream_t st) {
    if (s.T <= 0) return hipSuccess;
    // token rows per workgroup: the batch itself up to kRowsMaxT
    switch (s.T < kRowsMaxT ? s.T : kRowsMaxT) {
        case 1: launch_rows<1>(s, x, wr, bias, logits, st); break;
        case 2: launch_rows<2>(s, x, wr, bias, logits, st); break;
        case 3: launch_rows<3>(s, x, wr, bias, logits, st); break;
        case 4: launch_rows<4>(s, x, wr, bias, logits, st); break;
        case 5: launch_rows<5>(s, x, wr, bias, logits, st); break;
        case 6: launch_rows<6>(s, x, wr, bias, logits, st); break;
        case 7: launch_rows<7>(s, x, wr, bias, logits, st); break;
        default: launch_rows<kRowsMaxT>(s, x, wr, bias, logits, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_route(const moe_shape& s, const uint16_t* x, const float* wr, const float* bias,
                        float* logits, int32_t* ids, float* w, hipStream_t st) {
    if (wr) {
        if (s.T <= 4 * kRowsMaxT) {
            const hipError_t err = launch_router_logits(s, x, wr, bias, logits, st);
            if (err != hipSuccess) return err;
        } else {
            router_mfma_kernel<<<dim3(ceil_div(s.T, kRouterTokens), ceil_div(s.E, 16)), kRouterWaves * 64, 0, st>>>(
                x, wr, bias, logits, s.T, s.d, s.E);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    topk_kernel<<<ceil_div(s.T, 4), 256, 0, st>>>(logits, ids, w, s.T, s.E, s.k);
    return hipGetLastError();
}

}  // namespace qrmoe
