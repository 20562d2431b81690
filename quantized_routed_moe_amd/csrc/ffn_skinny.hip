// Expert FFN for few rows per expert (decode, speculative verify, short
// batches): streams each activated expert's quantised weights from HBM once,
// dequantises them in registers and multiplies them against at most 16 token
// rows at a time on the matrix cores.
//
// This is the block-sparse routed-expert kernel of "antirez ds4: DeepSeek
// Metal inference" (section 技术深度解析: only the activated experts'
// weights are loaded, dequantised on the fly), re-designed for gfx950:
//
//  * Work item = (active expert, tile of 16*NT weight rows).  The active
//    expert is found on the device from offsets[E+1] (no host round trip);
//    blocks past the number of active experts exit at once.
//  * A workgroup of KSPLIT waves splits K; each wave reads 16-byte code
//    chunks (one 32-element group per lane) straight into registers, and the
//    partial 16x16 tiles are summed across waves in LDS in a fixed order.
//  * MFMA 16x16x32 bf16 with the weights as the A operand (16 weight rows)
//    and up to 16 token rows as the B operand; fp32 accumulation.
//
// MXFP4 (A6 of the pages' formats): the gfx950 scaled fp4->bf16 conversion
// applies the e8m0 scale exactly, so the bf16 A operand is the exact weight.
// In MFMA j of a K step, lane group g (= lane/16) supplies elements 8j..8j+7
// of group 4s+g, and the token operand supplies the same elements of x.
//
// Q2 (2-bit group-asymmetric, w = scale*q + min): a bf16 operand cannot hold
// scale*q + min exactly, so each MFMA covers ONE group (all four lane groups
// supply slices of the same group) with A = bf16(1 + q/4), which is exact
// (bit pattern 0x3F80 | q << 5).  With C = sum (1 + q/4) x and xs = sum x
// over the group (a second MFMA against a ones operand), the group's
// contribution is
//     (4*scale)*C + (min - 4*scale)*xs  ==  sum (scale*q + min) x,
// added in fp32.  (An offset of 1 rather than a larger power of two keeps
// the cancellation between C and xs, and so the rounding error, small.)  The code bytes and per-row scale/min are re-laid through a
// wave-private LDS area so that every lane finds the slice it needs.
//
// MODE 0: gate and up (N = f, K = d, token operand = x rows gathered by
//         perm), epilogue act = bf16_rne(silu(g) * u).
// MODE 1: down (N = d, K = f, token operand = act rows), epilogue y (fp32);
//         the extra last workgroup zeroes y rows at or past offsets[E].
#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kUnroll = 4;

template <int FMT, int MODE, int KSPLIT, int NT>
__global__ __launch_bounds__(KSPLIT * 64) void ffn_skinny_kernel(FfnArgs a) {
    constexpr int NMAT = MODE == 0 ? 2 : 1;
    constexpr int NTILE = NMAT * NT;
    const int N = MODE == 0 ? a.f : a.d;
    const int K = MODE == 0 ? a.d : a.f;
    const int G = K / kGroup;
    const int S = ceil_div(G, 4);
    const int ntiles = N / (16 * NT);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    __shared__ __align__(16) f32x4 red[KSPLIT][NTILE][kWave];
    // Q2 only: wave-private re-layout areas
    __shared__ __align__(16) u32x2 q2codes[FMT == MOE_FMT_Q2G32 ? KSPLIT : 1][NTILE][16][4];
    __shared__ __align__(16) float2 q2sm[FMT == MOE_FMT_Q2G32 ? KSPLIT : 1][NTILE][4][16];

    if (MODE == 1 && blockIdx.x == gridDim.x - 1) {
        // rows past offsets[E] (pairs with an invalid expert id) read as zero
        const int r_lo = a.offsets[a.E], r_hi = a.T * a.k;
        const int n4 = a.d / 4;
        for (long long i = tid; i < static_cast<long long>(r_hi - r_lo) * n4; i += blockDim.x)
            reinterpret_cast<float4*>(a.y + static_cast<size_t>(r_lo) * a.d)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }

    const int ai = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
    const int e = nth_active_expert(a.offsets, a.E, ai);
    if (e < 0) return;
    const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
    const int slot = a.slot_of_expert ? a.slot_of_expert[e] : e;
    const int n0 = nt * 16 * NT;
    if (slot < 0 || slot >= a.num_slots) {
        if (tid == 0 && nt == 0) raise_status(a.status, MOE_DEV_BAD_SLOT);
        if (MODE == 1) {
            for (int i = tid; i < (r1 - r0) * 16 * NT; i += blockDim.x)
                a.y[static_cast<size_t>(r0 + i / (16 * NT)) * a.d + n0 + i % (16 * NT)] = 0.f;
        }
        return;
    }

    const int row = lane & 15, g = lane >> 4;
    const int s_beg = (S * wave) / KSPLIT, s_end = (S * (wave + 1)) / KSPLIT;

    // per-lane row bases of the weight packs
    const uint8_t* cbase[NMAT][NT];
    const uint8_t* sbase[NMAT][NT];
    const uint16_t* mbase[NMAT][NT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
        const int mat = MODE == 0 ? m : 2;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const size_t n = static_cast<size_t>(slot) * N + n0 + 16 * t + row;
            if constexpr (FMT == MOE_FMT_MXFP4) {
                cbase[m][t] = a.codes[mat] + n * (K / 2);
                sbase[m][t] = a.scales[mat] + n * G;
                mbase[m][t] = nullptr;
            } else {
                cbase[m][t] = a.codes[mat] + n * (K / 4);
                sbase[m][t] = a.scales[mat] + n * G * 2;
                mbase[m][t] = a.mins[mat] + n * G;
            }
        }
    }

    for (int c0 = r0; c0 < r1; c0 += 16) {
        const int r = c0 + row;          // token column of this lane (B operand)
        const bool colok = r < r1;
        const uint16_t* brow;
        if (MODE == 0) brow = a.x + static_cast<size_t>(colok ? a.perm[r] / a.k : 0) * a.d;
        else brow = a.act + static_cast<size_t>(colok ? r : 0) * a.f;

        f32x4 acc[NMAT][NT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[m][t] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int sb = s_beg; sb < s_end; sb += kUnroll) {
            if constexpr (FMT == MOE_FMT_MXFP4) {
                u32x4 cv[kUnroll][NMAT][NT];
                uint32_t sc[kUnroll][NMAT][NT];
                u32x4 bv[kUnroll][4];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int gi = 4 * (sb + u) + g;
                    const bool ok = (sb + u) < s_end && gi < G;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            cv[u][m][t] = ok ? *reinterpret_cast<const u32x4*>(cbase[m][t] + gi * 16) : u32x4{0u, 0u, 0u, 0u};
                            sc[u][m][t] = ok ? sbase[m][t][gi] : 127u;
                        }
                    const u32x4* bp = reinterpret_cast<const u32x4*>(brow + gi * kGroup);
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[u][j] = (ok && colok) ? bp[j] : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    float scl[NMAT][NT];
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int t = 0; t < NT; ++t) scl[m][t] = e8m0_to_f32(sc[u][m][t]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x8 b = bf16x8_from_u32x4(bv[u][j]);
#pragma unroll
                        for (int m = 0; m < NMAT; ++m)
#pragma unroll
                            for (int t = 0; t < NT; ++t)
                                acc[m][t] = mfma16x16x32(mxfp4x8_to_bf16(cv[u][m][t][j], scl[m][t]), b, acc[m][t]);
                    }
                }
            } else {
                // ---------------- Q2: one group per MFMA
                u32x2 cv[kUnroll][NMAT][NT];
                uint32_t smv[kUnroll][NMAT][NT];   // fp16 scale (low) | fp16 min (high)
                u32x4 bv[kUnroll][4];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int s = sb + u;
                    const int gl = 4 * s + g;      // group this lane loads (lane-group layout)
                    const bool okl = s < s_end && gl < G;
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            cv[u][m][t] = okl ? *reinterpret_cast<const u32x2*>(cbase[m][t] + gl * 8) : u32x2{0u, 0u};
                            const uint32_t sv = okl ? reinterpret_cast<const uint16_t*>(sbase[m][t])[gl] : 0u;
                            const uint32_t mv = okl ? mbase[m][t][gl] : 0u;
                            smv[u][m][t] = sv | (mv << 16);
                        }
                    // token operand for MFMA j: group 4s+j, elements 8g..8g+7
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int gj = 4 * s + j;
                        const bool okj = s < s_end && gj < G && colok;
                        bv[u][j] = okj ? *reinterpret_cast<const u32x4*>(brow + gj * kGroup + 8 * g) : u32x4{0u, 0u, 0u, 0u};
                    }
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    // re-lay codes and scale/min through LDS (wave-private area)
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            q2codes[FMT == MOE_FMT_Q2G32 ? wave : 0][m * NT + t][row][g] = cv[u][m][t];
                            const float sf = fp16_to_f32(smv[u][m][t]);
                            const float mf = fp16_to_f32(smv[u][m][t] >> 16);
                            q2sm[FMT == MOE_FMT_Q2G32 ? wave : 0][m * NT + t][g][row] = make_float2(4.f * sf, fmaf(-4.f, sf, mf));
                        }
                    __builtin_amdgcn_wave_barrier();
                    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bf16x8 b = bf16x8_from_u32x4(bv[u][j]);
                        const f32x4 xs = mfma16x16x32(ones, b, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                        for (int m = 0; m < NMAT; ++m)
#pragma unroll
                            for (int t = 0; t < NT; ++t) {
                                const u32x2 cw = q2codes[FMT == MOE_FMT_Q2G32 ? wave : 0][m * NT + t][row][j];
                                const uint32_t c16 = ((g & 2) ? cw[1] : cw[0]) >> (16 * (g & 1));
                                // eight 2-bit codes -> eight bf16(1 + q/4), two per dword
                                u32x4 av;
#pragma unroll
                                for (int h = 0; h < 4; ++h) {
                                    const uint32_t c4 = c16 >> (4 * h);
                                    av[h] = ((c4 & 3u) << 5) | ((c4 & 0xcu) << 19) | 0x3f803f80u;
                                }
                                const f32x4 cq = mfma16x16x32(bf16x8_from_u32x4(av), b, f32x4{0.f, 0.f, 0.f, 0.f});
                                const float4* smp = reinterpret_cast<const float4*>(&q2sm[FMT == MOE_FMT_Q2G32 ? wave : 0][m * NT + t][j][4 * g]);
                                const float4 sm01 = smp[0], sm23 = smp[1];
                                f32x4 ac = acc[m][t];
                                ac[0] = fmaf(sm01.x, cq[0], fmaf(sm01.y, xs[0], ac[0]));
                                ac[1] = fmaf(sm01.z, cq[1], fmaf(sm01.w, xs[1], ac[1]));
                                ac[2] = fmaf(sm23.x, cq[2], fmaf(sm23.y, xs[2], ac[2]));
                                ac[3] = fmaf(sm23.z, cq[3], fmaf(sm23.w, xs[3], ac[3]));
                                acc[m][t] = ac;
                            }
                    }
                    __builtin_amdgcn_wave_barrier();
                }
            }
        }

        // cross-wave reduction in fixed wave order, then the epilogue
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int t = 0; t < NT; ++t) red[wave][m * NT + t][lane] = acc[m][t];
        __syncthreads();
        for (int idx = tid; idx < 16 * 16 * NT; idx += KSPLIT * 64) {
            const int col = idx / (16 * NT), nl = idx % (16 * NT);
            const int t = nl / 16, nn = nl % 16;
            const int src = col + 16 * (nn / 4), i = nn % 4;
            const int rr = c0 + col;
            if (rr < r1) {
                float v[NMAT];
#pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                    float s = red[0][m * NT + t][src][i];
#pragma unroll
                    for (int w = 1; w < KSPLIT; ++w) s += red[w][m * NT + t][src][i];
                    v[m] = s;
                }
                const int n = n0 + nl;
                if constexpr (MODE == 0) {
                    a.act[static_cast<size_t>(rr) * a.f + n] = f32_to_bf16_rne(silu_mul(v[0], v[NMAT - 1]));
                } else {
                    a.y[static_cast<size_t>(rr) * a.d + n] = v[0];
                }
            }
        }
        __syncthreads();
    }
}

template <int FMT>
static hipError_t launch_skinny(const moe_shape& s, const FfnArgs& a, hipStream_t st) {
    constexpr int KS = 4, NT = 1;
    const int umax = s.E < s.T * s.k ? s.E : s.T * s.k;
    ffn_skinny_kernel<FMT, 0, KS, NT><<<umax * (s.f / (16 * NT)), KS * 64, 0, st>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_skinny_kernel<FMT, 1, KS, NT><<<umax * (s.d / (16 * NT)) + 1, KS * 64, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_ffn_skinny(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    if (fmt == MOE_FMT_MXFP4) return launch_skinny<MOE_FMT_MXFP4>(s, a, st);
    return launch_skinny<MOE_FMT_Q2G32>(s, a, st);
}

}  // namespace qrmoe

namespace qrmoe {

hipError_t launch_ffn(const moe_shape& s, int fmt, const FfnArgs& a, hipStream_t st) {
    return launch_ffn_skinny(s, fmt, a, st);
}

}  // namespace qrmoe
