// Device helpers shared by the gfx950 kernels of the routed MoE layer:
// number formats (bf16, e2m1 / e8m0, 2-bit groups), MFMA operand types and
// small wave64 utilities.  Everything here is written for CDNA4 (gfx950),
// wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace qrmoe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 64;
constexpr int kGroup = 32;             // elements per quantisation group (MX block)
constexpr size_t kWsHeader = 256;      // workspace header: device status word
constexpr int kLastBlockCounter = 16;  // header word (byte 64): last-workgroup counter of fused routing
constexpr int kChainPollWord = 32;     // header word (byte 128): poll limit of the prefill hand-off (0: default)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern (NaN stays NaN, quietened).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// IEEE binary16 bit pattern (low 16 bits) -> float (exact).
__device__ __forceinline__ float fp16_to_f32(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xffffu)));
}

// Two bf16 (as one dword: low half = element 0) -> two floats.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- MXFP4

// e8m0 byte -> float 2^(b-127).  Bytes 1..254 give normal floats exactly;
// byte 0 (2^-127) is a float32 subnormal and is built separately.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Eight e2m1 codes (one dword, element 0 in the low nibble) times the block
// scale -> eight bf16 in MFMA operand order.  Uses the gfx950 scaled
// conversion, which applies the scale exactly (the product is representable
// in bf16 for every code and every scale whose result is a normal bf16).
__device__ __forceinline__ bf16x8 mxfp4x8_to_bf16(uint32_t codes, float scale) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// ---------------------------------------------------------------- MFMA

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) + 0..7] and B[8*(l/16) + 0..7][l%16];
// it receives C[4*(l/16) + 0..3][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16) * B(16x32) + C.  Lane l supplies A[l%32][8*(l/32) + 0..7] and
// B[8*(l/32) + 0..7][l%32]; it receives C[8*(i/4) + 4*(l/32) + i%4][l%32] in
// element i (0..15).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bf16x8_from_u32x4(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 bf16x8_zero() {
    return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// ---------------------------------------------------------------- misc

// ---- MXFP8 activations (OCP MX v1.0: E4M3 elements, one E8M0 scale per 32)

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32x64 block-scaled product, A = 32 E2M1 weights per lane (16 bytes of
// a tile-layout piece, one K block of 32), B = 32 E4M3 token bytes per lane,
// fp32 accumulation; sa / sb are the E8M0 scale bytes of the lane's A row
// block and B column block.  Lane layout (measured on gfx950): lane l holds
// A row l%32 and B column l%32; A's 32 elements are K block l/32, B's bytes
// 0..15 and 16..31 are elements [16(l/32), +16) of K blocks 0 and 1, and
// B's scale is that of K block l/32.
__device__ __forceinline__ f32x16 mfma_scale_fp4_fp8(u32x4 a, i32x8 b, f32x16 c, int sa, int sb) {
    const i32x8 a8 = {static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                      0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b, c, 4, 0, 0, sa, 0, sb);
}

// The same product with B = 32 E2M1 token values per lane (16 bytes, K
// block l/32, as A) and B's scale that of K block l/32.
__device__ __forceinline__ f32x16 mfma_scale_fp4_fp4(u32x4 a, u32x4 b, f32x16 c, int sa, int sb) {
    const i32x8 a8 = {static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3]),
                      0, 0, 0, 0};
    const i32x8 b8 = {static_cast<int>(b[0]), static_cast<int>(b[1]), static_cast<int>(b[2]), static_cast<int>(b[3]),
                      0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, 4, 4, 0, sa, 0, sb);
}

// E8M0 scale byte of a block whose largest magnitude is amax:
// floor(log2 amax) - 8 + 127 (8 = E4M3's largest exponent), clamped to
// 0..254; 0 for an all-zero block.
__device__ __forceinline__ int mx8_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0;
    const int e = ilogbf(amax) - 8 + 127;
    return e < 0 ? 0 : e > 254 ? 254 : e;
}

// MXFP4 (E2M1 elements): floor(log2 amax) - 2 + 127 (2 = E2M1's largest
// exponent), clamped to 0..254; 0 for an all-zero block.
__device__ __forceinline__ int mx4_scale_byte(float amax) {
    if (!(amax > 0.f)) return 0;
    const int e = ilogbf(amax) - 2 + 127;
    return e < 0 ? 0 : e > 254 ? 254 : e;
}

// A value (already divided by the block scale) to its E2M1 code: nearest of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6, a tie going to the even code (even mantissa),
// magnitudes above 6 clamped to 6, the sign in bit 3, zero made +0.  The
// magnitude code counts the decision points passed: a tie stays below the
// point when the lower neighbour's code is even (0.25, 1.25, 2.5, 5) and
// passes it when the upper one's is (0.75, 1.75, 3.5).
__device__ __forceinline__ uint32_t e2m1_rne_sat(float v) {
    const float a = fabsf(v);
    const uint32_t c = static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
                       static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
                       static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
                       static_cast<uint32_t>(a > 5.f);
    return c | (v < 0.f && c != 0 ? 8u : 0u);
}

// Four values (already divided by the block scale) to E4M3 codes, low byte
// first: round to nearest even (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950) after
// clamping to +-448 (saturation), and -0 turned into +0.  Checked against
// rounding written out in integer steps on 4.2 M values around every E4M3
// value and midpoint: identical.
__device__ __forceinline__ uint32_t e4m3x4_rne_sat(float a, float b, float c, float d) {
    auto cl = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
    uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false));
    w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), static_cast<int>(w), true));
    const uint32_t m = w & 0x7F7F7F7Fu;                          // magnitudes
    const uint32_t nz = ((m + 0x7F7F7F7Fu) | m) & 0x80808080u;   // bit 7 of each nonzero byte
    return m | (w & nz);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    // silu(g) * u = g / (1 + exp(-g)) * u
    return g / (1.0f + expf(-g)) * u;
}

// v of lane `src` (a wave-uniform index) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// One step of a wave max over DPP: every lane the control moves data into
// takes max(own, moved); the others keep their value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const int lo = static_cast<int>(static_cast<uint32_t>(v));
    const int hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
    const uint32_t mlo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false));
    const uint32_t mhi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false));
    const uint64_t m = (static_cast<uint64_t>(mhi) << 32) | mlo;
    return m > v ? m : v;
}

// Maximum of a 64-bit value over the 64 lanes, returned to every lane.  Row
// shifts by 1, 2, 4, 8 leave each row's maximum in its lane 15; row
// broadcasts 15 and 31 carry those into lane 63, which is then read out.
// Register-to-register (DPP), no LDS round trips.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = dpp_max_u64<0x111, 0xf>(v);   // row_shr:1
    v = dpp_max_u64<0x112, 0xf>(v);   // row_shr:2
    v = dpp_max_u64<0x114, 0xf>(v);   // row_shr:4
    v = dpp_max_u64<0x118, 0xf>(v);   // row_shr:8
    v = dpp_max_u64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_max_u64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_f32(float v) {
    const int b = __float_as_int(v);
    // lanes the control moves no data into receive 0 (old = 0) and keep v
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, b, CTRL, ROW_MASK, 0xf, false));
}

// Sum of a float over the 64 lanes in a fixed order (the shifts and
// broadcasts of wave_max_u64), returned to every lane.
__device__ __forceinline__ float wave_sum_f32(float v) {
    v = dpp_add_f32<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add_f32<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add_f32<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add_f32<0x118, 0xf>(v);   // row_shr:8
    v = dpp_add_f32<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_add_f32<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return lane_value(v, 63);
}

__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bit) {
    atomicOr(status, bit);
}

// Active-expert lookup from offsets[E+1]: every lane of the calling wave
// receives the id of the `a`-th expert (in id order) that owns at least one
// row, or -1 if fewer than a+1 experts are active.  E <= 64.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ offsets, int E, int a) {
    const int lane = threadIdx.x & (kWave - 1);
    int cnt = 0;
    if (lane < E) cnt = offsets[lane + 1] - offsets[lane];
    const uint64_t mask = __ballot(cnt > 0);
    const uint64_t below = lane ? (mask & ((~0ull) >> (64 - lane))) : 0ull;
    const bool hit = cnt > 0 && __popcll(below) == a;
    const uint64_t hitmask = __ballot(hit);
    return hitmask ? __ffsll(static_cast<unsigned long long>(hitmask)) - 1 : -1;
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// s_waitcnt vmcnt(N), leaving the other counters alone (gfx950 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS pointee type of the global -> LDS load builtin.
typedef __attribute__((address_space(3))) void lds_void;

}  // namespace qrmoe
