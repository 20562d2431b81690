// Measurement kernels of the roofline (include/moe_peak.h): a chip-wide HBM
// read stream and a dense matrix-core loop, timed by the caller.
#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "../../include/moe_peak.h"
#include "common.hpp"

namespace qrmoe {

constexpr int kStreamThreads = 512;
constexpr int kStreamUnroll = 8;   // 16-byte loads in flight per thread per round

// Grid-stride read of n16 16-byte chunks: each round a thread issues
// kStreamUnroll loads kStreamUnroll * stride apart, so a wave reads whole
// 1 KB runs and every workgroup keeps 64 KB in flight.
__global__ __launch_bounds__(kStreamThreads) void peak_stream_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                                     uint32_t* __restrict__ sink) {
    const size_t stride = static_cast<size_t>(gridDim.x) * kStreamThreads;
    size_t i = static_cast<size_t>(blockIdx.x) * kStreamThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(buf + i);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    // one word per workgroup: xor over the lanes of each wave, then the waves
    for (int o = 32; o > 0; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o));
    __shared__ uint32_t part[kStreamThreads / kWave];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int w = 0; w < kStreamThreads / kWave; ++w) r ^= part[w];
        sink[blockIdx.x] = r;
    }
}

// Eight independent accumulator chains per wave, operands in registers that
// depend on the lane (so the compiler cannot fold them).
template <int KIND>
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.f;
    if constexpr (KIND == 0) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 7) * 0.125f);
            b[i] = static_cast<__bf16>(static_cast<float>((lane * 3 + i) & 7) * 0.0625f);
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
    } else if constexpr (KIND == 1) {
        const u32x4 a = {0x22222222u ^ static_cast<uint32_t>(lane), 0x12121212u, 0x21212121u, 0x11111111u};
        i32x8 b;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = 0x38383838 ^ (lane << (i & 3));
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = mfma_scale_fp4_fp8(a, b, acc[c], 127, 127);
        }
    } else {
        const u32x4 a = {0x22222222u ^ static_cast<uint32_t>(lane), 0x12121212u, 0x21212121u, 0x11111111u};
        const u32x4 b = {0x11111111u, 0x21212121u ^ static_cast<uint32_t>(lane), 0x12121212u, 0x22222222u};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] = mfma_scale_fp4_fp4(a, b, acc[c], 127, 127);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// One wave waits on the constant 100 MHz clock (s_memrealtime) until
// `ticks` have passed; the loop ends on time alone.
__global__ __launch_bounds__(64) void peak_hold_kernel(uint64_t ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(127);
}

}  // namespace qrmoe

extern "C" {

int moe_peak_stream(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink) return MOE_ERR_NULL;
    if (bytes == 0 || bytes % 16 || workgroups < 0) return MOE_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return MOE_ERR_ALIGN;
    const int g = workgroups ? workgroups : 2048;
    qrmoe::peak_stream_kernel<<<g, qrmoe::kStreamThreads, 0, stream>>>(static_cast<const qrmoe::u32x4*>(buf),
                                                                        bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_peak_mfma(int32_t kind, int32_t iters, int32_t workgroups, float* sink, hipStream_t stream) {
    if (!sink) return MOE_ERR_NULL;
    if (kind < 0 || kind > 2 || iters < 1 || workgroups < 0) return MOE_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(sink) % 4) return MOE_ERR_ALIGN;
    const int g = workgroups ? workgroups : 1024;
    if (kind == 0) qrmoe::peak_mfma_kernel<0><<<g, 256, 0, stream>>>(iters, sink);
    else if (kind == 1) qrmoe::peak_mfma_kernel<1><<<g, 256, 0, stream>>>(iters, sink);
    else qrmoe::peak_mfma_kernel<2><<<g, 256, 0, stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_peak_hold(uint32_t microseconds, hipStream_t stream) {
    if (microseconds < 1 || microseconds > 1000000) return MOE_ERR_SHAPE;
    qrmoe::peak_hold_kernel<<<1, 64, 0, stream>>>(static_cast<uint64_t>(microseconds) * 100u);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
