// Weighted combine: out[t] = sum_j w[t][j] * y[inv[t*k + j]], summed in
// j order (deterministic; no atomics).  One workgroup per token, four floats
// per thread per pass over d.  y is read once and out written once, so both
// go through non-temporal accesses (they do not displace cached lines; at
// 2048 tokens this measured ~1.5 % off the layer step).  Products and sums are rounded separately (no
// fused multiply-add), so for k <= 2 the result equals the scatter-add of
// the weighted expert outputs that moe_layer fuses into the down projection.
#include "common.hpp"
#include "kernels.hpp"

namespace qrmoe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                       const int32_t* __restrict__ inv,
                                                       const float* __restrict__ w,
                                                       float* __restrict__ out, int d, int k,
                                                       const float* __restrict__ y_shared) {
    const int t = blockIdx.x;
    const int d4 = d / 4;
    for (int i = threadIdx.x; i < d4; i += blockDim.x) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const float wj = w[static_cast<size_t>(t) * k + j];
            const int r = inv[static_cast<size_t>(t) * k + j];
            const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y + static_cast<size_t>(r) * d) + i);
            const float4 v = make_float4(q[0], q[1], q[2], q[3]);
            acc.x = __fadd_rn(acc.x, __fmul_rn(wj, v.x));
            acc.y = __fadd_rn(acc.y, __fmul_rn(wj, v.y));
            acc.z = __fadd_rn(acc.z, __fmul_rn(wj, v.z));
            acc.w = __fadd_rn(acc.w, __fmul_rn(wj, v.w));
        }
        if (y_shared) {     // the shared expert, weight 1, after the routed terms
            const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(y_shared + static_cast<size_t>(t) * d) + i);
            const float4 v = make_float4(q[0], q[1], q[2], q[3]);
            acc.x = __fadd_rn(acc.x, v.x);
            acc.y = __fadd_rn(acc.y, v.y);
            acc.z = __fadd_rn(acc.z, v.z);
            acc.w = __fadd_rn(acc.w, v.w);
        }
        const f32x4 o = {acc.x, acc.y, acc.z, acc.w};
        __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out + static_cast<size_t>(t) * d) + i);
    }
}

__global__ void clear_header_kernel(uint32_t* header) {
    if (threadIdx.x < kWsHeader / 4) header[threadIdx.x] = 0u;
}

hipError_t launch_combine(const moe_shape& s, const float* y, const int32_t* inv, const float* w,
                          float* out, hipStream_t st, bool shared) {
    const float* ys = shared ? y + static_cast<size_t>(s.T) * s.k * s.d : nullptr;
    combine_kernel<<<s.T, 256, 0, st>>>(y, inv, w, out, s.d, s.k, ys);
    return hipGetLastError();
}

hipError_t launch_clear_header(uint32_t* header, hipStream_t st) {
    clear_header_kernel<<<1, 64, 0, st>>>(header);
    return hipGetLastError();
}

}  // namespace qrmoe
