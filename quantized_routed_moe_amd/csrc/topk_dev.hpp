// Top-k of one token by one wave, and the routing of a small batch in LDS
// (top-k + stable counting sort), shared by the top-k kernel, the fused
// small-batch routing kernel and the skinny FFN's in-workgroup routing.
#pragma once

#include "common.hpp"

namespace qrmoe {

// Sortable key of a finite float: larger float -> larger unsigned key; -0 and
// +0 share the key of +0.
__device__ __forceinline__ uint32_t float_key(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of one token by one wave; lane e holds expert e's logit.  k rounds of
// a 64-bit wave max over (key(logit) << 32 | 63 - e) pick experts in (logit
// desc, id asc) order.  The softmax over the selected logits is taken against
// the first (largest) one and summed in selection order.
__device__ __forceinline__ void topk_wave(const float* __restrict__ lrow, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int E, int k) {
    const int lane = threadIdx.x & 63;
    const float l = lane < E ? lrow[lane] : 0.f;
    uint64_t key = lane < E ? ((static_cast<uint64_t>(float_key(l)) << 32) | static_cast<uint32_t>(63 - lane)) : 0ull;
    int my_sel = -1;       // lane j < k: expert chosen in round j
    float my_l = 0.f;      // its logit
    float lmax = 0.f;
    for (int j = 0; j < k; ++j) {
        const uint64_t m = wave_max_u64(key);
        const int e = 63 - static_cast<int>(m & 63u);
        const float le = lane_value(l, e);
        if (j == 0) lmax = le;
        if (lane == j) { my_sel = e; my_l = le; }
        if (lane == e) key = 0ull;
    }
    const float ex = lane < k ? expf(my_l - lmax) : 0.f;
    float sum = 0.f;       // selection order: lane 0, 1, ..., k-1
    for (int j = 0; j < k; ++j) sum += lane_value(ex, j);
    if (lane < k) {
        ids[lane] = my_sel;
        w[lane] = ex / sum;
    }
}

// Routing of a batch of at most kRoutedMaxPairs pairs, held in LDS.
constexpr int kRoutedMaxPairs = 64;
struct SmallRouting {
    int32_t ids[kRoutedMaxPairs];
    float w[kRoutedMaxPairs];
    int32_t perm[kRoutedMaxPairs + 16];   // + a shared expert's rows (up to 16 tokens)
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

}  // namespace qrmoe
