// Device-side body of the dispatch, shared by the standalone dispatch kernel
// and the fused small-T routing kernel (see dispatch.hip for the method).
#pragma once

#include "common.hpp"

namespace qrmoe {

// One workgroup of THREADS threads sorts the n_pairs pairs by expert id.
template <int THREADS>
__device__ __forceinline__ void dispatch_block(const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                               uint32_t* __restrict__ status, int n_pairs, int E) {
    constexpr int kWaves = THREADS / kWave;
    __shared__ int cnt[kMaxExperts + 1];
    __shared__ int base[kMaxExperts + 1];
    __shared__ int wcnt[kWaves][kMaxExperts + 1];
    __shared__ int bad;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid <= E) cnt[tid] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int p = tid; p < n_pairs; p += THREADS) {
        int e = ids[p];
        if (e < 0 || e >= E) { e = E; bad = 1; }
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (wave == 0) {           // exclusive scan of the counts over a wave (E <= 64)
        const int c = lane < E ? cnt[lane] : 0;
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o);
            if (lane >= o) incl += v;
        }
        if (lane < E) {
            base[lane] = incl - c;
            offsets[lane] = incl - c;
        }
        if (lane == 63) {      // lanes >= E hold 0, so this is the number of valid pairs
            base[E] = incl;
            offsets[E] = incl;
        }
        if (lane == 0 && bad) raise_status(status, MOE_DEV_BAD_EXPERT_ID);
    }
    __syncthreads();
    const uint64_t lt_mask = lane ? ((~0ull) >> (64 - lane)) : 0ull;
    for (int p0 = 0; p0 < n_pairs; p0 += THREADS) {
        const int p = p0 + tid;
        const bool valid = p < n_pairs;
        int e = E + 1;                                   // padding lanes: matches no real id
        if (valid) {
            e = ids[p];
            if (e < 0 || e >= E) e = E;
        }
        // lanes with the same e: AND of per-bit agreement masks (e < 128)
        uint64_t same = ~0ull;
#pragma unroll
        for (int b = 0; b < 7; ++b) {
            const uint64_t ones = __ballot((e >> b) & 1);
            same &= ((e >> b) & 1) ? ones : ~ones;
        }
        const int rank = __popcll(same & lt_mask);
        const bool leader = (same >> lane) == 1ull;     // highest lane of its group
        // clear every [wave][expert] count: a wave that holds no pair of
        // expert e never writes wcnt[wave][e], and the scan below reads it
        for (int i = tid; i < kWaves * (kMaxExperts + 1); i += THREADS) (&wcnt[0][0])[i] = 0;
        __syncthreads();
        if (valid && leader) wcnt[wave][e] = __popcll(same);
        __syncthreads();
        if (tid <= E) {                                  // exclusive scan over waves
            int run = 0;
            for (int w = 0; w < kWaves; ++w) {
                const int c = wcnt[w][tid];
                wcnt[w][tid] = run;
                run += c;
            }
            cnt[tid] = run;                              // this tile's total for expert tid
        }
        __syncthreads();
        if (valid) {
            const int r = base[e] + wcnt[wave][e] + rank;
            perm[r] = p;
            inv[p] = r;
        }
        __syncthreads();
        if (tid <= E) base[tid] += cnt[tid];
        __syncthreads();
    }
}

}  // namespace qrmoe
