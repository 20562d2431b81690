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
    constexpr int kPer = 4;                      // sub-tiles of 64 pairs per wave and chunk
    constexpr int kSub = kWaves * kPer;          // sub-tiles per chunk
    constexpr int kChunk = kSub * kWave;         // pairs per chunk
    constexpr int kParts = 8;                    // threads per bucket in the scan over sub-tiles
    static_assert(kSub % kParts == 0 && (kMaxExperts + 1) * kParts <= THREADS, "dispatch scan layout");
    __shared__ int cnt[kMaxExperts + 1];
    __shared__ int base[kMaxExperts + 1];
    __shared__ int wcnt[kSub][kMaxExperts + 1];
    __shared__ int bad;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t lt_mask = lane ? ((~0ull) >> (64 - lane)) : 0ull;
    // Sub-tile st (= wave * kPer + j) of the chunk at c0 holds its pairs
    // st * 64 .. +63 in lane order, so sub-tiles, and lanes within one,
    // follow the pair order.  classify() gives each of this thread's pairs
    // its bucket (E for ids outside [0, E), E + 1 past n_pairs), its rank
    // among the lanes of its sub-tile with the same bucket (lanes with the
    // same bucket: AND of per-bit agreement masks, buckets < 128), the size
    // of that group and whether it is the group's highest lane.
    int e[kPer], rank[kPer], gsize[kPer];
    bool valid[kPer], leader[kPer];
    auto classify = [&](int c0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = c0 + (wave * kPer + j) * kWave + lane;
            valid[j] = p < n_pairs;
            int ej = E + 1;
            if (valid[j]) {
                ej = ids[p];
                if (ej < 0 || ej >= E) ej = E;
            }
            uint64_t same = ~0ull;
#pragma unroll
            for (int b = 0; b < 7; ++b) {
                const uint64_t ones = __ballot((ej >> b) & 1);
                same &= ((ej >> b) & 1) ? ones : ~ones;
            }
            e[j] = ej;
            rank[j] = __popcll(same & lt_mask);
            gsize[j] = __popcll(same);
            leader[j] = (same >> lane) == 1ull;
        }
    };
    // Pass 1: counts per bucket (one LDS atomic per group of equal ids in a
    // sub-tile; the counts do not depend on the atomics' order).  The first
    // chunk's classification stays in registers for pass 2.
    if (tid <= E) cnt[tid] = 0;
    if (tid == 0) bad = 0;
    for (int i = tid; i < kSub * (kMaxExperts + 1); i += THREADS) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    for (int c0 = kChunk; c0 < n_pairs; c0 += kChunk) {       // chunks 1, 2, ... first
        classify(c0);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (valid[j] && leader[j]) {
                atomicAdd(&cnt[e[j]], gsize[j]);
                if (e[j] == E) bad = 1;
            }
        }
    }
    if (n_pairs > 0) {
        classify(0);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (valid[j] && leader[j]) {
                atomicAdd(&cnt[e[j]], gsize[j]);
                if (e[j] == E) bad = 1;
            }
        }
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
    // Pass 2, chunk by chunk (chunk 0 classified above; wcnt cleared).
    for (int c0 = 0; c0 < n_pairs; c0 += kChunk) {
        if (c0 > 0) {
            // clear every [sub-tile][bucket] count: a sub-tile that holds no
            // pair of bucket b never writes wcnt[st][b], and the scan reads it
            for (int i = tid; i < kSub * (kMaxExperts + 1); i += THREADS) (&wcnt[0][0])[i] = 0;
            classify(c0);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (valid[j] && leader[j]) wcnt[wave * kPer + j][e[j]] = gsize[j];
        __syncthreads();
        // exclusive scan of each bucket's counts over the sub-tiles: kParts
        // threads per bucket, each summing kSub / kParts consecutive
        // sub-tiles, then a scan across the kParts threads (adjacent lanes)
        if (tid < (E + 1) * kParts) {
            constexpr int kPerPart = kSub / kParts;
            const int b = tid / kParts, part = tid % kParts;
            int v[kPerPart];
            int sum = 0;
#pragma unroll
            for (int i = 0; i < kPerPart; ++i) {
                v[i] = wcnt[part * kPerPart + i][b];
                sum += v[i];
            }
            int incl = sum;
#pragma unroll
            for (int o = 1; o < kParts; o <<= 1) {
                const int t = __shfl_up(incl, o, kParts);
                if (part >= o) incl += t;
            }
            int run = incl - sum;
#pragma unroll
            for (int i = 0; i < kPerPart; ++i) {
                wcnt[part * kPerPart + i][b] = run;
                run += v[i];
            }
            if (part == kParts - 1) cnt[b] = incl;       // this chunk's total for bucket b
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            if (valid[j]) {
                const int p = c0 + (wave * kPer + j) * kWave + lane;
                const int r = base[e[j]] + wcnt[wave * kPer + j][e[j]] + rank[j];
                perm[r] = p;
                inv[p] = r;
            }
        }
        __syncthreads();
        if (tid <= E) base[tid] += cnt[tid];
    }
}

}  // namespace qrmoe
