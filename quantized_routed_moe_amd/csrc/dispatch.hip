// Token-by-expert dispatch: a stable counting sort of the T*k (token, slot)
// pairs by expert id.  It is what lets every activated expert's weights be
// streamed once for all of its rows -- the block-sparse routed-expert
// kernel of "antirez ds4: DeepSeek Metal inference" (section 技术深度解析).
//
// One workgroup of 1024 threads.  Pass 1 counts pairs per expert (LDS
// integer atomics: the counts do not depend on their order).  An exclusive
// scan gives offsets.  Pass 2 walks the pairs in chunks of 4096, as 64
// sub-tiles of 64 consecutive pairs (four per wave); inside a sub-tile, the
// lanes holding the same expert are found with seven ballots (one per bit
// of the id), so a pair's rank among equal ids is a popcount over lower
// lanes; the per-sub-tile counts are scanned over the sub-tiles in LDS,
// eight threads per expert, so a chunk takes four barriers.
// Nothing depends on atomic ordering, so the permutation is deterministic
// and stable.  Ids outside [0, E) go to an extra bucket E after all valid
// pairs and raise MOE_DEV_BAD_EXPERT_ID.  Batches of at most 64 pairs take
// a one-wave kernel with the same order.
#include "common.hpp"
#include "dispatch_dev.hpp"
#include "kernels.hpp"

namespace qrmoe {

constexpr int kDispThreads = 1024;

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, uint32_t* __restrict__ status, int n_pairs, int E, int shared_rows, int k) {
    dispatch_block<kDispThreads>(ids, offsets, perm, inv, status, n_pairs, E);
    for (int t = threadIdx.x; t < shared_rows; t += kDispThreads) perm[n_pairs + t] = t * k;
}

// At most 64 pairs: one wave, one pair per lane.  A pair's row is the
// number of pairs in lower buckets plus the number of earlier pairs in its
// own bucket (the same stable order as above, invalid ids in bucket E); the
// 1024-thread kernel's chunk machinery costs more than the sort here.
constexpr int kDispSmallPairs = 64;

__global__ __launch_bounds__(64) void dispatch_small_kernel(
    const int32_t* __restrict__ ids, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, uint32_t* __restrict__ status, int n_pairs, int E, int shared_rows, int k) {
    const int lane = threadIdx.x;
    int b = E + 1;                               // lanes past n_pairs take no part
    if (lane < n_pairs) {
        b = ids[lane];
        if (b < 0 || b >= E) b = E;
    }
    int lower = 0, earlier = 0, below_lane = 0;
    for (int q = 0; q < n_pairs; ++q) {
        const int bq = lane_value(b, q);
        lower += bq < b;
        earlier += (bq == b) & (q < lane);
        below_lane += bq < lane;
    }
    if (lane < n_pairs) {
        perm[lower + earlier] = lane;
        inv[lane] = lower + earlier;
    }
    if (lane < E) offsets[lane] = below_lane;
    const uint64_t valid = __ballot(lane < n_pairs && b < E);
    const uint64_t bad = __ballot(lane < n_pairs && b == E);
    if (lane == 0) {
        offsets[E] = __popcll(valid);
        if (bad) raise_status(status, MOE_DEV_BAD_EXPERT_ID);
    }
    if (lane < shared_rows) perm[n_pairs + lane] = lane * k;
}

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, int32_t* offsets, int32_t* perm,
                           int32_t* inv, uint32_t* status, hipStream_t st, bool shared) {
    const int n_pairs = s.T * s.k;
    if (n_pairs <= kDispSmallPairs)
        dispatch_small_kernel<<<1, 64, 0, st>>>(ids, offsets, perm, inv, status, n_pairs, s.E,
                                                 shared ? s.T : 0, s.k);
    else
        dispatch_kernel<<<1, kDispThreads, 0, st>>>(ids, offsets, perm, inv, status, n_pairs, s.E,
                                                    shared ? s.T : 0, s.k);
    return hipGetLastError();
}

}  // namespace qrmoe
