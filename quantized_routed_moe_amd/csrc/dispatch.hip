// Token-by-expert dispatch: a stable counting sort of the T*k (token, slot)
// pairs by expert id.  It is what lets every activated expert's weights be
// streamed once for all of its rows -- the block-sparse routed-expert
// kernel of "antirez ds4: DeepSeek Metal inference" (section 技术深度解析).
//
// One workgroup of 1024 threads.  Pass 1 counts pairs per expert (LDS
// integer atomics: the counts do not depend on their order).  An exclusive
// scan gives offsets.  Pass 2 walks the pairs in tiles of 1024; inside a
// wave, the lanes holding the same expert are found with seven ballots (one
// per bit of the id), so a pair's rank among equal ids is a popcount over
// lower lanes; per-wave totals are scanned across the 16 waves in LDS.
// Nothing depends on atomic ordering, so the permutation is deterministic
// and stable.  Ids outside [0, E) go to an extra bucket E after all valid
// pairs and raise MOE_DEV_BAD_EXPERT_ID.
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

hipError_t launch_dispatch(const moe_shape& s, const int32_t* ids, int32_t* offsets, int32_t* perm,
                           int32_t* inv, uint32_t* status, hipStream_t st, bool shared) {
    dispatch_kernel<<<1, kDispThreads, 0, st>>>(ids, offsets, perm, inv, status, s.T * s.k, s.E,
                                                shared ? s.T : 0, s.k);
    return hipGetLastError();
}

}  // namespace qrmoe
