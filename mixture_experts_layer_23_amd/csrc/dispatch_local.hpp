// dispatch_local.hpp -- the per-chunk step of dispatch (ruDNN user guide, section 5): the counts
// of a chunk's (token, slot) pairs per expert and each pair's stable rank among the chunk's pairs
// of the same expert.  Used by the dispatch kernel of its own and by the routing kernel's
// epilogue when routing and dispatch run together.
#pragma once

#include "device.hpp"

namespace rudnn {

// The chunk holds `n` pairs; ids(p) is the expert id of chunk pair p (p in (token, slot) order).
// count(e, v) receives the number of pairs with id e; ranks[p] = number of earlier pairs with the
// same id, or -1 for an id >= E (such a pair is not counted).  Lanes of a wavefront holding the
// same id are found with one ballot per id bit (id_bits = ceil(log2 E)); the first W wavefronts take
// 64 W pairs per round and LDS counters carry across wavefronts and rounds.  run [E] and
// wcnt [W][E] are LDS, contiguous.  Every thread of the block calls it together (it holds barriers).
template <int W, typename IdFn, typename CountFn>
__device__ __forceinline__ void chunk_ranks(IdFn ids, int n, int E, int id_bits, int* run, int* wcnt, CountFn count,
                                            int32_t* __restrict__ ranks) {
    for (int i = threadIdx.x; i < (W + 1) * E; i += blockDim.x) run[i] = 0;
    __syncthreads();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const bool worker = wave < W;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < n; r0 += 64 * W) {
        const int p = r0 + (int)threadIdx.x;
        const bool in = worker && p < n;
        const uint32_t e = in ? ids(p) : 0xffffffffu;
        const bool valid = in && e < (uint32_t)E;
        // lanes holding the same id: agree with this lane on every id bit
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < id_bits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1u));
            peers &= ((e >> b) & 1u) ? ones : ~ones;
        }
        const int rank = __popcll(peers & lt_mask);
        const bool leader = valid && rank == 0;  // the lowest lane of its id
        if (leader) wcnt[wave * E + e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int r = run[e] + rank;
            for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
            ranks[p] = r;
        } else if (in) {
            ranks[p] = -1;
        }
        if (r0 + 64 * W < n) {  // another round: carry this one's counts
            __syncthreads();
            if (leader) {  // one leader per id and wavefront: wavefronts holding the same id add concurrently
                atomicAdd(&run[e], __popcll(peers));
                wcnt[wave * E + e] = 0;
            }
            __syncthreads();
        }
    }
    __syncthreads();
    // counts: the carried counts plus the last round's wavefront counts
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = run[e];
        for (int w = 0; w < W; ++w) c += wcnt[w * E + e];
        count(e, c);
    }
}

}  // namespace rudnn
