// route.hip -- softmax / top-k routing (ruDNN user guide, section 4 "Routing contract").
//
// A group of G adjacent lanes owns one row of logits [T, E] (G = 1 .. 64, a power of two, so a
// wavefront covers 64 / G rows); lane l of the group holds experts [l * NPER, (l + 1) * NPER),
// so a wavefront's loads cover 64 / G consecutive rows contiguously.  The selection itself
// (exact top-k on the logits, FP32 softmax of the winners) is route_row in route_select.hpp, or
// route_row_sorted (same results, less VALU work) for 16-bit logits in whole 16-byte lane chunks.
// With the dispatch epilogue (routing and dispatch in one pass) the block's pairs are one dispatch
// chunk and the block also does dispatch's per-chunk step.
// HBM traffic per row: E * sizeof(logits) read, k * (4 + sizeof(logits)) written.
#include <type_traits>

#include "device.hpp"
#include "dispatch_local.hpp"
#include "internal.hpp"
#include "route_select.hpp"

namespace rudnn {

// VEC: the row chunk of every lane is NPER whole elements, 16-byte aligned (E % NPER == 0).
// DISPATCH: the block's pairs are also one dispatch chunk: after routing, the block writes the
// chunk's per-expert counts and each pair's rank among the chunk's pairs of the same expert
// (dispatch_local.hpp), from the winners it holds in LDS.
template <typename LT, int NPER, int G, bool VEC, int THREADS, bool DISPATCH>
__global__ __launch_bounds__(THREADS) void route_kernel(const LT* __restrict__ logits, int64_t T, int E, int k,
                                                        int renorm, uint32_t* __restrict__ idx, LT* __restrict__ w,
                                                        int id_bits, int32_t* __restrict__ chunk_counts,
                                                        int32_t* __restrict__ ranks) {
    typedef typename RouteBits<LT>::raw R;
    extern __shared__ float s_sel[];  // [rows per block][k] winner ids, then [rows per block][k] e_j, then
                                      // (DISPATCH) the chunk step's counters
    constexpr int RPB = THREADS / G;
    const int lane = lane_id(), l = lane % G, rb = threadIdx.x / G;
    const int64_t row = (int64_t)blockIdx.x * RPB + rb;
    uint32_t* si = reinterpret_cast<uint32_t*>(s_sel) + rb * k;
    float* se = s_sel + RPB * k + rb * k;
    const bool live = row < T;  // whole groups are live or not; no early return (shuffles)
    const int e0 = l * NPER;
    const R* x = reinterpret_cast<const R*>(logits) + (live ? row : 0) * (int64_t)E + e0;

    R raw[NPER];
    if (VEC) {
        constexpr int PER16 = 16 / (int)sizeof(R);
        static_assert(NPER % PER16 == 0, "whole 16-byte pieces per lane");
#pragma unroll
        for (int c = 0; c < NPER / PER16; ++c) {
            uint4 q = make_uint4(0, 0, 0, 0);
            if (live && e0 < E) q = *reinterpret_cast<const uint4*>(x + c * PER16);
            __builtin_memcpy(raw + c * PER16, &q, 16);
        }
    } else {
#pragma unroll
        for (int s = 0; s < NPER; ++s) raw[s] = (live && e0 + s < E) ? x[s] : (R)0;
    }
    if constexpr (VEC && sizeof(R) == 2) {
        // whole 16-byte lane chunks (E % NPER == 0): sorted per-lane lists (k is block-uniform)
        if (NPER == 16 && k <= 8)
            route_row_sorted<LT, NPER, G, (NPER == 16 ? 8 : NPER)>(raw, E, k, renorm, live, row, si, se, idx, w);
        else
            route_row_sorted<LT, NPER, G, NPER>(raw, E, k, renorm, live, row, si, se, idx, w);
    } else {
        route_row<LT, NPER, G>(raw, E, k, renorm, live, row, si, se, idx, w);
    }
    if constexpr (DISPATCH) {
        // si now holds every live row's stored ids (NaN rows included); pair p = rb * k + j
        const uint32_t* ids = reinterpret_cast<const uint32_t*>(s_sel);
        const int64_t row0 = (int64_t)blockIdx.x * RPB;
        const int n = (int)(min((int64_t)RPB, T - row0) * k);
        int* cnt = reinterpret_cast<int*>(s_sel + 2 * RPB * k);
        chunk_ranks<THREADS / 64>([&](int p) { return ids[p]; }, n, E, id_bits, cnt, cnt + E,
                                  [&](int e, int c) { chunk_counts[(int64_t)e * gridDim.x + blockIdx.x] = c; },
                                  ranks + row0 * k);
    }
}

template <typename LT, int NPER, int G, int THREADS, bool DISPATCH>
static void launch_route_g(const LT* l, int64_t T, int Ei, int ki, int r, uint32_t* idx, LT* wo, int32_t* counts,
                           int32_t* ranks, hipStream_t s) {
    constexpr int RPB = THREADS / G;
    const dim3 grid((unsigned)((T + RPB - 1) / RPB)), block(THREADS);
    const size_t smem = (size_t)RPB * ki * 8 + (DISPATCH ? (size_t)(THREADS / 64 + 1) * Ei * sizeof(int) : 0);
    const bool vec = Ei % NPER == 0 && (NPER * sizeof(LT)) % 16 == 0 && ((uintptr_t)l % 16) == 0;
    const int bits = DISPATCH ? dispatch_id_bits(Ei) : 0;
    if (vec)
        route_kernel<LT, NPER, G, true, THREADS, DISPATCH><<<grid, block, smem, s>>>(l, T, Ei, ki, r, idx, wo, bits,
                                                                                     counts, ranks);
    else
        route_kernel<LT, NPER, G, false, THREADS, DISPATCH><<<grid, block, smem, s>>>(l, T, Ei, ki, r, idx, wo, bits,
                                                                                      counts, ranks);
}

// Lanes per row: the smallest power of two G with G * 16 >= E (16 values per lane), at least 1
// (route_lanes).  Plain routing uses 256-thread blocks; with the dispatch epilogue the block size
// is route_dispatch_threads (a block's rows are one dispatch chunk).
template <typename LT, int THREADS, bool DISPATCH>
static void launch_route_e(const LT* l, int64_t T, int64_t E, int ki, int r, uint32_t* idx, LT* wo, int32_t* counts,
                           int32_t* ranks, hipStream_t s) {
    const int Ei = (int)E;
    if (E <= 8)
        launch_route_g<LT, 8, 1, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 16)
        launch_route_g<LT, 16, 1, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 32)
        launch_route_g<LT, 16, 2, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 64)
        launch_route_g<LT, 16, 4, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 128)
        launch_route_g<LT, 16, 8, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 256)
        launch_route_g<LT, 16, 16, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else if (E <= 512)
        launch_route_g<LT, 16, 32, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
    else
        launch_route_g<LT, 16, 64, THREADS, DISPATCH>(l, T, Ei, ki, r, idx, wo, counts, ranks, s);
}

template <typename LT>
static hipError_t launch_route_t(const void* logits, int64_t T, int64_t E, int64_t k, bool renorm, uint32_t* idx,
                                 void* w, void* dispatch_ws, hipStream_t s) {
    const LT* l = (const LT*)logits;
    LT* wo = (LT*)w;
    const int ki = (int)k, r = renorm ? 1 : 0;
    timing_before(RUDNN_MOE_KERNEL_ROUTE, s);
    if (!dispatch_ws) {
        launch_route_e<LT, 256, false>(l, T, E, ki, r, idx, wo, nullptr, nullptr, s);
    } else {
        int32_t* counts = (int32_t*)dispatch_ws;
        int32_t* ranks = (int32_t*)((unsigned char*)dispatch_ws + dispatch_ranks_offset(T, k, E));
        if (route_dispatch_threads(T, E) == 1024)
            launch_route_e<LT, 1024, true>(l, T, E, ki, r, idx, wo, counts, ranks, s);
        else
            launch_route_e<LT, 256, true>(l, T, E, ki, r, idx, wo, counts, ranks, s);
    }
    timing_after(RUDNN_MOE_KERNEL_ROUTE, s);
    return hipGetLastError();
}

hipError_t launch_route(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                        uint32_t* idx, void* w, hipStream_t s, void* dispatch_ws) {
    switch (ldt) {
    case RUDNN_MOE_F32: return launch_route_t<float>(logits, T, E, k, renorm, idx, w, dispatch_ws, s);
    case RUDNN_MOE_F16: return launch_route_t<f16>(logits, T, E, k, renorm, idx, w, dispatch_ws, s);
    default: return launch_route_t<bf16>(logits, T, E, k, renorm, idx, w, dispatch_ws, s);
    }
}

}  // namespace rudnn
