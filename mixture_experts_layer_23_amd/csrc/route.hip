// route.hip -- softmax / top-k routing (ruDNN user guide, section 4 "Routing contract").
//
// A group of G adjacent lanes owns one row of logits [T, E] (G = 1 .. 64, a power of two, so a
// wavefront covers 64 / G rows); lane l of the group holds experts [l * NPER, (l + 1) * NPER),
// so a wavefront's loads cover 64 / G consecutive rows contiguously.  The selection itself
// (exact top-k on the logits, FP32 softmax of the winners) is route_row in route_select.hpp, or
// route_row_sorted (same results, less VALU work) for 16-bit logits in whole 16-byte lane chunks.
// HBM traffic per row: E * sizeof(logits) read, k * (4 + sizeof(logits)) written.
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"
#include "route_select.hpp"

namespace rudnn {

constexpr int ROUTE_THREADS = 256;

// VEC: the row chunk of every lane is NPER whole elements, 16-byte aligned (E % NPER == 0).
template <typename LT, int NPER, int G, bool VEC>
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const LT* __restrict__ logits, int64_t T, int E, int k,
                                                              int renorm, uint32_t* __restrict__ idx,
                                                              LT* __restrict__ w) {
    typedef typename RouteBits<LT>::raw R;
    extern __shared__ float s_sel[];  // [rows per block][k] winner ids, then [rows per block][k] e_j
    constexpr int RPB = ROUTE_THREADS / G;
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
}

template <typename LT, int NPER, int G>
static void launch_route_g(const LT* l, int64_t T, int Ei, int ki, int r, uint32_t* idx, LT* wo, hipStream_t s) {
    constexpr int RPB = ROUTE_THREADS / G;
    const dim3 grid((unsigned)((T + RPB - 1) / RPB)), block(ROUTE_THREADS);
    const size_t smem = (size_t)RPB * ki * 8;
    const bool vec = Ei % NPER == 0 && (NPER * sizeof(LT)) % 16 == 0 && ((uintptr_t)l % 16) == 0;
    if (vec)
        route_kernel<LT, NPER, G, true><<<grid, block, smem, s>>>(l, T, Ei, ki, r, idx, wo);
    else
        route_kernel<LT, NPER, G, false><<<grid, block, smem, s>>>(l, T, Ei, ki, r, idx, wo);
}

// Lanes per row: the smallest power of two G with G * 16 >= E (16 values per lane), at least 1.
template <typename LT>
static hipError_t launch_route_t(const void* logits, int64_t T, int64_t E, int64_t k, bool renorm, uint32_t* idx,
                                 void* w, hipStream_t s) {
    const LT* l = (const LT*)logits;
    LT* wo = (LT*)w;
    const int Ei = (int)E, ki = (int)k, r = renorm ? 1 : 0;
    timing_before(RUDNN_MOE_KERNEL_ROUTE, s);
    if (E <= 8)
        launch_route_g<LT, 8, 1>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 16)
        launch_route_g<LT, 16, 1>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 32)
        launch_route_g<LT, 16, 2>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 64)
        launch_route_g<LT, 16, 4>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 128)
        launch_route_g<LT, 16, 8>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 256)
        launch_route_g<LT, 16, 16>(l, T, Ei, ki, r, idx, wo, s);
    else if (E <= 512)
        launch_route_g<LT, 16, 32>(l, T, Ei, ki, r, idx, wo, s);
    else
        launch_route_g<LT, 16, 64>(l, T, Ei, ki, r, idx, wo, s);
    timing_after(RUDNN_MOE_KERNEL_ROUTE, s);
    return hipGetLastError();
}

hipError_t launch_route(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                        uint32_t* idx, void* w, hipStream_t s) {
    switch (ldt) {
    case RUDNN_MOE_F32: return launch_route_t<float>(logits, T, E, k, renorm, idx, w, s);
    case RUDNN_MOE_F16: return launch_route_t<f16>(logits, T, E, k, renorm, idx, w, s);
    default: return launch_route_t<bf16>(logits, T, E, k, renorm, idx, w, s);
    }
}

}  // namespace rudnn
