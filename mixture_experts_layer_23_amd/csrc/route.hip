// route.hip -- softmax / top-k routing (ruDNN user guide, section 4 "Routing contract").
//
// One 64-lane wavefront owns one row of logits [T, E].  Expert e lives in lane e % 64,
// register slot e / 64, so the slot order followed by the lane order is the id order.
//   1. NaN-row test: a ballot over "x is NaN or +inf" and over "x is not -inf".
//   2. FP32 softmax: wave max, exp(x - max), wave sum, one reciprocal.
//   3. k selection rounds: the wave max of the remaining probabilities, then per slot a
//      ballot of the lanes holding exactly that value; the first slot with a hit and its
//      lowest lane give the lowest id among equal probabilities (ties favour lower ids).
//      The winner is removed by setting it to -1 (probabilities are >= 0).
//   4. Lane j keeps the j-th winner; optional renormalisation by the wave sum of the k
//      selected values; one rounding to the logits dtype.
// HBM traffic per row: E * sizeof(logits) read, k * (4 + sizeof(logits)) written.
#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

constexpr int ROUTE_ROWS_PER_BLOCK = 4;  // 4 waves of 64 lanes

template <typename LT, int NPER>
__global__ __launch_bounds__(256) void route_kernel(const LT* __restrict__ logits, int64_t T, int E, int k,
                                                    int renorm, uint32_t* __restrict__ idx, LT* __restrict__ w) {
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * ROUTE_ROWS_PER_BLOCK + (threadIdx.x >> 6);
    if (row >= T) return;  // uniform per wave
    const LT* x = logits + row * (int64_t)E;

    float v[NPER];
    bool nan_or_posinf = false, not_neginf = false;
#pragma unroll
    for (int s = 0; s < NPER; ++s) {
        const int e = s * 64 + lane;
        float f = -INFINITY;
        if (e < E) {
            f = to_f32(x[e]);
            nan_or_posinf |= (f != f) || (f == INFINITY);
            not_neginf |= (f != -INFINITY);
        }
        v[s] = f;
    }
    if (__ballot(nan_or_posinf) != 0 || __ballot(not_neginf) == 0) {
        // NaN row: NaN weights, indices 0..k-1 (every probability NaN, read as a full tie).
        if (lane < k) {
            idx[row * k + lane] = (uint32_t)lane;
            w[row * k + lane] = from_f32<LT>(__builtin_nanf(""));
        }
        return;
    }

    float m = v[0];
#pragma unroll
    for (int s = 1; s < NPER; ++s) m = fmaxf(m, v[s]);
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < NPER; ++s) {
        v[s] = expf(v[s] - m);  // exp(-inf) = 0 exactly; padding lanes hold -inf
        sum += v[s];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int s = 0; s < NPER; ++s) v[s] = (s * 64 + lane < E) ? v[s] * inv : -1.0f;

    uint32_t my_id = 0;
    float my_p = 0.f;
    for (int j = 0; j < k; ++j) {
        float best = v[0];
#pragma unroll
        for (int s = 1; s < NPER; ++s) best = fmaxf(best, v[s]);
        const float pm = wave_max(best);
        int sel = -1;
#pragma unroll
        for (int s = 0; s < NPER; ++s) {
            const uint64_t hit = __ballot(v[s] == pm);
            if (sel < 0 && hit != 0) sel = s * 64 + __builtin_ctzll(hit);
        }
#pragma unroll
        for (int s = 0; s < NPER; ++s)
            if (s * 64 + lane == sel) v[s] = -1.0f;
        if (lane == j) {
            my_id = (uint32_t)sel;
            my_p = pm;
        }
    }
    float wt = my_p;
    if (renorm) {
        const float den = wave_sum(lane < k ? my_p : 0.f);
        wt = my_p / den;
    }
    if (lane < k) {
        idx[row * k + lane] = my_id;
        w[row * k + lane] = from_f32<LT>(wt);
    }
}

template <typename LT>
static hipError_t launch_route_t(const void* logits, int64_t T, int64_t E, int64_t k, bool renorm, uint32_t* idx,
                                 void* w, hipStream_t s) {
    const dim3 grid((unsigned)((T + ROUTE_ROWS_PER_BLOCK - 1) / ROUTE_ROWS_PER_BLOCK)), block(256);
    const LT* l = (const LT*)logits;
    LT* wo = (LT*)w;
    const int Ei = (int)E, ki = (int)k, r = renorm ? 1 : 0;
    timing_before(RUDNN_MOE_KERNEL_ROUTE, s);
    if (E <= 64)
        route_kernel<LT, 1><<<grid, block, 0, s>>>(l, T, Ei, ki, r, idx, wo);
    else if (E <= 128)
        route_kernel<LT, 2><<<grid, block, 0, s>>>(l, T, Ei, ki, r, idx, wo);
    else if (E <= 256)
        route_kernel<LT, 4><<<grid, block, 0, s>>>(l, T, Ei, ki, r, idx, wo);
    else if (E <= 512)
        route_kernel<LT, 8><<<grid, block, 0, s>>>(l, T, Ei, ki, r, idx, wo);
    else
        route_kernel<LT, 16><<<grid, block, 0, s>>>(l, T, Ei, ki, r, idx, wo);
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
