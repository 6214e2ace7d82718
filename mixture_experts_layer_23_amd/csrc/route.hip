// route.hip -- softmax / top-k routing (ruDNN user guide, section 4 "Routing contract").
//
// A group of G adjacent lanes owns one row of logits [T, E] (G = 1 .. 64, a power of two, so a
// wavefront covers 64 / G rows); lane l of the group holds experts [l * NPER, (l + 1) * NPER),
// so a wavefront's loads cover 64 / G consecutive rows contiguously.
//
// Softmax is strictly increasing, so the k largest probabilities are the experts with the k
// largest logits; selection therefore runs on the logits themselves (exact), with equal logits
// going to the lower id, and only the selected probabilities are formed.
//   1. NaN-row test: a group ballot over "x is NaN or +inf" and over "x is not -inf".
//   2. Keys: the logit's bits mapped to an order-preserving unsigned integer (-0 taken as +0),
//      above the complement of the expert id, so a larger key is a larger logit or, for equal
//      logits, a lower id.  16-bit logits give 32-bit keys, FP32 logits 64-bit keys.
//   3. k rounds: every lane takes its largest key below the previous winner, the group takes
//      the largest of those.  The first winner is the row maximum m.
//   4. FP32: e_j = exp(x_j - m) for the winners; w_j = e_j / sum_j e_j with renormalisation,
//      else w_j = e_j / sum over all experts of exp(x - m); one rounding to the logits dtype.
// HBM traffic per row: E * sizeof(logits) read, k * (4 + sizeof(logits)) written.
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

constexpr int ROUTE_THREADS = 256;

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
template <int G>
__device__ __forceinline__ uint32_t group_max_key(uint32_t key) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) key = max(key, (uint32_t)__shfl_xor(key, m, 64));
    return key;
}
template <int G>
__device__ __forceinline__ uint64_t group_max_key(uint64_t key) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)key, m, 64), hi = __shfl_xor((uint32_t)(key >> 32), m, 64);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        key = o > key ? o : key;
    }
    return key;
}

// Logit bits, their order-preserving key and back.
template <typename LT>
struct RouteBits;
template <>
struct RouteBits<float> {
    typedef uint32_t raw;
    typedef uint64_t key;
    static constexpr int SHIFT = 32;
    static constexpr raw SIGN = 0x80000000u, EXP = 0x7f800000u;
};
template <>
struct RouteBits<bf16> {
    typedef uint16_t raw;
    typedef uint32_t key;
    static constexpr int SHIFT = 16;
    static constexpr raw SIGN = 0x8000u, EXP = 0x7f80u;
};
template <>
struct RouteBits<f16> {
    typedef uint16_t raw;
    typedef uint32_t key;
    static constexpr int SHIFT = 16;
    static constexpr raw SIGN = 0x8000u, EXP = 0x7c00u;
};

template <typename LT>
__device__ __forceinline__ typename RouteBits<LT>::key make_key(typename RouteBits<LT>::raw b, int id) {
    typedef RouteBits<LT> B;
    typedef typename B::key K;
    typedef typename B::raw R;
    if (b == B::SIGN) b = 0;                                  // -0 -> +0
    const R ord = (b & B::SIGN) ? (R)~b : (R)(b | B::SIGN);  // order-preserving
    const K low = (K)(((K)1 << B::SHIFT) - 1);
    return ((K)ord << B::SHIFT) | (low - (K)id);
}
template <typename LT>
__device__ __forceinline__ float key_logit(typename RouteBits<LT>::key k) {
    typedef RouteBits<LT> B;
    typedef typename B::raw R;
    const R ord = (R)(k >> B::SHIFT);
    const R b = (ord & B::SIGN) ? (R)(ord & ~B::SIGN) : (R)~ord;
    LT v;
    __builtin_memcpy(&v, &b, sizeof(v));
    return to_f32(v);
}
template <typename LT>
__device__ __forceinline__ uint32_t key_id(typename RouteBits<LT>::key k) {
    typedef typename RouteBits<LT>::key K;
    const K low = (K)(((K)1 << RouteBits<LT>::SHIFT) - 1);
    return (uint32_t)(low - (k & low));
}

// VEC: the row chunk of every lane is NPER whole elements, 16-byte aligned (E % NPER == 0).
template <typename LT, int NPER, int G, bool VEC>
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const LT* __restrict__ logits, int64_t T, int E, int k,
                                                              int renorm, uint32_t* __restrict__ idx,
                                                              LT* __restrict__ w) {
    typedef RouteBits<LT> B;
    typedef typename B::raw R;
    typedef typename B::key K;
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
    const R NEG_INF = (R)(B::SIGN | B::EXP), POS_INF = B::EXP;
    bool nan_or_posinf = false, not_neginf = false;
    K key[NPER];
#pragma unroll
    for (int s = 0; s < NPER; ++s) {
        const bool in = e0 + s < E;
        const R b = raw[s];
        nan_or_posinf |= in && (((R)(b & (R)~B::SIGN) > B::EXP) || b == POS_INF);
        not_neginf |= in && b != NEG_INF;
        key[s] = in ? make_key<LT>(b, e0 + s) : (K)0;  // 0: below every real key
    }
    const int gshift = lane - l;  // first lane of the group
    const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull);
    const bool nan_row =
        ((__ballot(nan_or_posinf) >> gshift) & gmask) != 0 || ((__ballot(not_neginf) >> gshift) & gmask) == 0;

    K prev = ~(K)0;
    float m = 0.f, den = 0.f;
    for (int j = 0; j < k; ++j) {
        K best = 0;
#pragma unroll
        for (int s = 0; s < NPER; ++s) best = max(best, key[s] < prev ? key[s] : (K)0);
        const K win = group_max_key<G>(best);
        prev = win;
        const float xw = key_logit<LT>(win);
        if (j == 0) m = xw;
        const float e = expf(xw - m);  // -inf logits give 0 exactly
        den += e;
        if (l == 0) {
            si[j] = key_id<LT>(win);
            se[j] = e;
        }
    }
    if (!renorm) {  // denominator over all experts
        float sum = 0.f;
#pragma unroll
        for (int s = 0; s < NPER; ++s) {
            if (e0 + s < E) {
                LT v;
                __builtin_memcpy(&v, &raw[s], sizeof(v));
                sum += expf(to_f32(v) - m);
            }
        }
        den = group_sum<G>(sum);
    }
    __syncthreads();
    if (!live) return;
    for (int j = l; j < k; j += G) {
        if (nan_row) {
            // NaN row: NaN weights, indices 0..k-1 (every probability NaN, read as a full tie)
            idx[row * k + j] = (uint32_t)j;
            w[row * k + j] = from_f32<LT>(__builtin_nanf(""));
        } else {
            idx[row * k + j] = si[j];
            w[row * k + j] = from_f32<LT>(se[j] / den);
        }
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
