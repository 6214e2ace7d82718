// route_select.hpp -- the per-row top-k selection of softmax routing (ruDNN user guide,
// section 4 "Routing contract"), shared by the router that reads logits from memory
// (route.hip) and the router fused behind the gate projection (route_projected.hip).
//
// A group of G adjacent lanes (G = 1 .. 64, a power of two) owns one row of E logits; lane l of
// the group holds the raw bits of experts [l * NPER, (l + 1) * NPER).
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
#pragma once

#include "device.hpp"

namespace rudnn {

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

// Routes one row held by a group of G lanes (steps 1-4 above) and, for a live row, stores its
// k indices and weights at idx/w[row * k ..].  raw: this lane's NPER logit bits, experts
// e0 = (lane % G) * NPER onwards (entries at e >= E are ignored).  si/se: this group's k-entry
// LDS scratch (winner ids, e_j), touched only by live rows.  Every thread of the block must call
// it together (it holds a barrier); whole groups are live or not.
template <typename LT, int NPER, int G>
__device__ __forceinline__ void route_row(const typename RouteBits<LT>::raw (&raw)[NPER], int E, int k, int renorm,
                                          bool live, int64_t row, uint32_t* si, float* se, uint32_t* __restrict__ idx,
                                          LT* __restrict__ w) {
    typedef RouteBits<LT> B;
    typedef typename B::raw R;
    typedef typename B::key K;
    const int lane = lane_id(), l = lane % G, e0 = l * NPER;
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
        if (live && l == 0) {
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
    if (live) {
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
}

}  // namespace rudnn
