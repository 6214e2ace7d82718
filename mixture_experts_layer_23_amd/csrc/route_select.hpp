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
// Lane permutations inside the 16-lane rows of a wavefront, as DPP moves (no LDS round trip):
// STEP 0 swaps lanes 2i and 2i + 1, STEP 1 swaps the pairs of each quad, STEP 2 mirrors each
// 8-lane half row, STEP 3 each 16-lane row.  Taking a maximum with STEP 0, 1, .. in turn leaves
// every aligned group of 2, 4, 8, 16 lanes holding its group's maximum (a mirror pairs each lane
// with one in the other half of its group, which by then holds that half's maximum).
template <int STEP>
__device__ __forceinline__ uint32_t row_perm(uint32_t v) {
    constexpr int CTRL = STEP == 0 ? 0xb1 : STEP == 1 ? 0x4e : STEP == 2 ? 0x141 : 0x140;  // quad_perm / mirrors
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int STEP>
__device__ __forceinline__ uint64_t row_perm(uint64_t v) {
    return ((uint64_t)row_perm<STEP>((uint32_t)(v >> 32)) << 32) | row_perm<STEP>((uint32_t)v);
}
template <typename K>
__device__ __forceinline__ K xor_lanes(K v, int m) {
    if constexpr (sizeof(K) == 4) {
        return (K)__shfl_xor((uint32_t)v, m, 64);
    } else {
        const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
        return ((K)hi << 32) | lo;
    }
}
// The largest key of each aligned group of G lanes, in every lane of the group.
template <int G, typename K>
__device__ __forceinline__ K group_max_key(K key) {
    if constexpr (G >= 2) key = max(key, row_perm<0>(key));
    if constexpr (G >= 4) key = max(key, row_perm<1>(key));
    if constexpr (G >= 8) key = max(key, row_perm<2>(key));
    if constexpr (G >= 16) key = max(key, row_perm<3>(key));
    if constexpr (G >= 32) key = max(key, xor_lanes(key, 16));
    if constexpr (G >= 64) key = max(key, xor_lanes(key, 32));
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
                si[j] = (uint32_t)j;  // si keeps the stored ids (read by the dispatch epilogue)
                w[row * k + j] = from_f32<LT>(__builtin_nanf(""));
            } else {
                idx[row * k + j] = si[j];
                w[row * k + j] = from_f32<LT>(se[j] / den);
            }
        }
    }
}

// The same routing for 16-bit logits whose lanes hold whole NPER-element chunks (E % NPER == 0),
// with less VALU work per row:
//   * codes: ord = 0x8000 + |x| for x >= +0 and 0x8000 - |x| for x <= -0 (both zeros 0x8000),
//     built two logits at a time with packed 16-bit integer operations; key = ord << 16 above
//     the complemented id, as in make_key (ord differs from make_key's by a constant for
//     negatives, which leaves the order unchanged);
//   * NaN-row test from the lane's largest and smallest code: +inf or +NaN give ord >= 0x8000 +
//     EXP, -NaN ord < 0x8000 - EXP, -inf exactly 0x8000 - EXP;
//   * selection: each lane sorts its L largest keys once (a bitonic network; L = 8 takes the top
//     8 of 16 by sorting both halves and merging), then every round takes the group maximum of
//     the lanes' heads and the winning lane shifts its list by one.  Since keys are unique in a
//     row, this yields the same k winners in the same order as the k rounds of route_row.
template <typename LT>
__device__ __forceinline__ float ord_logit(uint32_t key) {
    const uint32_t ord = key >> 16;
    const uint16_t b = ord >= 0x8000u ? (uint16_t)(ord - 0x8000u) : (uint16_t)(0x8000u | (0x8000u - ord));
    LT v;
    __builtin_memcpy(&v, &b, sizeof(v));
    return to_f32(v);
}

// key[a] >= key[b] afterwards
template <typename K>
__device__ __forceinline__ void key_order(K& a, K& b) {
    const K x = a, y = b;
    if constexpr (sizeof(K) == 4) {
        a = max(x, y);
        b = min(x, y);
    } else {
        const bool gt = x > y;
        a = gt ? x : y;
        b = gt ? y : x;
    }
}

// Bitonic sort, descending, of key[B .. B + N) (N a power of two).
template <int B, int N, typename K, int NPER>
__device__ __forceinline__ void key_sort(K (&key)[NPER]) {
#pragma unroll
    for (int kk = 2; kk <= N; kk <<= 1)
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & kk) == 0)
                        key_order(key[B + i], key[B + l]);
                    else
                        key_order(key[B + l], key[B + i]);
                }
            }
}

// The L largest of the NPER keys, sorted descending, in key[0 .. L): the whole chunk (L == NPER)
// or the top 8 of 16 (sort both halves, keep the larger of key[i] and key[15 - i], which leaves
// the top 8 as one bitonic sequence, and merge it).
template <int L, typename K, int NPER>
__device__ __forceinline__ void sort_top(K (&key)[NPER]) {
    static_assert(L == NPER || (L == 8 && NPER == 16), "the whole chunk or the top 8 of 16");
    if constexpr (L == NPER) {
        key_sort<0, NPER>(key);
    } else {
        key_sort<0, 8>(key);
        key_sort<8, 8>(key);
#pragma unroll
        for (int i = 0; i < 8; ++i) key[i] = key[i] > key[15 - i] ? key[i] : key[15 - i];  // max
#pragma unroll
        for (int j = 4; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i ^ j) > i) key_order(key[i], key[i ^ j]);
    }
}

// k rounds over per-lane lists sorted by sort_top<L>: the group maximum of the lists' heads wins
// and its lane shifts its list by one (keys are unique in a row, so exactly one lane holds it).
// Calls on_win(j, win) for round j.
template <int G, int L, typename K, int NPER, typename F>
__device__ __forceinline__ void select_sorted(K (&key)[NPER], int k, F on_win) {
    for (int j = 0; j < k; ++j) {
        const K win = group_max_key<G>(key[0]);
        const bool hit = key[0] == win;
#pragma unroll
        for (int p = 0; p < L - 1; ++p) key[p] = hit ? key[p + 1] : key[p];
        key[L - 1] = hit ? (K)0 : key[L - 1];
        on_win(j, win);
    }
}

template <typename LT, int NPER, int G, int L>
__device__ __forceinline__ void route_row_sorted(const uint16_t (&raw)[NPER], int E, int k, int renorm, bool live,
                                                 int64_t row, uint32_t* si, float* se, uint32_t* __restrict__ idx,
                                                 LT* __restrict__ w) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    typedef short ss2 __attribute__((ext_vector_type(2)));
    static_assert(NPER % 2 == 0 && (L == NPER || (L == 8 && NPER == 16)), "list of the whole chunk or top 8 of 16");
    constexpr uint32_t EXP = RouteBits<LT>::EXP, POS = 0x8000u + EXP, NEG = 0x8000u - EXP;
    const int lane = lane_id(), l = lane % G, e0 = l * NPER;
    const bool lane_in = e0 < E;  // whole chunks: a lane's entries are all in or all out
    uint32_t key[NPER];
    us2 omax = {0, 0}, omin = {0xffff, 0xffff};
#pragma unroll
    for (int p = 0; p < NPER / 2; ++p) {
        us2 v;
        __builtin_memcpy(&v, &raw[2 * p], sizeof(v));
        const us2 neg = (us2)(((ss2)v) >> (ss2)15);  // 0xffff where the sign bit is set
        const us2 mag = v & (us2)0x7fff;
        const us2 ord = (us2)0x8000 + ((mag ^ neg) - neg);
        omax = __builtin_elementwise_max(omax, ord);
        omin = __builtin_elementwise_min(omin, ord);
        key[2 * p] = lane_in ? (((uint32_t)ord.x << 16) | (0xffffu - (uint32_t)(e0 + 2 * p))) : 0u;
        key[2 * p + 1] = lane_in ? (((uint32_t)ord.y << 16) | (0xffffu - (uint32_t)(e0 + 2 * p + 1))) : 0u;
    }
    const uint32_t hi = max((uint32_t)omax.x, (uint32_t)omax.y), lo = min((uint32_t)omin.x, (uint32_t)omin.y);
    // the row maximum (the first winner's logit) and, without renormalisation, the denominator over
    // all experts, before the sort: the raw logits are then dead during the selection
    const float m = ord_logit<LT>(group_max_key<G>(lane_in ? hi : 0u) << 16);
    float den = 0.f;
    if (!renorm) {
        float sum = 0.f;
        if (lane_in) {
#pragma unroll
            for (int s = 0; s < NPER; ++s) {
                LT v;
                __builtin_memcpy(&v, &raw[s], sizeof(v));
                sum += expf(to_f32(v) - m);
            }
        }
        den = group_sum<G>(sum);
    }
    const bool nan_or_posinf = lane_in && (hi >= POS || lo < NEG);
    const bool not_neginf = lane_in && !(hi == NEG && lo == NEG);
    const int gshift = lane - l;  // first lane of the group
    const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull);
    const bool nan_row =
        ((__ballot(nan_or_posinf) >> gshift) & gmask) != 0 || ((__ballot(not_neginf) >> gshift) & gmask) == 0;

    sort_top<L>(key);

    select_sorted<G, L>(key, k, [&](int j, uint32_t win) __attribute__((always_inline)) {
        const float e = expf(ord_logit<LT>(win) - m);  // -inf logits give 0 exactly
        if (renorm) den += e;
        if (live && l == 0) {
            si[j] = 0xffffu - (win & 0xffffu);
            se[j] = e;
        }
    });
    __syncthreads();
    if (live) {
        for (int j = l; j < k; j += G) {
            if (nan_row) {
                idx[row * k + j] = (uint32_t)j;
                si[j] = (uint32_t)j;
                w[row * k + j] = from_f32<LT>(__builtin_nanf(""));
            } else {
                idx[row * k + j] = si[j];
                w[row * k + j] = from_f32<LT>(se[j] / den);
            }
        }
    }
}

}  // namespace rudnn
