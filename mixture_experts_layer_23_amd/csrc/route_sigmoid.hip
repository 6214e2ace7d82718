// route_sigmoid.hip -- group-limited sigmoid routing (ruDNN user guide, section 10:
// route_sigmoid_grouped with GroupRoutingOptions top_k, groups, selected_groups,
// group_top_two, renormalize, scale, and an optional FP32 correction bias [E]).
//
// A group of G adjacent lanes owns one row of logits [T, E] (the lane layout of the softmax
// router: lane l of the group holds experts [l * NPER, (l + 1) * NPER), NPER = 16).  Per row, in FP32:
//   1. s_e = 1 / (1 + exp(-x_e)), evaluated in FP64 and rounded once to FP32 (sigmoid_f32);
//      corrected score c_e = s_e + bias_e (the bias only steers the choice).  s and c go to LDS.
//   2. Group scores from LDS, lane l taking groups l, l + G, ...: the largest c of the group,
//      or the sum of its two largest (group_top_two).  A NaN corrected score or a NaN group
//      score makes the row a NaN row (indices 0..k-1, NaN weights).
//   3. selected_groups rounds over order-preserving keys (score bits above the complemented
//      group id) choose the groups, ties to the lower group.
//   4. k rounds over the experts of the chosen groups (keys: c bits above the complemented
//      expert id; experts of other groups have key 0) choose the experts, ties to the lower id:
//      each lane sorts its largest keys once and a round takes the largest of the lanes' heads.
//   5. w_j = s_j, divided by the FP32 sum of the selected s (j ascending) when renormalising,
//      times scale, rounded once to the logits dtype.
#include "device.hpp"
#include "internal.hpp"
#include "route_select.hpp"  // group_max_key: the group maximum by DPP row permutations

namespace rudnn {

constexpr int SIG_THREADS = 256;


// FP32 value -> order-preserving 32 bits (-0 taken as +0), above the complement of an id.
__device__ __forceinline__ uint64_t sig_key(float v, uint32_t id) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0;
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(0xffffffffu - id);
}

// The sigmoid rounded once to FP32 from an FP64 evaluation: FP64 exp and a correctly rounded FP64
// division put the FP64 value within a few FP64 ulps of the exact one, so the FP32 result is the
// correctly rounded sigmoid unless the exact value lies within about 2^-50 (relative) of an FP32
// rounding midpoint.  An FP32 reciprocal of 1 + exp(-x) would leave the last FP32 bit uncertain,
// and with it the order of near-equal scores.  +inf -> 1, -inf -> 0, NaN -> NaN.
__device__ __forceinline__ float sigmoid_f32(float x) { return (float)(1.0 / (1.0 + exp(-(double)x))); }

// VEC: every lane's NPER logits (and bias entries) are whole, 16-byte aligned vectors inside the
// row (E % NPER == 0): one vector load each, and the scores go to LDS as 16-byte stores.
template <typename LT, int NPER, int G, bool VEC>
__global__ __launch_bounds__(SIG_THREADS) void route_sigmoid_kernel(const LT* __restrict__ logits,
                                                                    const float* __restrict__ bias, int64_t T, int E,
                                                                    int k, int groups, int nsel, int top_two,
                                                                    int renorm, float scale,
                                                                    uint32_t* __restrict__ idx, LT* __restrict__ w) {
    constexpr int RPB = SIG_THREADS / G;
    // groups per lane: groups <= min(E, 128) <= min(NPER * G, 128)
    constexpr int GPL = (128 + G - 1) / G < NPER ? (128 + G - 1) / G : NPER;
    extern __shared__ float smem[];  // c [RPB][E], s [RPB][E], winners [RPB][k]
    const int lane = lane_id(), l = lane % G, rb = threadIdx.x / G;
    const int64_t row = (int64_t)blockIdx.x * RPB + rb;
    const bool live = row < T;  // whole groups are live or not; no early return (shuffles, barriers)
    float* sc = smem + rb * E;
    float* ss = smem + RPB * E + rb * E;
    uint32_t* swin = reinterpret_cast<uint32_t*>(smem + 2 * RPB * E) + rb * k;
    const int e0 = l * NPER, per = E / groups;
    const LT* x = logits + (live ? row : 0) * (int64_t)E;

    // 1. sigmoid and corrected scores (slots past E are computed on a clamped id, then masked)
    float c[NPER];
    bool bad = false;
    if constexpr (VEC) {
        float xv[NPER], bv[NPER] = {};
        const bool in = e0 < E;  // whole chunks: a lane's entries are all in or all out
        {
            constexpr int PER16 = 16 / (int)sizeof(LT);
            LT t[NPER];
#pragma unroll
            for (int q = 0; q < NPER / PER16; ++q) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (in) v = *reinterpret_cast<const uint4*>(x + e0 + q * PER16);
                __builtin_memcpy(t + q * PER16, &v, 16);
            }
#pragma unroll
            for (int i = 0; i < NPER; ++i) xv[i] = to_f32(t[i]);
            if (bias && in) {
#pragma unroll
                for (int q = 0; q < NPER / 4; ++q) {
                    const float4 b4 = *reinterpret_cast<const float4*>(bias + e0 + q * 4);
                    bv[4 * q] = b4.x, bv[4 * q + 1] = b4.y, bv[4 * q + 2] = b4.z, bv[4 * q + 3] = b4.w;
                }
            }
        }
        float sgv[NPER];
#pragma unroll
        for (int i = 0; i < NPER; ++i) {
            sgv[i] = sigmoid_f32(xv[i]);
            c[i] = bias ? sgv[i] + bv[i] : sgv[i];
            bad |= in && c[i] != c[i];
        }
        if (in) {
#pragma unroll
            for (int q = 0; q < NPER / 4; ++q) {
                *reinterpret_cast<float4*>(sc + e0 + q * 4) = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
                *reinterpret_cast<float4*>(ss + e0 + q * 4) =
                    make_float4(sgv[4 * q], sgv[4 * q + 1], sgv[4 * q + 2], sgv[4 * q + 3]);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < NPER; ++s) {
            const int e = e0 + s;
            const int ec = e < E ? e : E - 1;
            const float xv = to_f32(x[ec]);
            const float sg = sigmoid_f32(xv);
            const float cv = bias ? sg + bias[ec] : sg;
            c[s] = cv;
            if (e < E) {
                bad |= cv != cv;
                sc[e] = cv;
                ss[e] = sg;
            }
        }
    }
    __syncthreads();

    // 2. group scores: from registers when each group is a power-of-two run of whole lane chunks,
    //    else from LDS (lane l taking groups l, l + G, ...)
    uint64_t gkey[GPL];
#pragma unroll
    for (int q = 0; q < GPL; ++q) gkey[q] = 0;
    const int lpg = per / NPER;  // lanes per group
    if (per % NPER == 0 && (lpg & (lpg - 1)) == 0) {
        float t1 = -INFINITY, t2 = -INFINITY;  // this lane's two largest
#pragma unroll
        for (int s = 0; s < NPER; ++s) {
            const float v = c[s];
            if (v > t1) {
                t2 = t1;
                t1 = v;
            } else if (v > t2) {
                t2 = v;
            }
        }
        for (int m = 1; m < lpg; m <<= 1) {  // merge the top two of the group's lanes
            const float o1 = __shfl_xor(t1, m, 64), o2 = __shfl_xor(t2, m, 64);
            const float n1 = fmaxf(t1, o1);
            const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
            t1 = n1, t2 = n2;
        }
        const int g = e0 / per;
        if (e0 < E && e0 % per == 0) {  // the group's first lane holds its key
            const float gs = top_two ? t1 + t2 : t1;
            bad |= gs != gs;
            gkey[0] = sig_key(gs, (uint32_t)g);
        }
    } else {
#pragma unroll
        for (int q = 0; q < GPL; ++q) {
            const int g = l + q * G;
            if (g < groups) {
                float t1 = -INFINITY, t2 = -INFINITY;  // the two largest corrected scores
                for (int i = 0; i < per; ++i) {
                    const float v = sc[g * per + i];
                    if (v > t1) {
                        t2 = t1;
                        t1 = v;
                    } else if (v > t2) {
                        t2 = v;
                    }
                }
                const float gs = top_two ? t1 + t2 : t1;
                bad |= gs != gs;
                gkey[q] = sig_key(gs, (uint32_t)g);
            }
        }
    }
    const int gshift = lane - l;
    const uint64_t gmask = G == 64 ? ~0ull : ((1ull << G) - 1ull);
    const bool nan_row = ((__ballot(bad) >> gshift) & gmask) != 0;

    // 3. groups by descending score
    uint32_t chosen[4] = {0u, 0u, 0u, 0u};  // bit g: group g selected (groups <= 128)
    uint64_t prev = ~0ull;
    for (int r = 0; r < nsel; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int q = 0; q < GPL; ++q) best = max(best, gkey[q] < prev ? gkey[q] : (uint64_t)0);
        const uint64_t win = group_max_key<G>(best);
        prev = win;
        const uint32_t g = 0xffffffffu - (uint32_t)win;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
            if ((int)(g >> 5) == wd) chosen[wd] |= 1u << (g & 31);
    }

    // 4. experts of the chosen groups by descending corrected score
    uint64_t key[NPER];
#pragma unroll
    for (int s = 0; s < NPER; ++s) {
        const int e = e0 + s;
        key[s] = 0;
        if (e < E) {
            const int g = e / per;
            const uint32_t wv = g < 32 ? chosen[0] : g < 64 ? chosen[1] : g < 96 ? chosen[2] : chosen[3];
            if ((wv >> (g & 31)) & 1u) key[s] = sig_key(c[s], (uint32_t)e);
        }
    }
    // each lane's largest keys sorted once; a round compares only the lists' heads
    float den = 0.f;
    auto take = [&](int j, uint64_t win) __attribute__((always_inline)) {
        const uint32_t id = 0xffffffffu - (uint32_t)win;
        const uint32_t idc = id < (uint32_t)E ? id : 0u;  // NaN rows may pick nothing valid
        den += ss[idc];
        if (l == 0) swin[j] = idc;
    };
    if constexpr (NPER == 16) {
        if (k <= 8) {  // block-uniform
            sort_top<8>(key);
            select_sorted<G, 8>(key, k, take);
        } else {
            sort_top<16>(key);
            select_sorted<G, 16>(key, k, take);
        }
    } else {
        sort_top<NPER>(key);
        select_sorted<G, NPER>(key, k, take);
    }
    __syncthreads();

    // 5. weights
    if (!live) return;
    for (int j = l; j < k; j += G) {
        if (nan_row) {
            idx[row * k + j] = (uint32_t)j;
            w[row * k + j] = from_f32<LT>(__builtin_nanf(""));
        } else {
            const uint32_t id = swin[j];
            const float v = renorm ? ss[id] / den : ss[id];
            idx[row * k + j] = id;
            w[row * k + j] = from_f32<LT>(v * scale);
        }
    }
}

template <typename LT, int NPER, int G>
static void launch_sig_g(const LT* l, const float* bias, int64_t T, int E, int k, int groups, int nsel, int top_two,
                         int renorm, float scale, uint32_t* idx, LT* w, hipStream_t s) {
    constexpr int RPB = SIG_THREADS / G;
    const dim3 grid((unsigned)((T + RPB - 1) / RPB)), block(SIG_THREADS);
    const size_t smem = (size_t)RPB * (2 * E + k) * 4;
    const bool vec = E % NPER == 0 && ((uintptr_t)l % 16) == 0 && ((uintptr_t)bias % 16) == 0;
    if (vec)
        route_sigmoid_kernel<LT, NPER, G, true><<<grid, block, smem, s>>>(l, bias, T, E, k, groups, nsel, top_two,
                                                                          renorm, scale, idx, w);
    else
        route_sigmoid_kernel<LT, NPER, G, false><<<grid, block, smem, s>>>(l, bias, T, E, k, groups, nsel, top_two,
                                                                           renorm, scale, idx, w);
}

template <typename LT>
static hipError_t launch_sig_t(const void* logits, const float* bias, int64_t T, int64_t E, int64_t k, int64_t groups,
                               int64_t nsel, bool top_two, bool renorm, double scale, uint32_t* idx, void* w,
                               hipStream_t s) {
    const LT* l = (const LT*)logits;
    LT* wo = (LT*)w;
    const int Ei = (int)E, ki = (int)k, gi = (int)groups, ni = (int)nsel, t2 = top_two ? 1 : 0, r = renorm ? 1 : 0;
    const float sc = (float)scale;
    timing_before(RUDNN_MOE_KERNEL_ROUTE_SIGMOID_GROUPED, s);
    // lanes per row: the smallest power of two G with 16 G >= E (16 experts per lane: fewer lanes
    // per row means fewer cross-lane steps in every selection round)
    if (E <= 16)
        launch_sig_g<LT, 16, 1>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else if (E <= 32)
        launch_sig_g<LT, 16, 2>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else if (E <= 64)
        launch_sig_g<LT, 16, 4>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else if (E <= 128)
        launch_sig_g<LT, 16, 8>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else if (E <= 256)
        launch_sig_g<LT, 16, 16>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else if (E <= 512)
        launch_sig_g<LT, 16, 32>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    else
        launch_sig_g<LT, 16, 64>(l, bias, T, Ei, ki, gi, ni, t2, r, sc, idx, wo, s);
    timing_after(RUDNN_MOE_KERNEL_ROUTE_SIGMOID_GROUPED, s);
    return hipGetLastError();
}

hipError_t launch_route_sigmoid_grouped(const void* logits, rudnn_moe_dtype ldt, const float* bias, int64_t T,
                                        int64_t E, int64_t k, int64_t groups, int64_t selected_groups, bool top_two,
                                        bool renorm, double scale, uint32_t* idx, void* w, hipStream_t s) {
    switch (ldt) {
    case RUDNN_MOE_F32:
        return launch_sig_t<float>(logits, bias, T, E, k, groups, selected_groups, top_two, renorm, scale, idx, w, s);
    case RUDNN_MOE_F16:
        return launch_sig_t<f16>(logits, bias, T, E, k, groups, selected_groups, top_two, renorm, scale, idx, w, s);
    default:
        return launch_sig_t<bf16>(logits, bias, T, E, k, groups, selected_groups, top_two, renorm, scale, idx, w, s);
    }
}

}  // namespace rudnn
