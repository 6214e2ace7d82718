// combine.hip -- weighted combine back into token order (ruDNN user guide, sections 3 and 6:
// DispatchedTokens::combine restores the token order through the stored map and merges the
// expert outputs with the routing weights).
//
//   out[t, :] = dtype( sum_{j=0..k-1} w[t, j] * y[token_map[t, j], :] ),  FP32, j ascending.
//
// One wavefront per (token, 1 KiB piece of the row).  Lanes j < k load the token's map entry and
// weight; they are broadcast with readlane and every lane gathers one 16-byte vector of each of
// the k expert rows (all k loads issued before the arithmetic, streamed past the caches),
// accumulates in FP32 and writes one 16-byte vector of the output.  It is a pure gather: no
// atomics, deterministic.
// A map entry outside [0, T*k) (e.g. -1 for an expert id >= E at dispatch) makes the token's
// row NaN; nothing outside y is ever read.
// HBM traffic per token: k*H*s read + k*(4 + sw) read + H*s written.
#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

template <typename T, int N>
__device__ __forceinline__ void unpack(const u32x4& v, float (&f)[N]) {
    const T* p = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = to_f32(p[i]);
}
template <typename T, int N>
__device__ __forceinline__ u32x4 pack(const float (&f)[N]) {
    u32x4 v;
    T* p = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = from_f32<T>(f[i]);
    return v;
}

#ifndef RUDNN_COMBINE_NT
#define RUDNN_COMBINE_NT 1
#endif
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) {
    if (RUDNN_COMBINE_NT) return __builtin_nontemporal_load(p);
    return *p;
}
__device__ __forceinline__ void store_stream(u32x4 v, u32x4* p) {
    if (RUDNN_COMBINE_NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// One wavefront per (token, piece of 64 16-byte vectors of the row).  KMAX > 0: k <= KMAX known
// at compile time, so all k loads are issued before the arithmetic; KMAX == 0: any k.
template <typename T, typename WT, int KMAX>
__global__ __launch_bounds__(256) void combine_vec_kernel(const u32x4* __restrict__ y, const int32_t* __restrict__ map,
                                                          const WT* __restrict__ w, int64_t T_, int k,
                                                          int64_t row_vecs, int pieces, u32x4* __restrict__ out) {
    constexpr int N = 16 / sizeof(T);
    const int lane = lane_id();
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = wv / pieces;
    if (t >= T_) return;
    const int64_t i = (wv - t * pieces) * 64 + lane;
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = map[t * k + lane];
        my_w = to_f32(w[t * k + lane]);
    }
    const int64_t rows = T_ * k;  // y holds T*k rows; a map entry outside [0, rows) is invalid
    const bool bad = __ballot(lane < k && (my_row < 0 || my_row >= rows)) != 0;
    if (i >= row_vecs) return;
    float acc[N];
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = 0.f;
    if (bad) {
#pragma unroll
        for (int q = 0; q < N; ++q) acc[q] = __builtin_nanf("");
    } else if (KMAX > 0) {
        u32x4 v[KMAX > 0 ? KMAX : 1];
#pragma unroll
        for (int j = 0; j < (KMAX > 0 ? KMAX : 1); ++j)
            if (j < k) v[j] = load_stream(y + (int64_t)readlane(my_row, j) * row_vecs + i);
#pragma unroll
        for (int j = 0; j < (KMAX > 0 ? KMAX : 1); ++j) {
            if (j < k) {
                float f[N];
                unpack<T, N>(v[j], f);
                const float wj = readlane(my_w, j);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[q] += wj * f[q];
            }
        }
    } else {
        for (int j = 0; j < k; ++j) {
            float f[N];
            unpack<T, N>(load_stream(y + (int64_t)readlane(my_row, j) * row_vecs + i), f);
            const float wj = readlane(my_w, j);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[q] += wj * f[q];
        }
    }
    store_stream(pack<T, N>(acc), out + t * row_vecs + i);
}

// Element-wise form for rows whose byte length is not a multiple of 16.
template <typename T, typename WT>
__global__ __launch_bounds__(256) void combine_elem_kernel(const T* __restrict__ y, const int32_t* __restrict__ map,
                                                           const WT* __restrict__ w, int64_t T_, int k, int64_t H,
                                                           T* __restrict__ out) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T_) return;
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = map[t * k + lane];
        my_w = to_f32(w[t * k + lane]);
    }
    const int64_t rows = T_ * k;
    const bool bad = __ballot(lane < k && (my_row < 0 || my_row >= rows)) != 0;
    for (int64_t c = lane; c < H; c += 64) {
        float acc = 0.f;
        if (bad) {
            acc = __builtin_nanf("");
        } else {
            for (int j = 0; j < k; ++j) acc += readlane(my_w, j) * to_f32(y[(int64_t)readlane(my_row, j) * H + c]);
        }
        out[t * H + c] = from_f32<T>(acc);
    }
}

template <typename T, typename WT>
static void launch_combine_t(const void* y, const int32_t* map, const void* w, int64_t T_, int64_t k, int64_t H,
                             void* out, hipStream_t s) {
    const dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
    const int ki = (int)k;
    const size_t row_bytes = (size_t)H * sizeof(T);
    const bool vec = row_bytes % 16 == 0 && (uintptr_t)y % 16 == 0 && (uintptr_t)out % 16 == 0;
    if (!vec) {
        combine_elem_kernel<T, WT><<<grid, block, 0, s>>>((const T*)y, map, (const WT*)w, T_, ki, H, (T*)out);
        return;
    }
    const int64_t rv = (int64_t)(row_bytes / 16);
    const int pieces = (int)((rv + 63) / 64);
    const dim3 vgrid((unsigned)((T_ * pieces + 3) / 4));
    const u32x4* yv = (const u32x4*)y;
    u32x4* ov = (u32x4*)out;
    const WT* wt = (const WT*)w;
    if (k <= 1)
        combine_vec_kernel<T, WT, 1><<<vgrid, block, 0, s>>>(yv, map, wt, T_, ki, rv, pieces, ov);
    else if (k <= 2)
        combine_vec_kernel<T, WT, 2><<<vgrid, block, 0, s>>>(yv, map, wt, T_, ki, rv, pieces, ov);
    else if (k <= 4)
        combine_vec_kernel<T, WT, 4><<<vgrid, block, 0, s>>>(yv, map, wt, T_, ki, rv, pieces, ov);
    else if (k <= 8)
        combine_vec_kernel<T, WT, 8><<<vgrid, block, 0, s>>>(yv, map, wt, T_, ki, rv, pieces, ov);
    else
        combine_vec_kernel<T, WT, 0><<<vgrid, block, 0, s>>>(yv, map, wt, T_, ki, rv, pieces, ov);
}

template <typename T>
static void launch_combine_w(const void* y, const int32_t* map, const void* w, rudnn_moe_dtype wdt, int64_t T_,
                             int64_t k, int64_t H, void* out, hipStream_t s) {
    switch (wdt) {
    case RUDNN_MOE_F32: launch_combine_t<T, float>(y, map, w, T_, k, H, out, s); break;
    case RUDNN_MOE_F16: launch_combine_t<T, f16>(y, map, w, T_, k, H, out, s); break;
    default: launch_combine_t<T, bf16>(y, map, w, T_, k, H, out, s); break;
    }
}

hipError_t launch_combine(const void* y, rudnn_moe_dtype dt, const int32_t* map, const void* w, rudnn_moe_dtype wdt,
                          int64_t T_, int64_t k, int64_t H, void* out, hipStream_t s) {
    timing_before(RUDNN_MOE_KERNEL_COMBINE, s);
    switch (dt) {
    case RUDNN_MOE_F32: launch_combine_w<float>(y, map, w, wdt, T_, k, H, out, s); break;
    case RUDNN_MOE_F16: launch_combine_w<f16>(y, map, w, wdt, T_, k, H, out, s); break;
    default: launch_combine_w<bf16>(y, map, w, wdt, T_, k, H, out, s); break;
    }
    timing_after(RUDNN_MOE_KERNEL_COMBINE, s);
    return hipGetLastError();
}

}  // namespace rudnn
