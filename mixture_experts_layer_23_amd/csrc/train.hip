// train.hip -- first-order MoE training (ruDNN user guide, section 12 "MoE-Training erster
// Ordnung"): the FP32 router weights of a fixed selection and their logits gradient, and the
// backward of combine and of dispatch.
//
// selected_router (one wavefront per row): score = the softmax over all E experts of the row
// (max-subtracted, FP32) or the sigmoid of each logit; w_j = scale * score(i_j) / S with
// S = sum_j score(i_j) when renormalising (a repeated index counts each time), else 1.  The
// gradient of sum_j g_j w_j in closed form, with G_e = sum_{j: i_j = e} g_j, n_e = #{j: i_j = e}:
//   softmax:             dx_e = scale * p_e * (G_e - sum_j g_j p_{i_j})
//   softmax, renormed:   dx_e = scale * (p_e / S) * (G_e - n_e * sum_j g_j p_{i_j} / S)
//   sigmoid:             dx_e = scale * s_e (1 - s_e) * G_e
//   sigmoid, renormed:   dx_e = scale * s_e (1 - s_e) / S * (G_e - n_e * sum_j g_j s_{i_j} / S)
// rounded once to the logits dtype.  An index outside [0, E) makes the row NaN (weights and
// gradient); no memory is read through it.
//
// combine_backward (one wavefront per token): dexpert[map[t,j]] = dtype(w[t,j] * dout[t]) and
// dweights[t,j] = sum_h dout[t,h] * y[map[t,j],h] in FP32 (lane partial sums, then a wavefront
// sum; for k <= 8 every lane issues the dout vector and all k row vectors of an iteration before
// the arithmetic).  A token with a map entry outside [0, rows) gets NaN dweights and no dexpert
// row for that entry.  HBM per token: k*H*s (y) + H*s (dout) read, k*H*s written.
//
// dispatch_backward (one wavefront per token and 1 KiB piece of the row): dinput[t] =
// dtype(sum_j ddispatched[map[t,j]]), FP32, j ascending, no weights; NaN row for an invalid
// map entry.  HBM per token: k*H*s read + H*s written.
#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

// ---- selected router weights and their gradient ----

template <typename IT>
__device__ __forceinline__ int64_t load_index(const void* p, int64_t i) {
    return (int64_t)reinterpret_cast<const IT*>(p)[i];
}

template <typename LT, typename IT, bool BWD>
__global__ __launch_bounds__(256) void selected_router_kernel(const LT* __restrict__ logits, int64_t T, int E,
                                                              const void* __restrict__ indices, int k, int sigmoid,
                                                              int renorm, float scale,
                                                              const float* __restrict__ grad_weights,
                                                              float* __restrict__ weights,
                                                              LT* __restrict__ grad_logits) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wavefronts
    const LT* x = logits + t * E;
    int64_t ij = 0;
    bool valid = true;
    if (lane < k) {
        ij = load_index<IT>(indices, t * k + lane);
        valid = ij >= 0 && ij < E;
    }
    const bool bad = __ballot(!valid) != 0;
    const int my_e = valid && lane < k ? (int)ij : 0;

    // softmax normaliser (max-subtracted); unused for the sigmoid
    float m = -__builtin_inff(), z = 1.f;
    if (!sigmoid) {
        for (int e = lane; e < E; e += 64) m = fmaxf(m, to_f32(x[e]));
        m = wave_max(m);
        float s = 0.f;
        for (int e = lane; e < E; e += 64) s += expf(to_f32(x[e]) - m);
        z = wave_sum(s);
    }
    auto score = [&](float v) { return sigmoid ? 1.f / (1.f + expf(-v)) : expf(v - m) / z; };

    const float sc_j = lane < k && !bad ? score(to_f32(x[my_e])) : 0.f;
    const float S = renorm ? wave_sum(sc_j) : 1.f;
    if (!BWD) {
        if (lane < k) weights[t * k + lane] = bad ? __builtin_nanf("") : scale * sc_j / S;
        return;
    }
    LT* gx = grad_logits + t * E;
    if (bad) {
        for (int e = lane; e < E; e += 64) gx[e] = from_f32<LT>(__builtin_nanf(""));
        return;
    }
    const float g_j = lane < k ? grad_weights[t * k + lane] : 0.f;
    const float B = wave_sum(g_j * sc_j) / S;  // sum_j g_j score(i_j) / S
    for (int e = lane; e < E; e += 64) {
        float G = 0.f, n = 0.f;
        for (int j = 0; j < k; ++j) {
            const int ej = readlane(my_e, j);
            if (ej == e) {
                G += readlane(g_j, j);
                n += 1.f;
            }
        }
        const float v = to_f32(x[e]);
        float d;
        if (sigmoid) {
            const float s = 1.f / (1.f + expf(-v));
            d = renorm ? scale * s * (1.f - s) / S * (G - n * B) : scale * s * (1.f - s) * G;
        } else {
            const float p = expf(v - m) / z;
            d = renorm ? scale * (p / S) * (G - n * B) : scale * p * (G - B);
        }
        gx[e] = from_f32<LT>(d);
    }
}

template <typename LT, typename IT>
static void launch_sr(const void* logits, int64_t T, int64_t E, const void* idx, int64_t k, bool sigmoid,
                      bool renorm, double scale, const float* gw, float* w, void* gl, hipStream_t s) {
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    if (gw)
        selected_router_kernel<LT, IT, true><<<grid, block, 0, s>>>((const LT*)logits, T, (int)E, idx, (int)k,
                                                                    sigmoid, renorm, (float)scale, gw, nullptr,
                                                                    (LT*)gl);
    else
        selected_router_kernel<LT, IT, false><<<grid, block, 0, s>>>((const LT*)logits, T, (int)E, idx, (int)k,
                                                                     sigmoid, renorm, (float)scale, nullptr, w,
                                                                     nullptr);
}

template <typename LT>
static void launch_sr_i(const void* logits, int64_t T, int64_t E, const void* idx, rudnn_moe_index_type it,
                        int64_t k, bool sigmoid, bool renorm, double scale, const float* gw, float* w, void* gl,
                        hipStream_t s) {
    switch (it) {
    case RUDNN_MOE_I32: launch_sr<LT, int32_t>(logits, T, E, idx, k, sigmoid, renorm, scale, gw, w, gl, s); break;
    case RUDNN_MOE_I64: launch_sr<LT, int64_t>(logits, T, E, idx, k, sigmoid, renorm, scale, gw, w, gl, s); break;
    default: launch_sr<LT, uint32_t>(logits, T, E, idx, k, sigmoid, renorm, scale, gw, w, gl, s); break;
    }
}

hipError_t launch_selected_router(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, const void* idx,
                                  rudnn_moe_index_type it, int64_t k, bool sigmoid, bool renorm, double scale,
                                  const float* grad_weights, float* weights, void* grad_logits, hipStream_t s) {
    timing_before(RUDNN_MOE_KERNEL_SELECTED_ROUTER, s);
    switch (ldt) {
    case RUDNN_MOE_F32:
        launch_sr_i<float>(logits, T, E, idx, it, k, sigmoid, renorm, scale, grad_weights, weights, grad_logits, s);
        break;
    case RUDNN_MOE_F16:
        launch_sr_i<f16>(logits, T, E, idx, it, k, sigmoid, renorm, scale, grad_weights, weights, grad_logits, s);
        break;
    default:
        launch_sr_i<bf16>(logits, T, E, idx, it, k, sigmoid, renorm, scale, grad_weights, weights, grad_logits, s);
        break;
    }
    timing_after(RUDNN_MOE_KERNEL_SELECTED_ROUTER, s);
    return hipGetLastError();
}

// ---- combine and dispatch backward (16-byte vectors of the rows) ----

template <typename T, int N>
__device__ __forceinline__ void unpack16(const u32x4& v, float (&f)[N]) {
    const T* p = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = to_f32(p[i]);
}
template <typename T, int N>
__device__ __forceinline__ u32x4 pack16(const float (&f)[N]) {
    u32x4 v;
    T* p = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = from_f32<T>(f[i]);
    return v;
}

// KMAX > 0: k <= KMAX known at compile time, so each lane issues the dout vector and all k expert
// row vectors of an iteration before the arithmetic (the rows read once, streamed past the
// caches); KMAX == 0: any k, one slot at a time.
template <typename T, typename WT, int KMAX>
__global__ __launch_bounds__(256) void combine_backward_kernel(const u32x4* __restrict__ y,
                                                               const int32_t* __restrict__ map,
                                                               const WT* __restrict__ w,
                                                               const u32x4* __restrict__ dout, int64_t T_, int k,
                                                               int64_t rows, int64_t row_vecs,
                                                               u32x4* __restrict__ dexp, float* __restrict__ dw) {
    constexpr int N = 16 / sizeof(T);
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T_) return;
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = map[t * k + lane];
        my_w = to_f32(w[t * k + lane]);
    }
    const bool ok_me = my_row >= 0 && my_row < rows;
    const bool bad = __ballot(lane < k && !ok_me) != 0;
    float part = 0.f;  // lane j < k ends with dweights[t, j]
    if constexpr (KMAX > 0) {
        float acc[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) acc[j] = 0.f;
        for (int64_t i = lane; i < row_vecs; i += 64) {
            const u32x4 gv = dout[t * row_vecs + i];
            u32x4 v[KMAX];
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                const int r = readlane(my_row, j);  // wave-uniform
                if (j < k && r >= 0 && r < rows) v[j] = __builtin_nontemporal_load(y + (int64_t)r * row_vecs + i);
            }
            float g[N];
            unpack16<T, N>(gv, g);
#pragma unroll
            for (int j = 0; j < KMAX; ++j) {
                const int r = readlane(my_row, j);
                if (!(j < k && r >= 0 && r < rows)) continue;
                const float wj = readlane(my_w, j);
                float yy[N], o[N];
                unpack16<T, N>(v[j], yy);
#pragma unroll
                for (int q = 0; q < N; ++q) {
                    acc[j] += g[q] * yy[q];
                    o[q] = wj * g[q];
                }
                dexp[(int64_t)r * row_vecs + i] = pack16<T, N>(o);
            }
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            if (j >= k) break;
            const float sj = wave_sum(acc[j]);
            if (lane == j) part = sj;
        }
    } else {
        for (int j = 0; j < k; ++j) {
            const int r = readlane(my_row, j);
            const float wj = readlane(my_w, j);
            const bool ok = r >= 0 && r < rows;  // wave-uniform
            float acc = 0.f;
            for (int64_t i = lane; i < row_vecs; i += 64) {
                float g[N], o[N];
                unpack16<T, N>(dout[t * row_vecs + i], g);
                if (ok) {
                    float yy[N];
                    unpack16<T, N>(y[(int64_t)r * row_vecs + i], yy);
#pragma unroll
                    for (int q = 0; q < N; ++q) {
                        acc += g[q] * yy[q];
                        o[q] = wj * g[q];
                    }
                    dexp[(int64_t)r * row_vecs + i] = pack16<T, N>(o);
                }
            }
            acc = wave_sum(acc);
            if (lane == j) part = acc;
        }
    }
    if (lane < k) dw[t * k + lane] = bad ? __builtin_nanf("") : part;
}

// KMAX as in combine_backward_kernel: all k row vectors loaded before the sum.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void dispatch_backward_kernel(const u32x4* __restrict__ d,
                                                                const int32_t* __restrict__ map, int64_t T_, int k,
                                                                int64_t rows, int64_t row_vecs, int pieces,
                                                                u32x4* __restrict__ out) {
    constexpr int N = 16 / sizeof(T);
    const int lane = lane_id();
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = wv / pieces;
    if (t >= T_) return;
    const int64_t i = (wv - t * pieces) * 64 + lane;
    const int my_row = lane < k ? map[t * k + lane] : -1;
    const bool bad = __ballot(lane < k && (my_row < 0 || my_row >= rows)) != 0;
    if (i >= row_vecs) return;
    float acc[N];
#pragma unroll
    for (int q = 0; q < N; ++q) acc[q] = bad ? __builtin_nanf("") : 0.f;
    if (!bad && KMAX > 0) {
        u32x4 v[KMAX > 0 ? KMAX : 1];
#pragma unroll
        for (int j = 0; j < (KMAX > 0 ? KMAX : 1); ++j)
            if (j < k) v[j] = __builtin_nontemporal_load(d + (int64_t)readlane(my_row, j) * row_vecs + i);
#pragma unroll
        for (int j = 0; j < (KMAX > 0 ? KMAX : 1); ++j) {
            if (j < k) {
                float f[N];
                unpack16<T, N>(v[j], f);
#pragma unroll
                for (int q = 0; q < N; ++q) acc[q] += f[q];
            }
        }
    } else if (!bad) {
        for (int j = 0; j < k; ++j) {
            float f[N];
            unpack16<T, N>(d[(int64_t)readlane(my_row, j) * row_vecs + i], f);
#pragma unroll
            for (int q = 0; q < N; ++q) acc[q] += f[q];
        }
    }
    out[t * row_vecs + i] = pack16<T, N>(acc);
}

template <typename DT, typename WT>
static void launch_cb(const void* y, const int32_t* map, const void* w, const void* dout, int64_t T, int64_t k,
                      int64_t H, int64_t rows, void* dexp, float* dw, hipStream_t s) {
    const int64_t row_vecs = H * (int64_t)sizeof(DT) / 16;
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const u32x4 *yv = (const u32x4*)y, *gv = (const u32x4*)dout;
    const WT* wt = (const WT*)w;
    u32x4* ov = (u32x4*)dexp;
    const int ki = (int)k;
    if (k <= 2)
        combine_backward_kernel<DT, WT, 2><<<grid, block, 0, s>>>(yv, map, wt, gv, T, ki, rows, row_vecs, ov, dw);
    else if (k <= 4)
        combine_backward_kernel<DT, WT, 4><<<grid, block, 0, s>>>(yv, map, wt, gv, T, ki, rows, row_vecs, ov, dw);
    else if (k <= 8)
        combine_backward_kernel<DT, WT, 8><<<grid, block, 0, s>>>(yv, map, wt, gv, T, ki, rows, row_vecs, ov, dw);
    else
        combine_backward_kernel<DT, WT, 0><<<grid, block, 0, s>>>(yv, map, wt, gv, T, ki, rows, row_vecs, ov, dw);
}

template <typename DT>
static void launch_cb_w(const void* y, const int32_t* map, const void* w, rudnn_moe_dtype wdt, const void* dout,
                        int64_t T, int64_t k, int64_t H, int64_t rows, void* dexp, float* dw, hipStream_t s) {
    switch (wdt) {
    case RUDNN_MOE_F32: launch_cb<DT, float>(y, map, w, dout, T, k, H, rows, dexp, dw, s); break;
    case RUDNN_MOE_F16: launch_cb<DT, f16>(y, map, w, dout, T, k, H, rows, dexp, dw, s); break;
    default: launch_cb<DT, bf16>(y, map, w, dout, T, k, H, rows, dexp, dw, s); break;
    }
}

hipError_t launch_combine_backward(const void* y, rudnn_moe_dtype dt, const int32_t* map, const void* w,
                                   rudnn_moe_dtype wdt, const void* dout, int64_t T, int64_t k, int64_t H,
                                   int64_t rows, void* dexp, float* dw, hipStream_t s) {
    timing_before(RUDNN_MOE_KERNEL_COMBINE_BACKWARD, s);
    switch (dt) {
    case RUDNN_MOE_F32: launch_cb_w<float>(y, map, w, wdt, dout, T, k, H, rows, dexp, dw, s); break;
    case RUDNN_MOE_F16: launch_cb_w<f16>(y, map, w, wdt, dout, T, k, H, rows, dexp, dw, s); break;
    default: launch_cb_w<bf16>(y, map, w, wdt, dout, T, k, H, rows, dexp, dw, s); break;
    }
    timing_after(RUDNN_MOE_KERNEL_COMBINE_BACKWARD, s);
    return hipGetLastError();
}

template <typename DT>
static void launch_db(const void* d, const int32_t* map, int64_t T, int64_t k, int64_t H, int64_t rows, void* out,
                      hipStream_t s) {
    const int64_t row_vecs = H * (int64_t)sizeof(DT) / 16;
    const int pieces = (int)((row_vecs + 63) / 64);
    const int64_t waves = T * pieces;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    const u32x4* dv = (const u32x4*)d;
    u32x4* ov = (u32x4*)out;
    const int ki = (int)k;
    if (k <= 2)
        dispatch_backward_kernel<DT, 2><<<grid, block, 0, s>>>(dv, map, T, ki, rows, row_vecs, pieces, ov);
    else if (k <= 4)
        dispatch_backward_kernel<DT, 4><<<grid, block, 0, s>>>(dv, map, T, ki, rows, row_vecs, pieces, ov);
    else if (k <= 8)
        dispatch_backward_kernel<DT, 8><<<grid, block, 0, s>>>(dv, map, T, ki, rows, row_vecs, pieces, ov);
    else
        dispatch_backward_kernel<DT, 0><<<grid, block, 0, s>>>(dv, map, T, ki, rows, row_vecs, pieces, ov);
}

hipError_t launch_dispatch_backward(const void* d, rudnn_moe_dtype dt, const int32_t* map, int64_t T, int64_t k,
                                    int64_t H, int64_t rows, void* out, hipStream_t s) {
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_BACKWARD, s);
    switch (dt) {
    case RUDNN_MOE_F32: launch_db<float>(d, map, T, k, H, rows, out, s); break;
    case RUDNN_MOE_F16: launch_db<f16>(d, map, T, k, H, rows, out, s); break;
    default: launch_db<bf16>(d, map, T, k, H, rows, out, s); break;
    }
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_BACKWARD, s);
    return hipGetLastError();
}

}  // namespace rudnn
