// device.hpp -- small device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rudnn {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // a 16-byte copy unit

// Storage <-> fp32.  Narrowing rounds to nearest even (v_cvt_pk_bf16_f32 / v_cvt_f16_f32).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(f16 v) { return (float)v; }
template <typename T>
__device__ __forceinline__ T from_f32(float v) { return (T)v; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Butterfly reductions over the 64 lanes of a wavefront; every lane receives the result.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Exclusive prefix sum over v[0..n) (n <= blockDim.x <= 1024) held one value per thread;
// returns thread i's exclusive sum and writes the grand total to *total (all threads).
// `scratch` is __shared__ int[16 + 1].
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int lane = lane_id(), wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    if (lane == 63) scratch[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nwaves; ++w) {
            int t = scratch[w];
            scratch[w] = run;
            run += t;
        }
        scratch[16] = run;
    }
    __syncthreads();
    int excl = scratch[wave] + incl - v;
    *total = scratch[16];
    __syncthreads();
    return excl;
}

}  // namespace rudnn
