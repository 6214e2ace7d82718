// internal.hpp -- host-side contract between the C-ABI layer (api.cpp) and the kernel files.
// Launchers only enqueue; argument validation happens in api.cpp before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/rudnn_moe.h"

namespace rudnn {

// Dispatch works on chunks of consecutive (token, slot) pairs; one block of the count and rank
// kernels owns one chunk.  The chunk is 256..4096 pairs (a multiple of the 256-thread block),
// about pairs / 512: enough blocks for the count and rank kernels.  Workspace: [nchunks, E]
// int32 per-chunk counts that the scan kernel turns into per-chunk bases in place, then [E]
// int32 expert totals.
#ifndef RUDNN_DISPATCH_CHUNKS
#define RUDNN_DISPATCH_CHUNKS 512
#endif
inline int64_t dispatch_chunk(int64_t pairs) {
    int64_t c = 256;
    while (c < 4096 && c * RUDNN_DISPATCH_CHUNKS < pairs) c *= 2;
    return c;
}
inline int64_t dispatch_chunks(int64_t pairs) {
    const int64_t c = dispatch_chunk(pairs);
    return (pairs + c - 1) / c;
}

// Kernel limits (documented in rudnn_moe.h as RUDNN_MOE_ERR_UNSUPPORTED).
constexpr int64_t MAX_EXPERTS = 1024;
constexpr int64_t MAX_TOP_K = 64;

inline size_t align_up(size_t n, size_t a = 256) { return (n + a - 1) / a * a; }
// Bytes of the dispatch workspace (see dispatch_chunk) and the offset of its expert totals.
inline size_t dispatch_totals_offset(int64_t pairs, int64_t E) {
    return align_up(sizeof(int32_t) * (size_t)(dispatch_chunks(pairs) * E));
}
inline size_t dispatch_workspace_bytes(int64_t pairs, int64_t E) {
    return dispatch_totals_offset(pairs, E) + align_up(sizeof(int32_t) * (size_t)E);
}
inline size_t dtype_size(rudnn_moe_dtype d) { return d == RUDNN_MOE_F32 ? 4 : 2; }

// Host-side checks shared by the entry points (api.cpp).  check_device: every pointer is device
// (or managed) memory of the stream's device.  check_dispatch_args: the argument checks of
// rudnn_moe_dispatch except those of its workspace.  dispatch_no_pairs: the T = 0 case (all
// offsets zero).
rudnn_moe_status check_device(hipStream_t s, std::initializer_list<const void*> ptrs);
rudnn_moe_status runtime(hipError_t e);
rudnn_moe_status check_dispatch_args(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input,
                                     rudnn_moe_dtype dt, int64_t H, const void* dispatched, const int32_t* offsets,
                                     const int32_t* token_map);
rudnn_moe_status dispatch_no_pairs(int32_t* offsets, int64_t E, hipStream_t stream);

// Per-thread one-shot timing hook (rudnn_moe_time_next_launch).
void timing_before(rudnn_moe_kernel k, hipStream_t s);
void timing_after(rudnn_moe_kernel k, hipStream_t s);

// ---- launchers (each returns hipGetLastError() after its launches) ----
hipError_t launch_route(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                        uint32_t* idx, void* w, hipStream_t s);

hipError_t launch_route_sigmoid_grouped(const void* logits, rudnn_moe_dtype ldt, const float* bias, int64_t T,
                                        int64_t E, int64_t k, int64_t groups, int64_t selected_groups, bool top_two,
                                        bool renorm, double scale, uint32_t* idx, void* w, hipStream_t s);

// Gate projection + routing (route_projected.hip).  The K split S (1: none) and the workspace
// it needs depend on T, H, E and the dtype only.
constexpr int64_t MAX_PROJECTED_EXPERTS = 256;
constexpr int64_t MAX_PROJECTED_HIDDEN = (int64_t)1 << 20;
int64_t projection_split(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dt);
size_t projection_workspace_bytes(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dt);
hipError_t launch_route_projected(const void* x, rudnn_moe_dtype dt, const void* router, int64_t T, int64_t H,
                                  int64_t E, int64_t k, bool renorm, void* logits_out, uint32_t* idx, void* w,
                                  void* workspace, hipStream_t s);

hipError_t launch_dispatch(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input, size_t row_bytes,
                           void* dispatched, int32_t* offsets, int32_t* token_map, int32_t* chunk_counts,
                           hipStream_t s);

// First-order training (train.hip).
hipError_t launch_selected_router(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, const void* idx,
                                  rudnn_moe_index_type it, int64_t k, bool sigmoid, bool renorm, double scale,
                                  const float* grad_weights, float* weights, void* grad_logits, hipStream_t s);
hipError_t launch_combine_backward(const void* y, rudnn_moe_dtype dt, const int32_t* map, const void* w,
                                   rudnn_moe_dtype wdt, const void* dout, int64_t T, int64_t k, int64_t H,
                                   int64_t rows, void* dexp, float* dw, hipStream_t s);
hipError_t launch_dispatch_backward(const void* d, rudnn_moe_dtype dt, const int32_t* map, int64_t T, int64_t k,
                                    int64_t H, int64_t rows, void* out, hipStream_t s);

// n int32 values set to v (a kernel, so that the call stays capturable in a HIP graph).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

hipError_t launch_combine(const void* y, rudnn_moe_dtype dt, const int32_t* token_map, const void* w,
                          rudnn_moe_dtype wdt, int64_t T, int64_t k, int64_t H, void* out, hipStream_t s);

// Expert GEMMs.  Workspace layout is owned by experts.hip.
size_t experts_workspace_bytes(int64_t E, int64_t H, int64_t I, rudnn_moe_dtype dt, int64_t rows);
// cache: NULL, or [rows, 2I] FP32 that receives the pre-activations [gate . x | up . x].
hipError_t launch_experts(const rudnn_moe_experts* ex, const void* dispatched, const int32_t* offsets, int64_t rows,
                          void* out, void* workspace, hipStream_t s, float* cache = nullptr);

// Experts backward (experts_backward.hip).  cached: the pre-activations come from the forward's
// cache (no room for them in the workspace); cache NULL recomputes them.
size_t experts_backward_workspace_bytes(int64_t E, int64_t I, rudnn_moe_dtype dt, int64_t rows, bool cached);
hipError_t launch_experts_backward(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets, int64_t rows,
                                   const float* cache, const void* dy, void* dx, float* dgate, float* dup,
                                   float* ddown, void* workspace, hipStream_t s);

}  // namespace rudnn
