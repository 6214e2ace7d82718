// internal.hpp -- host-side contract between the C-ABI layer (api.cpp) and the kernel files.
// Launchers only enqueue; argument validation happens in api.cpp before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/rudnn_moe.h"

namespace rudnn {

// Dispatch works on chunks of consecutive (token, slot) pairs; its per-chunk step (counts and
// local ranks) runs on one block per chunk.  A dispatch of its own uses chunks of dispatch_chunk
// pairs: 256..4096 (a multiple of the 256-thread block), about pairs / 512, enough blocks for the
// per-chunk kernel.  Routing and dispatch in one pass use one routing block's pairs as the chunk
// (route_dispatch_chunk).
#ifndef RUDNN_DISPATCH_CHUNKS
#define RUDNN_DISPATCH_CHUNKS 512
#endif
inline int64_t dispatch_chunk(int64_t pairs) {
    int64_t c = 256;
    while (c < 4096 && c * RUDNN_DISPATCH_CHUNKS < pairs) c *= 2;
    return c;
}

// Kernel limits (documented in rudnn_moe.h as RUDNN_MOE_ERR_UNSUPPORTED).
constexpr int64_t MAX_EXPERTS = 1024;
constexpr int64_t MAX_TOP_K = 64;

// Routing: lanes per row, the smallest power of two G with 16 G >= E (16 logits per lane).
inline int route_lanes(int64_t E) {
    int g = 1;
    while ((int64_t)g * 16 < E) g *= 2;
    return g;
}
// Threads per routing block with the dispatch epilogue: 1024 while that still leaves at least 256
// blocks, else 256.
inline int route_dispatch_threads(int64_t T, int64_t E) {
    return T >= (int64_t)256 * (1024 / route_lanes(E)) ? 1024 : 256;
}
// Pairs per chunk when routing and dispatch run in one pass (one routing block's rows), or 0 where
// that form is not used (chunks of fewer than 128 pairs would make the count table too long).
inline int64_t route_dispatch_chunk(int64_t T, int64_t E, int64_t k) {
    const int64_t c = (int64_t)(route_dispatch_threads(T, E) / route_lanes(E)) * k;
    return c >= 128 ? c : 0;
}

inline size_t align_up(size_t n, size_t a = 256) { return (n + a - 1) / a * a; }
// Dispatch workspace: [E, chunks] int32 per-chunk counts (the scan turns them into per-chunk bases
// in place), room for the larger chunk count of the two chunkings, then [E] int32 expert totals,
// then [T * k] int32 local ranks.
inline int64_t dispatch_max_chunks(int64_t T, int64_t k, int64_t E) {
    const int64_t pairs = T * k, c = dispatch_chunk(pairs), rc = route_dispatch_chunk(T, E, k);
    const int64_t n = (pairs + c - 1) / c, nr = rc > 0 ? (pairs + rc - 1) / rc : 0;
    return n > nr ? n : nr;
}
inline size_t dispatch_totals_offset(int64_t T, int64_t k, int64_t E) {
    return align_up(sizeof(int32_t) * (size_t)(dispatch_max_chunks(T, k, E) * E));
}
inline size_t dispatch_ranks_offset(int64_t T, int64_t k, int64_t E) {
    return dispatch_totals_offset(T, k, E) + align_up(sizeof(int32_t) * (size_t)E);
}
inline size_t dispatch_workspace_bytes(int64_t T, int64_t k, int64_t E) {
    return dispatch_ranks_offset(T, k, E) + align_up(sizeof(int32_t) * (size_t)(T * k));
}
int dispatch_id_bits(int64_t E);  // ceil(log2 E): the id bits the per-chunk ranking compares
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
hipError_t route_and_dispatch(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                              uint32_t* idx, void* w, const void* input, size_t row_bytes, void* dispatched,
                              int32_t* offsets, int32_t* token_map, void* ws, hipStream_t stream);

// Per-thread one-shot timing hook (rudnn_moe_time_next_launch).
void timing_before(rudnn_moe_kernel k, hipStream_t s);
void timing_after(rudnn_moe_kernel k, hipStream_t s);

// ---- launchers (each returns hipGetLastError() after its launches) ----
// dispatch_ws non-null: routing with the dispatch epilogue (chunks of route_dispatch_chunk pairs,
// whose counts and local ranks go to that dispatch workspace); route_dispatch_chunk must be > 0.
hipError_t launch_route(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                        uint32_t* idx, void* w, hipStream_t s, void* dispatch_ws = nullptr);

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

// ws: a dispatch workspace (dispatch_workspace_bytes).  launch_dispatch runs all three steps;
// launch_dispatch_after_local the scan and copy, after a per-chunk step with chunks of `chunk`
// pairs (the routing kernel's epilogue) has filled the workspace.
hipError_t launch_dispatch(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input, size_t row_bytes,
                           void* dispatched, int32_t* offsets, int32_t* token_map, void* ws, hipStream_t s);
hipError_t launch_dispatch_after_local(const uint32_t* idx, int64_t T, int64_t k, int64_t E, int64_t chunk,
                                       const void* input, size_t row_bytes, void* dispatched, int32_t* offsets,
                                       int32_t* token_map, void* ws, hipStream_t s);

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
