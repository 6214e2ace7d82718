// api.cpp -- the C ABI of rudnn_moe.h: host-side validation, workspace layout, launches.
//
// Every check runs on the host before the first launch (the counterpart of the guide's
// Result<_, MoeError>, ruDNN user guide sections 3 and 6); pure argument checks come first and
// make no HIP call, so they can be exercised without a GPU.
#include <cmath>
#include <mutex>

#include "internal.hpp"

using namespace rudnn;

namespace {

thread_local hipEvent_t g_timing[RUDNN_MOE_KERNEL_COUNT][2] = {};

bool valid_dtype(rudnn_moe_dtype d) { return d == RUDNN_MOE_F32 || d == RUDNN_MOE_F16 || d == RUDNN_MOE_BF16; }

struct Range {
    const void* p;
    size_t n;
};

bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Each output against every input and every other output.
bool any_overlap(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range& i : ins)
            if (overlap(*o, i)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return true;
    }
    return false;
}

constexpr int64_t INT32_LIMIT = (int64_t)1 << 31;

rudnn_moe_status check_route_args(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                  rudnn_moe_routing_options opt, const uint32_t* idx, const void* w) {
    if (T < 0 || E < 1) return RUDNN_MOE_ERR_SHAPE;
    if (opt.top_k < 1 || opt.top_k > E) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(ldt)) return RUDNN_MOE_ERR_DTYPE;
    if (E > MAX_EXPERTS || opt.top_k > MAX_TOP_K || T * opt.top_k >= INT32_LIMIT || T * E >= ((int64_t)1 << 40))
        return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!logits || !idx || !w) return RUDNN_MOE_ERR_ARGUMENT;
    const size_t ls = dtype_size(ldt), pk = (size_t)(T * opt.top_k);
    if (any_overlap({{idx, pk * 4}, {w, pk * ls}}, {{logits, (size_t)(T * E) * ls}})) return RUDNN_MOE_ERR_ARGUMENT;
    return RUDNN_MOE_OK;
}

// Option checks of section 10 (the ranges the guide gives GroupRoutingOptions).
rudnn_moe_status check_group_options(int64_t E, const rudnn_moe_group_routing_options& o) {
    if (E > MAX_EXPERTS || o.groups < 1 || o.groups > 128 || E % o.groups != 0) return RUDNN_MOE_ERR_ARGUMENT;
    const int64_t per = E / o.groups;
    if (o.selected_groups < 1 || o.selected_groups > o.groups) return RUDNN_MOE_ERR_ARGUMENT;
    if (o.top_k < 1 || o.top_k > MAX_TOP_K || o.top_k > o.selected_groups * per) return RUDNN_MOE_ERR_ARGUMENT;
    if (o.group_top_two && per < 2) return RUDNN_MOE_ERR_ARGUMENT;
    if (!(o.scale > 0.0) || !std::isfinite(o.scale)) return RUDNN_MOE_ERR_ARGUMENT;
    return RUDNN_MOE_OK;
}

// Limits of the fused gate projection + routing kernel (route_projected.hip).
rudnn_moe_status check_projection(rudnn_moe_dtype dt, int64_t H, int64_t E, int64_t k, int64_t T) {
    if (E > MAX_PROJECTED_EXPERTS || k > MAX_TOP_K || H >= MAX_PROJECTED_HIDDEN) return RUDNN_MOE_ERR_UNSUPPORTED;
    if ((H * (int64_t)dtype_size(dt)) % 16 || T * k >= INT32_LIMIT || T * E >= ((int64_t)1 << 40))
        return RUDNN_MOE_ERR_UNSUPPORTED;
    return RUDNN_MOE_OK;
}

rudnn_moe_status check_experts_view(const rudnn_moe_experts* ex) {
    if (!ex) return RUDNN_MOE_ERR_ARGUMENT;
    if (ex->num_experts < 1 || ex->hidden < 1 || ex->intermediate < 1) return RUDNN_MOE_ERR_SHAPE;
    if (!valid_dtype(ex->dtype)) return RUDNN_MOE_ERR_DTYPE;
    if (!ex->gate || !ex->up || !ex->down) return RUDNN_MOE_ERR_ARGUMENT;
    if (ex->num_experts > MAX_EXPERTS) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (ex->dtype != RUDNN_MOE_F32) {
        // 16-byte vector loads of the contraction axis: H and I multiples of 8, aligned bases
        if (ex->hidden % 8 || ex->intermediate % 8) return RUDNN_MOE_ERR_UNSUPPORTED;
        if ((uintptr_t)ex->gate % 16 || (uintptr_t)ex->up % 16 || (uintptr_t)ex->down % 16)
            return RUDNN_MOE_ERR_UNSUPPORTED;
    }
    const int64_t wsz = ex->num_experts * ex->hidden * ex->intermediate;
    if (ex->hidden >= INT32_LIMIT || ex->intermediate >= INT32_LIMIT || wsz >= ((int64_t)1 << 40))
        return RUDNN_MOE_ERR_UNSUPPORTED;
    return RUDNN_MOE_OK;
}

rudnn_moe_status check_experts_rows(const rudnn_moe_experts* ex, int64_t rows) {
    if (rows < 0) return RUDNN_MOE_ERR_SHAPE;
    const int64_t wide = ex->hidden > ex->intermediate ? ex->hidden : ex->intermediate;
    if (rows >= INT32_LIMIT || rows * wide >= INT32_LIMIT * 64) return RUDNN_MOE_ERR_UNSUPPORTED;
    return RUDNN_MOE_OK;
}

}  // namespace

namespace rudnn {

rudnn_moe_status check_device(hipStream_t s, std::initializer_list<const void*> ptrs) {
    int dev = -1;
    if (s) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess) {
            (void)hipGetLastError();
            return RUDNN_MOE_ERR_DEVICE;
        }
    } else if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return RUDNN_MOE_ERR_DEVICE;
    }
    for (const void* p : ptrs) {
        hipPointerAttribute_t a;
        if (hipPointerGetAttributes(&a, p) != hipSuccess) {
            (void)hipGetLastError();
            return RUDNN_MOE_ERR_DEVICE;
        }
        if ((a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeManaged) || a.device != dev)
            return RUDNN_MOE_ERR_DEVICE;
    }
    return RUDNN_MOE_OK;
}

rudnn_moe_status runtime(hipError_t e) { return e == hipSuccess ? RUDNN_MOE_OK : RUDNN_MOE_ERR_RUNTIME; }

rudnn_moe_status check_dispatch_args(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input,
                                     rudnn_moe_dtype dt, int64_t H, const void* dispatched, const int32_t* offsets,
                                     const int32_t* token_map) {
    if (T < 0 || E < 1 || H < 1) return RUDNN_MOE_ERR_SHAPE;
    if (k < 1 || k > E) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(dt)) return RUDNN_MOE_ERR_DTYPE;
    if (E > MAX_EXPERTS || k > MAX_TOP_K || T * k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (!offsets) return RUDNN_MOE_ERR_ARGUMENT;
    if (T > 0 && (!idx || !input || !dispatched || !token_map)) return RUDNN_MOE_ERR_ARGUMENT;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k), rb = (size_t)H * es;
    if (any_overlap({{dispatched, pk * rb}, {offsets, 4 * (size_t)(E + 1)}, {token_map, pk * 4}},
                    {{idx, pk * 4}, {input, (size_t)T * rb}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    return RUDNN_MOE_OK;
}

// Softmax routing followed by dispatch: in one pass where the routing blocks can serve as the
// dispatch chunks (route_dispatch_chunk > 0), else the two one after the other.
hipError_t route_and_dispatch(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E, int64_t k, bool renorm,
                              uint32_t* idx, void* w, const void* input, size_t row_bytes, void* dispatched,
                              int32_t* offsets, int32_t* token_map, void* ws, hipStream_t stream) {
    const int64_t chunk = route_dispatch_chunk(T, E, k);
    hipError_t e;
    if (chunk > 0) {
        e = launch_route(logits, ldt, T, E, k, renorm, idx, w, stream, ws);
        if (e == hipSuccess)
            e = launch_dispatch_after_local(idx, T, k, E, chunk, input, row_bytes, dispatched, offsets, token_map, ws,
                                            stream);
    } else {
        e = launch_route(logits, ldt, T, E, k, renorm, idx, w, stream);
        if (e == hipSuccess)
            e = launch_dispatch(idx, T, k, E, input, row_bytes, dispatched, offsets, token_map, ws, stream);
    }
    return e;
}

rudnn_moe_status dispatch_no_pairs(int32_t* offsets, int64_t E, hipStream_t stream) {
    rudnn_moe_status st;
    if ((st = check_device(stream, {offsets})) != RUDNN_MOE_OK) return st;
    return runtime(launch_fill_i32(offsets, E + 1, 0, stream));
}

void timing_before(rudnn_moe_kernel k, hipStream_t s) {
    if (g_timing[k][0]) hipEventRecord(g_timing[k][0], s);
}

void timing_after(rudnn_moe_kernel k, hipStream_t s) {
    if (g_timing[k][1]) hipEventRecord(g_timing[k][1], s);
    g_timing[k][0] = g_timing[k][1] = nullptr;
}

}  // namespace rudnn

extern "C" {

const char* rudnn_moe_status_string(rudnn_moe_status s) {
    switch (s) {
    case RUDNN_MOE_OK: return "ok";
    case RUDNN_MOE_ERR_SHAPE: return "invalid shape";
    case RUDNN_MOE_ERR_DTYPE: return "invalid or mismatched dtype";
    case RUDNN_MOE_ERR_ARGUMENT: return "invalid argument (top_k, null pointer or overlapping buffers)";
    case RUDNN_MOE_ERR_DEVICE: return "pointer is not device memory of the stream's device";
    case RUDNN_MOE_ERR_UNSUPPORTED: return "outside the kernels' supported limits";
    case RUDNN_MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case RUDNN_MOE_ERR_RUNTIME: return "HIP runtime error";
    }
    return "unknown status";
}

rudnn_moe_status rudnn_moe_time_next_launch(rudnn_moe_kernel kernel, hipEvent_t before, hipEvent_t after) {
    if ((int)kernel < 0 || (int)kernel >= RUDNN_MOE_KERNEL_COUNT) return RUDNN_MOE_ERR_ARGUMENT;
    g_timing[kernel][0] = before;
    g_timing[kernel][1] = after;
    return RUDNN_MOE_OK;
}

rudnn_moe_status rudnn_moe_route(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                 rudnn_moe_routing_options opt, uint32_t* idx, void* w, hipStream_t stream) {
    rudnn_moe_status st = check_route_args(logits, ldt, T, E, opt, idx, w);
    if (st != RUDNN_MOE_OK || T == 0) return st;
    if ((st = check_device(stream, {logits, idx, w})) != RUDNN_MOE_OK) return st;
    return runtime(launch_route(logits, ldt, T, E, opt.top_k, opt.renormalize != 0, idx, w, stream));
}

rudnn_moe_status rudnn_moe_route_sigmoid_grouped(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                                 const float* bias, rudnn_moe_group_routing_options opt, uint32_t* idx,
                                                 void* w, hipStream_t stream) {
    if (T < 0 || E < 1) return RUDNN_MOE_ERR_SHAPE;
    rudnn_moe_status st = check_group_options(E, opt);
    if (st != RUDNN_MOE_OK) return st;
    if (!valid_dtype(ldt)) return RUDNN_MOE_ERR_DTYPE;
    if (T * opt.top_k >= INT32_LIMIT || T * E >= ((int64_t)1 << 40)) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!logits || !idx || !w) return RUDNN_MOE_ERR_ARGUMENT;
    const size_t ls = dtype_size(ldt), pk = (size_t)(T * opt.top_k);
    if (any_overlap({{idx, pk * 4}, {w, pk * ls}}, {{logits, (size_t)(T * E) * ls}, {bias, bias ? 4 * (size_t)E : 0}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {logits, idx, w})) != RUDNN_MOE_OK) return st;
    if (bias && (st = check_device(stream, {bias})) != RUDNN_MOE_OK) return st;
    return runtime(launch_route_sigmoid_grouped(logits, ldt, bias, T, E, opt.top_k, opt.groups, opt.selected_groups,
                                                opt.group_top_two != 0, opt.renormalize != 0, opt.scale, idx, w,
                                                stream));
}

size_t rudnn_moe_route_projected_workspace_size(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dt) {
    if (T < 0 || H < 1 || E < 1 || E > MAX_PROJECTED_EXPERTS || !valid_dtype(dt)) return 0;
    return projection_workspace_bytes(T, H, E, dt);
}

rudnn_moe_status rudnn_moe_route_projected(const void* input, rudnn_moe_dtype dt, const void* router, int64_t T,
                                           int64_t H, int64_t E, rudnn_moe_routing_options opt, void* logits_out,
                                           uint32_t* idx, void* w, void* workspace, size_t workspace_size,
                                           hipStream_t stream) {
    if (T < 0 || H < 1 || E < 1) return RUDNN_MOE_ERR_SHAPE;
    if (opt.top_k < 1 || opt.top_k > E) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(dt)) return RUDNN_MOE_ERR_DTYPE;
    rudnn_moe_status st = check_projection(dt, H, E, opt.top_k, T);
    if (st != RUDNN_MOE_OK || T == 0) return st;
    if (!input || !router || !idx || !w) return RUDNN_MOE_ERR_ARGUMENT;
    if ((uintptr_t)input % 16 || (uintptr_t)router % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    const size_t need = projection_workspace_bytes(T, H, E, dt);
    if (need && (!workspace || workspace_size < need)) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t es = dtype_size(dt), pk = (size_t)(T * opt.top_k);
    if (any_overlap({{idx, pk * 4}, {w, pk * es}, {logits_out, logits_out ? (size_t)(T * E) * es : 0},
                     {workspace, need}},
                    {{input, (size_t)(T * H) * es}, {router, (size_t)(E * H) * es}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {input, router, idx, w})) != RUDNN_MOE_OK) return st;
    if (logits_out && (st = check_device(stream, {logits_out})) != RUDNN_MOE_OK) return st;
    if (need && (st = check_device(stream, {workspace})) != RUDNN_MOE_OK) return st;
    return runtime(launch_route_projected(input, dt, router, T, H, E, opt.top_k, opt.renormalize != 0, logits_out,
                                          idx, w, workspace, stream));
}

static bool valid_index_type(rudnn_moe_index_type t) {
    return t == RUDNN_MOE_U32 || t == RUDNN_MOE_I32 || t == RUDNN_MOE_I64;
}

static rudnn_moe_status selected_router_common(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                               const void* idx, rudnn_moe_index_type it, int64_t k,
                                               const rudnn_moe_router_weight_options& o, const float* gw,
                                               float* w, void* gl, hipStream_t stream) {
    if (T < 0 || E < 1) return RUDNN_MOE_ERR_SHAPE;
    if (k < 1 || k > E || k > MAX_TOP_K) return RUDNN_MOE_ERR_ARGUMENT;
    if ((o.scoring != 0 && o.scoring != 1) || !(o.scale > 0.0) || !std::isfinite(o.scale))
        return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(ldt) || !valid_index_type(it)) return RUDNN_MOE_ERR_DTYPE;
    if (E >= INT32_LIMIT || T * E >= ((int64_t)1 << 40) || T * k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!logits || !idx || (gw ? !gl : !w)) return RUDNN_MOE_ERR_ARGUMENT;
    const size_t ls = dtype_size(ldt), is = it == RUDNN_MOE_I64 ? 8 : 4, pk = (size_t)(T * k);
    const Range out = gw ? Range{gl, (size_t)(T * E) * ls} : Range{w, pk * 4};
    if (any_overlap({out}, {{logits, (size_t)(T * E) * ls}, {idx, pk * is}, {gw, gw ? pk * 4 : 0}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    rudnn_moe_status st;
    if ((st = check_device(stream, {logits, idx, gw ? (const void*)gl : (const void*)w})) != RUDNN_MOE_OK) return st;
    if (gw && (st = check_device(stream, {gw})) != RUDNN_MOE_OK) return st;
    return runtime(launch_selected_router(logits, ldt, T, E, idx, it, k, o.scoring == 1, o.renormalize != 0, o.scale,
                                          gw, w, gl, stream));
}

rudnn_moe_status rudnn_moe_selected_router_weights(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                                   const void* indices, rudnn_moe_index_type it, int64_t top_k,
                                                   rudnn_moe_router_weight_options opt, float* weights,
                                                   hipStream_t stream) {
    return selected_router_common(logits, ldt, T, E, indices, it, top_k, opt, nullptr, weights, nullptr, stream);
}

rudnn_moe_status rudnn_moe_selected_router_backward(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                                    const void* indices, rudnn_moe_index_type it, int64_t top_k,
                                                    rudnn_moe_router_weight_options opt, const float* grad_weights,
                                                    void* grad_logits, hipStream_t stream) {
    if (!grad_weights && T > 0) return RUDNN_MOE_ERR_ARGUMENT;
    return selected_router_common(logits, ldt, T, E, indices, it, top_k, opt, grad_weights ? grad_weights : nullptr,
                                  nullptr, grad_logits, stream);
}

// Rows of 16-byte vectors (the combine/dispatch backward kernels).
static rudnn_moe_status check_vector_rows(rudnn_moe_dtype dt, int64_t H, std::initializer_list<const void*> ptrs) {
    if ((H * (int64_t)dtype_size(dt)) % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    for (const void* p : ptrs)
        if ((uintptr_t)p % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    return RUDNN_MOE_OK;
}

rudnn_moe_status rudnn_moe_combine_backward(const void* y, rudnn_moe_dtype dt, const int32_t* token_map,
                                            const void* w, rudnn_moe_dtype wdt, const void* dout, int64_t T, int64_t k,
                                            int64_t H, void* dexp, float* dw, hipStream_t stream) {
    if (T < 0 || H < 1) return RUDNN_MOE_ERR_SHAPE;
    if (k < 1) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(dt) || !valid_dtype(wdt)) return RUDNN_MOE_ERR_DTYPE;
    if (k > MAX_TOP_K || T * k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!y || !token_map || !w || !dout || !dexp || !dw) return RUDNN_MOE_ERR_ARGUMENT;
    rudnn_moe_status st;
    if ((st = check_vector_rows(dt, H, {y, dout, dexp})) != RUDNN_MOE_OK) return st;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k);
    if (any_overlap({{dexp, pk * H * es}, {dw, pk * 4}},
                    {{y, pk * H * es}, {token_map, pk * 4}, {w, pk * dtype_size(wdt)}, {dout, (size_t)T * H * es}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {y, token_map, w, dout, dexp, dw})) != RUDNN_MOE_OK) return st;
    return runtime(launch_combine_backward(y, dt, token_map, w, wdt, dout, T, k, H, T * k, dexp, dw, stream));
}

rudnn_moe_status rudnn_moe_dispatch_backward(const void* d, rudnn_moe_dtype dt, const int32_t* token_map, int64_t T,
                                             int64_t k, int64_t H, void* out, hipStream_t stream) {
    if (T < 0 || H < 1) return RUDNN_MOE_ERR_SHAPE;
    if (k < 1) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(dt)) return RUDNN_MOE_ERR_DTYPE;
    if (k > MAX_TOP_K || T * k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!d || !token_map || !out) return RUDNN_MOE_ERR_ARGUMENT;
    rudnn_moe_status st;
    if ((st = check_vector_rows(dt, H, {d, out})) != RUDNN_MOE_OK) return st;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k);
    if (any_overlap({{out, (size_t)T * H * es}}, {{d, pk * H * es}, {token_map, pk * 4}})) return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {d, token_map, out})) != RUDNN_MOE_OK) return st;
    return runtime(launch_dispatch_backward(d, dt, token_map, T, k, H, T * k, out, stream));
}

size_t rudnn_moe_dispatch_workspace_size(int64_t T, int64_t top_k, int64_t E) {
    if (T < 0 || top_k < 1 || E < 1) return 0;
    return dispatch_workspace_bytes(T, top_k, E);
}

rudnn_moe_status rudnn_moe_dispatch(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input,
                                    rudnn_moe_dtype dt, int64_t H, void* dispatched, int32_t* offsets,
                                    int32_t* token_map, void* workspace, size_t workspace_size, hipStream_t stream) {
    rudnn_moe_status st = check_dispatch_args(idx, T, k, E, input, dt, H, dispatched, offsets, token_map);
    if (st != RUDNN_MOE_OK) return st;
    const size_t need = rudnn_moe_dispatch_workspace_size(T, k, E);
    if (T > 0 && (!workspace || workspace_size < need)) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k), rb = (size_t)H * es;
    if (any_overlap({{workspace, need}}, {{dispatched, pk * rb}, {offsets, 4 * (size_t)(E + 1)}, {token_map, pk * 4},
                                          {idx, pk * 4}, {input, (size_t)T * rb}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if (T == 0) return dispatch_no_pairs(offsets, E, stream);
    if ((st = check_device(stream, {idx, input, dispatched, offsets, token_map, workspace})) != RUDNN_MOE_OK) return st;
    return runtime(launch_dispatch(idx, T, k, E, input, rb, dispatched, offsets, token_map, workspace, stream));
}

rudnn_moe_status rudnn_moe_route_dispatch(const void* logits, rudnn_moe_dtype ldt, int64_t T, int64_t E,
                                          rudnn_moe_routing_options opt, const void* input, rudnn_moe_dtype dt,
                                          int64_t H, uint32_t* idx, void* w, void* dispatched, int32_t* offsets,
                                          int32_t* token_map, void* workspace, size_t workspace_size,
                                          hipStream_t stream) {
    rudnn_moe_status st = check_route_args(logits, ldt, T, E, opt, idx, w);
    if (st != RUDNN_MOE_OK) return st;
    const int64_t k = opt.top_k;
    if ((st = check_dispatch_args(idx, T, k, E, input, dt, H, dispatched, offsets, token_map)) != RUDNN_MOE_OK)
        return st;
    const size_t need = rudnn_moe_dispatch_workspace_size(T, k, E);
    if (T > 0 && (!workspace || workspace_size < need)) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k), rb = (size_t)H * es, ls = dtype_size(ldt);
    // outputs (indices, weights, rows, offsets, map, workspace) against each other and the inputs
    if (any_overlap({{idx, pk * 4}, {w, pk * ls}, {dispatched, pk * rb}, {offsets, 4 * (size_t)(E + 1)},
                     {token_map, pk * 4}, {workspace, need}},
                    {{logits, (size_t)(T * E) * ls}, {input, (size_t)T * rb}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if (T == 0) return dispatch_no_pairs(offsets, E, stream);
    if ((st = check_device(stream, {logits, input, idx, w, dispatched, offsets, token_map, workspace})) !=
        RUDNN_MOE_OK)
        return st;
    return runtime(route_and_dispatch(logits, ldt, T, E, k, opt.renormalize != 0, idx, w, input, rb, dispatched,
                                      offsets, token_map, workspace, stream));
}

size_t rudnn_moe_experts_workspace_size(const rudnn_moe_experts* ex, int64_t rows) {
    if (!ex || rows < 0 || ex->num_experts < 1 || ex->intermediate < 1 || !valid_dtype(ex->dtype)) return 0;
    return experts_workspace_bytes(ex->num_experts, ex->hidden, ex->intermediate, ex->dtype, rows);
}

namespace {
// experts_forward and its training variant (cache != NULL: [rows, 2I] FP32 pre-activations).
rudnn_moe_status experts_forward_common(const rudnn_moe_experts* ex, const void* dispatched, const int32_t* offsets,
                                        int64_t rows, void* out, float* cache, bool training, void* workspace,
                                        size_t workspace_size, hipStream_t stream) {
    rudnn_moe_status st = check_experts_view(ex);
    if (st != RUDNN_MOE_OK) return st;
    if ((st = check_experts_rows(ex, rows)) != RUDNN_MOE_OK) return st;
    if (rows == 0) return RUDNN_MOE_OK;
    if (!dispatched || !offsets || !out || (training && !cache)) return RUDNN_MOE_ERR_ARGUMENT;
    if (ex->dtype != RUDNN_MOE_F32 && ((uintptr_t)dispatched % 16 || (uintptr_t)out % 16))
        return RUDNN_MOE_ERR_UNSUPPORTED;
    if (training && (uintptr_t)cache % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    const size_t need = rudnn_moe_experts_workspace_size(ex, rows);
    if (!workspace || workspace_size < need) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t es = dtype_size(ex->dtype);
    const size_t wsz = (size_t)(ex->num_experts * ex->hidden * ex->intermediate) * es;
    const size_t xb = (size_t)rows * ex->hidden * es;
    const size_t cb = training ? (size_t)rows * 2 * ex->intermediate * 4 : 0;
    if (any_overlap({{out, xb}, {workspace, need}, {cache, cb}},
                    {{dispatched, xb}, {offsets, 4 * (size_t)(ex->num_experts + 1)}, {ex->gate, wsz}, {ex->up, wsz},
                     {ex->down, wsz}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {dispatched, offsets, out, workspace, ex->gate, ex->up, ex->down})) != RUDNN_MOE_OK)
        return st;
    if (training && (st = check_device(stream, {cache})) != RUDNN_MOE_OK) return st;
    return runtime(launch_experts(ex, dispatched, offsets, rows, out, workspace, stream, training ? cache : nullptr));
}
}  // namespace

rudnn_moe_status rudnn_moe_experts_forward(const rudnn_moe_experts* ex, const void* dispatched, const int32_t* offsets,
                                           int64_t rows, void* out, void* workspace, size_t workspace_size,
                                           hipStream_t stream) {
    return experts_forward_common(ex, dispatched, offsets, rows, out, nullptr, false, workspace, workspace_size,
                                  stream);
}

rudnn_moe_status rudnn_moe_experts_forward_training(const rudnn_moe_experts* ex, const void* dispatched,
                                                    const int32_t* offsets, int64_t rows, void* out, float* cache,
                                                    void* workspace, size_t workspace_size, hipStream_t stream) {
    return experts_forward_common(ex, dispatched, offsets, rows, out, cache, true, workspace, workspace_size, stream);
}

size_t rudnn_moe_experts_backward_workspace_size(const rudnn_moe_experts* ex, int64_t rows, int cached) {
    if (!ex || rows < 0 || ex->num_experts < 1 || ex->intermediate < 1 || !valid_dtype(ex->dtype)) return 0;
    return experts_backward_workspace_bytes(ex->num_experts, ex->intermediate, ex->dtype, rows, cached != 0);
}

rudnn_moe_status rudnn_moe_experts_backward(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets,
                                            int64_t rows, const float* cache, const void* dy, void* dx, float* dgate,
                                            float* dup, float* ddown, void* workspace, size_t workspace_size,
                                            hipStream_t stream) {
    rudnn_moe_status st = check_experts_view(ex);
    if (st != RUDNN_MOE_OK) return st;
    if ((st = check_experts_rows(ex, rows)) != RUDNN_MOE_OK) return st;
    const int64_t E = ex->num_experts, H = ex->hidden, I = ex->intermediate;
    const size_t es = dtype_size(ex->dtype);
    if ((H * (int64_t)es) % 16 || (I * (int64_t)es) % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (!offsets || !dgate || !dup || !ddown) return RUDNN_MOE_ERR_ARGUMENT;
    if (rows > 0 && (!x || !dy || !dx)) return RUDNN_MOE_ERR_ARGUMENT;
    for (const void* p : {(const void*)x, dy, (const void*)dx, (const void*)dgate, (const void*)dup,
                          (const void*)ddown, (const void*)cache, ex->gate, ex->up, ex->down})
        if ((uintptr_t)p % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    const size_t need = rudnn_moe_experts_backward_workspace_size(ex, rows, cache != nullptr);
    if (!workspace || workspace_size < need) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t wsz = (size_t)(E * H * I) * es, gsz = (size_t)(E * H * I) * 4, xb = (size_t)rows * H * es;
    const size_t cb = cache ? (size_t)rows * 2 * I * 4 : 0;
    if (any_overlap({{dx, xb}, {dgate, gsz}, {dup, gsz}, {ddown, gsz}, {workspace, need}},
                    {{x, xb}, {dy, xb}, {offsets, 4 * (size_t)(E + 1)}, {cache, cb}, {ex->gate, wsz},
                     {ex->up, wsz}, {ex->down, wsz}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {offsets, dgate, dup, ddown, workspace, ex->gate, ex->up, ex->down})) !=
        RUDNN_MOE_OK)
        return st;
    if (rows > 0 && (st = check_device(stream, {x, dy, dx})) != RUDNN_MOE_OK) return st;
    if (rows > 0 && cache && (st = check_device(stream, {cache})) != RUDNN_MOE_OK) return st;
    return runtime(
        launch_experts_backward(ex, x, offsets, rows, cache, dy, dx, dgate, dup, ddown, workspace, stream));
}

rudnn_moe_status rudnn_moe_combine(const void* y, rudnn_moe_dtype dt, const int32_t* token_map, const void* w,
                                   rudnn_moe_dtype wdt, int64_t T, int64_t k, int64_t H, void* out,
                                   hipStream_t stream) {
    if (T < 0 || H < 1) return RUDNN_MOE_ERR_SHAPE;
    if (k < 1) return RUDNN_MOE_ERR_ARGUMENT;
    if (!valid_dtype(dt) || !valid_dtype(wdt)) return RUDNN_MOE_ERR_DTYPE;
    if (k > MAX_TOP_K || T * k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return RUDNN_MOE_OK;
    if (!y || !token_map || !w || !out) return RUDNN_MOE_ERR_ARGUMENT;
    const size_t es = dtype_size(dt), pk = (size_t)(T * k);
    if (any_overlap({{out, (size_t)T * H * es}},
                    {{y, pk * H * es}, {token_map, pk * 4}, {w, pk * dtype_size(wdt)}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    rudnn_moe_status st;
    if ((st = check_device(stream, {y, token_map, w, out})) != RUDNN_MOE_OK) return st;
    return runtime(launch_combine(y, dt, token_map, w, wdt, T, k, H, out, stream));
}

namespace {
struct ForwardLayout {
    size_t idx, w, offsets, map, dws, disp, ews, y, proj, total;
};

// projected: the forward from the hidden states, which adds the projection's partial logits.
ForwardLayout forward_layout(const rudnn_moe_experts* ex, int64_t T, int64_t k, rudnn_moe_dtype ldt,
                             bool projected = false) {
    ForwardLayout L;
    const size_t es = dtype_size(ex->dtype), pk = (size_t)(T * k);
    size_t off = 0;
    auto take = [&](size_t n) {
        size_t at = off;
        off += align_up(n);
        return at;
    };
    L.idx = take(pk * 4);
    L.w = take(pk * dtype_size(ldt));
    L.offsets = take(4 * (size_t)(ex->num_experts + 1));
    L.map = take(pk * 4);
    L.dws = take(rudnn_moe_dispatch_workspace_size(T, k, ex->num_experts));
    L.disp = take(pk * ex->hidden * es);
    L.ews = take(experts_workspace_bytes(ex->num_experts, ex->hidden, ex->intermediate, ex->dtype, (int64_t)pk));
    L.y = take(pk * ex->hidden * es);
    L.proj = take(projected ? projection_workspace_bytes(T, ex->hidden, ex->num_experts, ex->dtype) : 0);
    L.total = off;
    return L;
}
}  // namespace

size_t rudnn_moe_forward_workspace_size(const rudnn_moe_experts* ex, int64_t T, int64_t top_k,
                                        rudnn_moe_dtype logits_dtype) {
    if (!ex || T < 0 || top_k < 1 || ex->num_experts < 1 || ex->hidden < 1 || ex->intermediate < 1 ||
        !valid_dtype(ex->dtype) || !valid_dtype(logits_dtype))
        return 0;
    return forward_layout(ex, T, top_k, logits_dtype).total;
}

size_t rudnn_moe_forward_projected_workspace_size(const rudnn_moe_experts* ex, int64_t T, int64_t top_k) {
    if (!ex || T < 0 || top_k < 1 || ex->num_experts < 1 || ex->hidden < 1 || ex->intermediate < 1 ||
        ex->num_experts > MAX_PROJECTED_EXPERTS || !valid_dtype(ex->dtype))
        return 0;
    return forward_layout(ex, T, top_k, ex->dtype, true).total;
}

}  // extern "C"

namespace {

// The forward of sections 6 and 10: routing (softmax or group-limited sigmoid, chosen by
// `sig`; or, with a router, softmax routing of the fused gate projection) -> dispatch ->
// experts -> combine, after the shared checks.
rudnn_moe_status forward_common(const rudnn_moe_experts* ex, const void* input, const void* logits,
                                rudnn_moe_dtype ldt, int64_t T, int64_t top_k, int renormalize,
                                const rudnn_moe_group_routing_options* sig, const float* bias, const void* router,
                                void* output, void* workspace, size_t workspace_size, hipStream_t stream) {
    rudnn_moe_status st = check_experts_view(ex);
    if (st != RUDNN_MOE_OK) return st;
    if (T < 0) return RUDNN_MOE_ERR_SHAPE;
    if (sig) {
        if ((st = check_group_options(ex->num_experts, *sig)) != RUDNN_MOE_OK) return st;
    } else if (top_k < 1 || top_k > ex->num_experts) {
        return RUDNN_MOE_ERR_ARGUMENT;
    }
    if (!valid_dtype(ldt)) return RUDNN_MOE_ERR_DTYPE;
    if (top_k > MAX_TOP_K || T * top_k >= INT32_LIMIT) return RUDNN_MOE_ERR_UNSUPPORTED;
    if ((st = check_experts_rows(ex, T * top_k)) != RUDNN_MOE_OK) return st;
    if (router && (st = check_projection(ldt, ex->hidden, ex->num_experts, top_k, T)) != RUDNN_MOE_OK) return st;
    if (T == 0) return RUDNN_MOE_OK;
    if (!input || !(router ? router : logits) || !output) return RUDNN_MOE_ERR_ARGUMENT;
    if ((ex->dtype != RUDNN_MOE_F32 || router) && ((uintptr_t)input % 16 || (uintptr_t)output % 16))
        return RUDNN_MOE_ERR_UNSUPPORTED;
    if (router && (uintptr_t)router % 16) return RUDNN_MOE_ERR_UNSUPPORTED;
    const ForwardLayout L = forward_layout(ex, T, top_k, ldt, router != nullptr);
    if (!workspace || workspace_size < L.total) return RUDNN_MOE_ERR_WORKSPACE;
    const size_t es = dtype_size(ex->dtype);
    const size_t wsz = (size_t)(ex->num_experts * ex->hidden * ex->intermediate) * es;
    const size_t xb = (size_t)T * ex->hidden * es;
    const size_t lb = logits ? (size_t)(T * ex->num_experts) * dtype_size(ldt) : 0;
    const size_t rb = router ? (size_t)(ex->num_experts * ex->hidden) * es : 0;
    if (any_overlap({{output, xb}, {workspace, L.total}},
                    {{input, xb}, {logits, lb}, {router, rb}, {ex->gate, wsz}, {ex->up, wsz}, {ex->down, wsz},
                     {bias, bias ? 4 * (size_t)ex->num_experts : 0}}))
        return RUDNN_MOE_ERR_ARGUMENT;
    if ((st = check_device(stream, {input, router ? router : logits, output, workspace, ex->gate, ex->up,
                                    ex->down})) != RUDNN_MOE_OK)
        return st;
    if (bias && (st = check_device(stream, {bias})) != RUDNN_MOE_OK) return st;
    unsigned char* ws = (unsigned char*)workspace;
    uint32_t* idx = (uint32_t*)(ws + L.idx);
    void* w = ws + L.w;
    int32_t* offsets = (int32_t*)(ws + L.offsets);
    int32_t* map = (int32_t*)(ws + L.map);
    void* disp = ws + L.disp;
    void* y = ws + L.y;
    const int64_t E = ex->num_experts, k = top_k, H = ex->hidden;
    hipError_t e;
    if (router)
        e = launch_route_projected(input, ldt, router, T, H, E, k, renormalize != 0, nullptr, idx, w, ws + L.proj,
                                   stream);
    else if (sig)
        e = launch_route_sigmoid_grouped(logits, ldt, bias, T, E, k, sig->groups, sig->selected_groups,
                                         sig->group_top_two != 0, sig->renormalize != 0, sig->scale, idx, w, stream);
    else
        e = route_and_dispatch(logits, ldt, T, E, k, renormalize != 0, idx, w, input, (size_t)H * es, disp, offsets,
                               map, ws + L.dws, stream);
    if (e == hipSuccess && (router || sig))
        e = launch_dispatch(idx, T, k, E, input, (size_t)H * es, disp, offsets, map, ws + L.dws, stream);
    if (e == hipSuccess) e = launch_experts(ex, disp, offsets, T * k, y, ws + L.ews, stream);
    if (e == hipSuccess) e = launch_combine(y, ex->dtype, map, w, ldt, T, k, H, output, stream);
    return runtime(e);
}

}  // namespace

extern "C" {

rudnn_moe_status rudnn_moe_forward(const rudnn_moe_experts* ex, const void* input, const void* logits,
                                   rudnn_moe_dtype ldt, int64_t T, rudnn_moe_routing_options opt, void* output,
                                   void* workspace, size_t workspace_size, hipStream_t stream) {
    return forward_common(ex, input, logits, ldt, T, opt.top_k, opt.renormalize, nullptr, nullptr, nullptr, output,
                          workspace, workspace_size, stream);
}

rudnn_moe_status rudnn_moe_forward_sigmoid_grouped(const rudnn_moe_experts* ex, const void* input,
                                                   const void* logits, rudnn_moe_dtype ldt, int64_t T,
                                                   const float* bias, rudnn_moe_group_routing_options opt,
                                                   void* output, void* workspace, size_t workspace_size,
                                                   hipStream_t stream) {
    return forward_common(ex, input, logits, ldt, T, opt.top_k, opt.renormalize, &opt, bias, nullptr, output,
                          workspace, workspace_size, stream);
}

rudnn_moe_status rudnn_moe_forward_projected(const rudnn_moe_experts* ex, const void* input, const void* router,
                                             int64_t T, rudnn_moe_routing_options opt, void* output, void* workspace,
                                             size_t workspace_size, hipStream_t stream) {
    if (!ex) return RUDNN_MOE_ERR_ARGUMENT;
    return forward_common(ex, input, nullptr, ex->dtype, T, opt.top_k, opt.renormalize, nullptr, nullptr, router,
                          output, workspace, workspace_size, stream);
}

}  // extern "C"
