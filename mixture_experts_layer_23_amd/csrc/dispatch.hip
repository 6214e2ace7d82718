// dispatch.hip -- capacity-free grouping of tokens by expert (ruDNN user guide, section 5
// "Expert weights and dispatch").
//
// The T*k (token, slot) pairs, flattened as a = t*k + j, are cut into chunks of consecutive
// pairs.  Three steps:
//   local  per chunk: the per-expert counts of its pairs, stored as chunk_counts[c, e] (every
//          entry written, nothing needs clearing; expert-major, so the scan reads contiguous
//          rows), and each pair's stable rank among the chunk's
//          pairs of the same expert (the lanes of a wavefront holding the same id are found with
//          one ballot per id bit, LDS counters carry across wavefronts and rounds).  Either a
//          kernel of its own (one block per chunk of dispatch_chunk pairs), or the epilogue of
//          the routing kernel when routing and dispatch run together (one chunk per routing
//          block, whose winners are already in LDS);
//   scan   one block per expert: the exclusive sum of its counts over the chunks (a block scan,
//          in place, turning counts into per-chunk bases) and the expert's total;
//   copy   one wavefront per token: the exclusive sum of the expert totals (once per block, in
//          LDS; block 0 stores expert_offsets), token_map[a] = offsets[e] + base[c, e] + rank,
//          and the row read from HBM once in 16-byte vectors and written to its k dispatched rows.
// Rows of an expert follow (t, j) order, and the result does not depend on scheduling (no global
// atomics).  HBM traffic: T*k*4 (ids) + T*H*s (tokens, once) + T*k*H*s (rows) + T*k*4 (map) plus
// the chunk ranks and counts (T*k*4 written and read; L2-resident at these sizes).
#include <mutex>

#include "device.hpp"
#include "dispatch_local.hpp"
#include "internal.hpp"

namespace rudnn {

__global__ __launch_bounds__(256) void dispatch_local_kernel(const uint32_t* __restrict__ idx, int64_t pairs, int E,
                                                             int id_bits, int chunk, int32_t* __restrict__ chunk_counts,
                                                             int32_t* __restrict__ ranks) {
    extern __shared__ int sm[];  // run [E], wcnt [4][E]
    const int64_t a0 = (int64_t)blockIdx.x * chunk;
    const int n = (int)min((int64_t)chunk, pairs - a0);
    const uint32_t* ids = idx + a0;
    chunk_ranks<4>([&](int p) { return ids[p]; }, n, E, id_bits, sm, sm + E,
                   [&](int e, int c) { chunk_counts[(int64_t)e * gridDim.x + blockIdx.x] = c; }, ranks + a0);
}

// Block e: the exclusive prefix of expert e's counts over the chunks (row e of the [E, chunks]
// table, contiguous), 4 chunks per thread and 1024 per pass, in place, and the expert's total.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks,
                                                            int32_t* __restrict__ totals) {
    __shared__ int scratch[17];
    int32_t* row = chunk_counts + (int64_t)blockIdx.x * nchunks;
    int running = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 4 * (int)blockDim.x) {
        const int c = c0 + 4 * (int)threadIdx.x;
        int v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = c + q < nchunks ? row[c + q] : 0;
        int pass_total;
        int acc = running + block_exclusive_scan(v[0] + v[1] + v[2] + v[3], scratch, &pass_total);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (c + q < nchunks) row[c + q] = acc;
            acc += v[q];
        }
        running += pass_total;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = running;
}

// One wavefront per token (4 per block); V is the copy unit (a 16-byte vector when the row allows
// it).  The row's loads go out before the map arithmetic, which only the stores wait for.
#ifndef RUDNN_COPY_UNROLL
#define RUDNN_COPY_UNROLL 4
#endif
template <typename V>
__global__ __launch_bounds__(256) void dispatch_copy_kernel(const V* __restrict__ x, int64_t T, int k, int E,
                                                            int64_t row_units, const uint32_t* __restrict__ idx,
                                                            int chunk, int nchunks, const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ totals,
                                                            const int32_t* __restrict__ ranks,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ token_map, V* __restrict__ out) {
    constexpr int U = RUDNN_COPY_UNROLL;  // copy units per lane and pass
    extern __shared__ int s_off[];       // [E] expert offsets
    __shared__ int scratch[17];
    for (int e0 = 0, carry = 0; e0 < E; e0 += blockDim.x) {  // E <= 1024: at most 4 passes
        const int e = e0 + (int)threadIdx.x;
        int pass_total;
        const int excl = block_exclusive_scan(e < E ? totals[e] : 0, scratch, &pass_total);
        if (e < E) s_off[e] = carry + excl;
        if (blockIdx.x == 0 && e < E) offsets[e] = carry + excl;
        carry += pass_total;
        if (blockIdx.x == 0 && threadIdx.x == 0 && e0 + (int)blockDim.x >= E) offsets[E] = carry;
    }
    __syncthreads();
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const V* src = x + t * row_units;
    int my_row = -1;  // lane j < k: the dispatched row of copy j, computed during the first pass
    for (int64_t i0 = 0; i0 < row_units; i0 += 64 * U) {
        V v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * 64 + lane < row_units) v[u] = src[i0 + u * 64 + lane];
        if (i0 == 0 && lane < k) {
            const int64_t a = t * k + lane;
            const uint32_t e = idx[a];
            if (e < (uint32_t)E) my_row = s_off[e] + base[(int64_t)e * nchunks + a / chunk] + ranks[a];
            token_map[a] = my_row;
        }
        for (int j = 0; j < k; ++j) {
            const int dst = readlane(my_row, j);
            if (dst < 0) continue;
            V* d = out + (int64_t)dst * row_units;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (i0 + u * 64 + lane < row_units) d[i0 + u * 64 + lane] = v[u];
        }
    }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
    if (n > 0) fill_i32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n, v);
    return hipGetLastError();
}

int dispatch_id_bits(int64_t E) {
    int b = 0;
    while (((int64_t)1 << b) < E) ++b;
    return b;
}

// The scan and copy steps, once the chunks' counts and local ranks (chunks of `chunk` pairs) are in
// the workspace `ws` (see dispatch_workspace_bytes).
hipError_t launch_dispatch_after_local(const uint32_t* idx, int64_t T, int64_t k, int64_t E, int64_t chunk,
                                       const void* input, size_t row_bytes, void* dispatched, int32_t* offsets,
                                       int32_t* token_map, void* ws, hipStream_t s) {
    const int64_t pairs = T * k;
    const int nchunks = (int)((pairs + chunk - 1) / chunk);
    const int Ei = (int)E;
    int32_t* counts = (int32_t*)ws;
    int32_t* totals = (int32_t*)((unsigned char*)ws + dispatch_totals_offset(T, k, E));
    const int32_t* ranks = (const int32_t*)((unsigned char*)ws + dispatch_ranks_offset(T, k, E));
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_SCAN, s);
    dispatch_scan_kernel<<<Ei, 256, 0, s>>>(counts, nchunks, totals);
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_SCAN, s);
    const int ki = (int)k, ci = (int)chunk;
    auto copy = [&](auto unit) {
        typedef decltype(unit) V;
        const int64_t units = (int64_t)(row_bytes / sizeof(V));
        dispatch_copy_kernel<V><<<(unsigned)((T + 3) / 4), 256, E * sizeof(int), s>>>(
            (const V*)input, T, ki, Ei, units, idx, ci, nchunks, counts, totals, ranks, offsets, token_map,
            (V*)dispatched);
    };
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_COPY, s);
    if (row_bytes % 16 == 0 && ((uintptr_t)input % 16) == 0 && ((uintptr_t)dispatched % 16) == 0)
        copy(u32x4{});
    else if (row_bytes % 4 == 0 && ((uintptr_t)input % 4) == 0 && ((uintptr_t)dispatched % 4) == 0)
        copy(uint32_t{});
    else
        copy(uint16_t{});
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_COPY, s);
    return hipGetLastError();
}

hipError_t launch_dispatch(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input, size_t row_bytes,
                           void* dispatched, int32_t* offsets, int32_t* token_map, void* ws, hipStream_t s) {
    const int64_t pairs = T * k;
    const int64_t chunk = dispatch_chunk(pairs);
    const int nchunks = (int)((pairs + chunk - 1) / chunk);
    int32_t* ranks = (int32_t*)((unsigned char*)ws + dispatch_ranks_offset(T, k, E));
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_COUNT, s);
    dispatch_local_kernel<<<nchunks, 256, 5 * E * sizeof(int), s>>>(idx, pairs, (int)E, dispatch_id_bits(E),
                                                                   (int)chunk, (int32_t*)ws, ranks);
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_COUNT, s);
    return launch_dispatch_after_local(idx, T, k, E, chunk, input, row_bytes, dispatched, offsets, token_map, ws, s);
}

}  // namespace rudnn

// ---- rudnn_moe_dispatch_no_alloc: the dispatch workspace in a buffer the library owns ----
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an address (on the host
// it is only a stand-in for the device symbol): the device address is looked up once per
// device with hipGetSymbolAddress, that device current, and the kernels get that pointer.
// Nothing in it needs clearing: the local step writes every count and rank the scan and copy
// kernels read.  All calls on one GPU share the array, so calls that overlap on one GPU race.
namespace rudnn {
namespace {

constexpr size_t DISPATCH_SCRATCH_BYTES = RUDNN_MOE_DISPATCH_NO_ALLOC_MAX_BYTES;
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) int32_t scratch[DISPATCH_SCRATCH_BYTES / sizeof(int32_t)];

std::mutex g_scratch_mutex;
int32_t* g_scratch[MAX_DEVICES] = {};

rudnn_moe_status stream_device(hipStream_t s, int* dev) {
    const hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return RUDNN_MOE_ERR_DEVICE;
    }
    return RUDNN_MOE_OK;
}

// The device address of `scratch` on `dev`, looked up on the first call for that device.
rudnn_moe_status scratch_address(int dev, int32_t** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return RUDNN_MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) {
            (void)hipGetLastError();
            return RUDNN_MOE_ERR_DEVICE;
        }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return RUDNN_MOE_ERR_DEVICE;
        }
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return RUDNN_MOE_ERR_RUNTIME;
        }
        g_scratch[dev] = (int32_t*)p;
    }
    *out = g_scratch[dev];
    return RUDNN_MOE_OK;
}

}  // namespace
}  // namespace rudnn

using namespace rudnn;

extern "C" rudnn_moe_status rudnn_moe_dispatch_no_alloc(const uint32_t* idx, int64_t T, int64_t k, int64_t E,
                                                        const void* input, rudnn_moe_dtype dt, int64_t H,
                                                        void* dispatched, int32_t* offsets, int32_t* token_map,
                                                        hipStream_t stream) {
    rudnn_moe_status st = check_dispatch_args(idx, T, k, E, input, dt, H, dispatched, offsets, token_map);
    if (st != RUDNN_MOE_OK) return st;
    if (dispatch_workspace_bytes(T, k, E) > DISPATCH_SCRATCH_BYTES) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return dispatch_no_pairs(offsets, E, stream);
    if ((st = check_device(stream, {idx, input, dispatched, offsets, token_map})) != RUDNN_MOE_OK) return st;
    int dev = -1;
    int32_t* scratch_ptr = nullptr;
    if ((st = stream_device(stream, &dev)) != RUDNN_MOE_OK) return st;
    if ((st = scratch_address(dev, &scratch_ptr)) != RUDNN_MOE_OK) return st;
    return runtime(launch_dispatch(idx, T, k, E, input, (size_t)H * dtype_size(dt), dispatched, offsets, token_map,
                                   scratch_ptr, stream));
}
