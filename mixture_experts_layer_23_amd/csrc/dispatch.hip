// dispatch.hip -- capacity-free grouping of tokens by expert (ruDNN user guide, section 5
// "Expert weights and dispatch").
//
// The T*k (token, slot) pairs, flattened as a = t*k + j, are cut into chunks of `chunk` pairs
// (256..4096, see dispatch_chunk).  Four kernels:
//   count  one block per chunk: LDS histogram of the chunk's expert ids, stored as
//          chunk_counts[c, e] (every entry written, so nothing needs clearing first);
//   scan   one block per expert: the exclusive sum of its counts over the chunks (a block scan,
//          in place, turning counts into per-chunk bases) and the expert's total;
//   rank   one block per chunk: the exclusive sum of the totals over experts (every block, in
//          LDS; block 0 stores it as expert_offsets[E+1]), then the stable rank of each pair
//          among the chunk's pairs of the same expert (the lanes of a wavefront holding the
//          same id are found with one ballot per id bit, LDS counters carry across the block's
//          waves and rounds); token_map[a] = offsets[e] + base[c, e] + rank.  Rows of an expert
//          therefore follow (t, j) order, and the result does not depend on scheduling (no
//          global atomics);
//   copy   one wavefront per (token, 2 KiB piece of the row): the piece is read from HBM once
//          in 16-byte vectors and written to the token's k dispatched rows (plain stores
//          measured faster here than non-temporal ones).
// HBM traffic: T*k*4 (ids, twice) + T*H*s (tokens, once) + T*k*H*s (rows) + T*k*4 (map).
#include <mutex>

#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

__global__ __launch_bounds__(256) void dispatch_count_kernel(const uint32_t* __restrict__ idx, int64_t pairs, int E,
                                                             int chunk, int32_t* __restrict__ chunk_counts) {
    extern __shared__ int hist[];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int64_t a0 = (int64_t)blockIdx.x * chunk;
    const int64_t a1 = min(pairs, a0 + chunk);
    for (int64_t a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
        const uint32_t e = idx[a];
        if (e < (uint32_t)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Block e: the exclusive prefix of expert e's counts over the chunks, 256 chunks per pass.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                            int32_t* __restrict__ totals) {
    __shared__ int scratch[17];
    const int e = blockIdx.x;
    int running = 0;
    for (int c0 = 0; c0 < nchunks; c0 += blockDim.x) {
        const int c = c0 + (int)threadIdx.x;
        const int v = c < nchunks ? chunk_counts[(int64_t)c * E + e] : 0;
        int pass_total;
        const int excl = block_exclusive_scan(v, scratch, &pass_total);
        if (c < nchunks) chunk_counts[(int64_t)c * E + e] = running + excl;
        running += pass_total;
    }
    if (threadIdx.x == 0) totals[e] = running;
}

__global__ __launch_bounds__(256) void dispatch_rank_kernel(const uint32_t* __restrict__ idx, int64_t pairs, int E,
                                                            int id_bits, int chunk,
                                                            const int32_t* __restrict__ chunk_base,
                                                            const int32_t* __restrict__ totals,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ token_map) {
    extern __shared__ int sm[];
    __shared__ int scratch[17];
    int* off = sm;           // [E]    expert offsets (exclusive sum of the totals)
    int* run = sm + E;       // [E]    pairs of expert e already ranked in earlier rounds
    int* wcnt = sm + 2 * E;  // [4][E] pairs of expert e held by wave w in this round
    for (int i = threadIdx.x; i < 5 * E; i += blockDim.x) sm[E + i] = 0;
    for (int e0 = 0, carry = 0; e0 < E; e0 += blockDim.x) {  // E <= 1024: at most 4 passes
        const int e = e0 + (int)threadIdx.x;
        int pass_total;
        const int excl = block_exclusive_scan(e < E ? totals[e] : 0, scratch, &pass_total);
        if (e < E) off[e] = carry + excl;
        carry += pass_total;
        if (blockIdx.x == 0 && threadIdx.x == 0 && e0 + (int)blockDim.x >= E) offsets[E] = carry;
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = off[e];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t a0 = (int64_t)blockIdx.x * chunk;
    const int64_t a1 = min(pairs, a0 + chunk);
    const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
    for (int64_t r0 = a0; r0 < a1; r0 += blockDim.x) {
        const int64_t a = r0 + threadIdx.x;
        const bool in = a < a1;
        const uint32_t e = in ? idx[a] : 0xffffffffu;
        const bool valid = in && e < (uint32_t)E;
        // Lanes holding the same id: agree with this lane on every id bit.
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < id_bits; ++b) {
            const uint64_t ones = __ballot(valid && ((e >> b) & 1u));
            peers &= ((e >> b) & 1u) ? ones : ~ones;
        }
        const int rank = __popcll(peers & lt_mask);
        const bool leader = valid && rank == 0;  // the lowest lane of its id
        if (leader) wcnt[wave * E + e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int r = run[e] + rank;
            for (int w = 0; w < wave; ++w) r += wcnt[w * E + e];
            token_map[a] = off[e] + base[e] + r;
        } else if (in) {
            token_map[a] = -1;
        }
        __syncthreads();
        if (leader) {  // one leader per id and wave: waves holding the same id add concurrently
            atomicAdd(&run[e], __popcll(peers));
            wcnt[wave * E + e] = 0;
        }
        __syncthreads();
    }
}

// One wavefront per (token, piece of 64 * RUDNN_COPY_UNROLL copy units); V is the copy unit (a
// 16-byte vector when the row allows it).
#ifndef RUDNN_COPY_UNROLL
#define RUDNN_COPY_UNROLL 2
#endif
#ifndef RUDNN_COPY_NT
#define RUDNN_COPY_NT 0
#endif
template <typename V>
__global__ __launch_bounds__(256) void dispatch_copy_kernel(const V* __restrict__ x, int64_t T, int k, int64_t row_units,
                                                            int pieces, const int32_t* __restrict__ token_map,
                                                            V* __restrict__ out) {
    constexpr int U = RUDNN_COPY_UNROLL;  // 64-unit pieces per wavefront
    const int lane = lane_id();
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = w / pieces;
    if (t >= T) return;
    const int64_t i0 = (w - t * pieces) * 64 * U + lane;
    const int my_row = lane < k ? token_map[t * k + lane] : -1;
    V v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (i0 + u * 64 < row_units) v[u] = x[t * row_units + i0 + u * 64];
    for (int j = 0; j < k; ++j) {
        const int dst = readlane(my_row, j);
        if (dst < 0) continue;
        V* d = out + (int64_t)dst * row_units;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (i0 + u * 64 < row_units) {
                if (RUDNN_COPY_NT)
                    __builtin_nontemporal_store(v[u], d + i0 + u * 64);
                else
                    d[i0 + u * 64] = v[u];
            }
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

hipError_t launch_dispatch(const uint32_t* idx, int64_t T, int64_t k, int64_t E, const void* input, size_t row_bytes,
                           void* dispatched, int32_t* offsets, int32_t* token_map, int32_t* chunk_counts,
                           hipStream_t s) {
    const int64_t pairs = T * k;
    const int chunk = (int)dispatch_chunk(pairs);
    const int nchunks = (int)dispatch_chunks(pairs);
    const int Ei = (int)E;
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_COUNT, s);
    dispatch_count_kernel<<<nchunks, 256, E * sizeof(int), s>>>(idx, pairs, Ei, chunk, chunk_counts);
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_COUNT, s);
    int32_t* totals = (int32_t*)((unsigned char*)chunk_counts + dispatch_totals_offset(pairs, E));
    int id_bits = 0;
    while (((int64_t)1 << id_bits) < E) ++id_bits;
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_SCAN, s);
    dispatch_scan_kernel<<<Ei, 256, 0, s>>>(chunk_counts, nchunks, Ei, totals);
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_SCAN, s);
    timing_before(RUDNN_MOE_KERNEL_DISPATCH_RANK, s);
    dispatch_rank_kernel<<<nchunks, 256, 6 * E * sizeof(int), s>>>(idx, pairs, Ei, id_bits, chunk, chunk_counts,
                                                                    totals, offsets, token_map);
    timing_after(RUDNN_MOE_KERNEL_DISPATCH_RANK, s);
    const int ki = (int)k;
    auto copy = [&](auto unit) {
        typedef decltype(unit) V;
        const int64_t units = (int64_t)(row_bytes / sizeof(V));
        const int pieces = (int)((units + 64 * RUDNN_COPY_UNROLL - 1) / (64 * RUDNN_COPY_UNROLL));
        const int64_t waves = T * pieces;
        dispatch_copy_kernel<V><<<(unsigned)((waves + 3) / 4), 256, 0, s>>>((const V*)input, T, ki, units, pieces,
                                                                          token_map, (V*)dispatched);
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

}  // namespace rudnn

// ---- rudnn_moe_dispatch_no_alloc: the per-chunk counts in a buffer the library owns ----
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never uses the array's name as an address (on the host
// it is only a stand-in for the device symbol): the device address is looked up once per
// device with hipGetSymbolAddress, that device current, and the kernels get that pointer.
// Nothing in it needs clearing: the count kernel writes every entry the scan and rank kernels
// read.  All calls on one GPU share the array, so calls that overlap on one GPU race.
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
    if (dispatch_workspace_bytes(T * k, E) > DISPATCH_SCRATCH_BYTES) return RUDNN_MOE_ERR_UNSUPPORTED;
    if (T == 0) return dispatch_no_pairs(offsets, E, stream);
    if ((st = check_device(stream, {idx, input, dispatched, offsets, token_map})) != RUDNN_MOE_OK) return st;
    int dev = -1;
    int32_t* counts = nullptr;
    if ((st = stream_device(stream, &dev)) != RUDNN_MOE_OK) return st;
    if ((st = scratch_address(dev, &counts)) != RUDNN_MOE_OK) return st;
    return runtime(launch_dispatch(idx, T, k, E, input, (size_t)H * dtype_size(dt), dispatched, offsets, token_map,
                                   counts, stream));
}
