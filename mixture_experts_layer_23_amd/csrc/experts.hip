// experts.hip -- bias-free SwiGLU experts on the dispatched rows (ruDNN user guide, sections
// 3 and 5: SwiGluExperts::forward_dispatched; gate/up [E,I,H], down [E,H,I]).
//
//   h[r, :] = dtype( silu(X_e gate_e^T) * (X_e up_e^T) )  for the rows r of expert e
//   y[r, :] = dtype( h_e down_e^T )
//
// Both products contract over a contiguous axis of both operands ("TN" GEMMs).  Three kernels:
//   plan     one block: clamps the device-side expert offsets to [0, rows], counts BM-row
//            tiles per expert and their exclusive prefix (no host round trip, no sync);
//   gate_up  grouped GEMM, N = I, fused epilogue silu(g) * u (two accumulator sets per tile);
//   down     grouped GEMM, N = H, K = I.
// BF16/F16: v_mfma_f32_32x32x16_{bf16,f16} with FP32 accumulators; 512-thread blocks of eight
// wavefronts, output tile 256 rows x 256 accumulator columns (gate_up: 128 of gate + 128 of up),
// K staged 64 at a time through LDS (row pitch 144 B against bank conflicts), double-buffered:
// the global loads of step k+1 are in flight while the MFMAs consume step k.
// F32: the same schedule with an FP32 FMA tile (64 x 64) -- there is no reduced-precision step.
//
// Tile order.  Tiles of expert e are enumerated in groups of GROUP_N n-tiles, all m-tiles of a
// group together, so tiles that run side by side share both their weight columns and their
// token rows.  Workgroup i runs on XCD i % 8 (round-robin); block i therefore takes logical
// tile (start of XCD i % 8's share) + i / 8, so each XCD walks a contiguous, equal share of
// the tile list and its 4 MB L2 sees the reuse.  The grid is sized for the worst case
// (floor(rows / BM) + min(E, rows) m-tiles); blocks beyond the real count exit at once.
#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GROUP_N = 8;

// ---------------------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------------------
struct Plan {
    int32_t* row_begin;  // [E]
    int32_t* row_count;  // [E]
    int32_t* mt_begin;   // [E + 1]
};

__global__ __launch_bounds__(1024) void experts_plan_kernel(const int32_t* __restrict__ offsets, int E, int rows,
                                                            int BM, Plan plan) {
    __shared__ int scratch[17];
    const int e = threadIdx.x;
    int tiles = 0;
    if (e < E) {
        const int a = min(max(offsets[e], 0), rows);
        const int b = min(max(offsets[e + 1], 0), rows);
        const int n = max(b - a, 0);
        plan.row_begin[e] = a;
        plan.row_count[e] = n;
        tiles = (n + BM - 1) / BM;
    }
    int total;
    const int excl = block_exclusive_scan(tiles, scratch, &total);
    if (e < E) plan.mt_begin[e] = excl;
    if (e == 0) plan.mt_begin[E] = total;
}

struct Tile {
    int e, row0, nrows, n0;
};

// Maps this block to a tile; false if the block has no tile.  `s_mt` is __shared__ int[E+1].
template <int BM, int BN>
__device__ __forceinline__ bool find_tile(const Plan& plan, int E, int N, int* s_mt, Tile& t) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_mt[i] = plan.mt_begin[i];
    __syncthreads();
    const int NT = (N + BN - 1) / BN;
    const int64_t total = (int64_t)s_mt[E] * NT;
    const int xcd = blockIdx.x & 7;
    const int64_t slot = blockIdx.x >> 3;
    const int64_t q = total >> 3, r = total & 7;
    const int64_t count = q + (xcd < r ? 1 : 0);
    if (slot >= count) return false;
    const int64_t L = xcd * q + min((int64_t)xcd, r) + slot;
    const int64_t M = L / NT;  // the expert owns m-tile rows [s_mt[e], s_mt[e+1])
    int lo = 0, hi = E - 1;    // largest e with s_mt[e] <= M
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_mt[mid] <= M)
            lo = mid;
        else
            hi = mid - 1;
    }
    const int e = lo;
    const int mt_e = s_mt[e + 1] - s_mt[e];
    const int64_t rr = L - (int64_t)s_mt[e] * NT;
    const int64_t g = rr / ((int64_t)GROUP_N * mt_e);
    const int64_t qq = rr - g * GROUP_N * mt_e;
    const int gn = (int)min((int64_t)GROUP_N, NT - g * GROUP_N);
    const int mt = (int)(qq / gn);
    const int nt = (int)(g * GROUP_N + qq % gn);
    t.e = e;
    t.row0 = plan.row_begin[e] + mt * BM;
    t.nrows = min(BM, plan.row_count[e] - mt * BM);
    t.n0 = nt * BN;
    return true;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------------------
// MFMA grouped GEMM (bf16 / f16)
// ---------------------------------------------------------------------------------------
template <typename T>
struct Mfma;
template <>
struct Mfma<bf16> {
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<f16> {
    typedef f16x8 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int MF_BM = 256;             // rows per tile
constexpr int MF_BK = 64;              // K elements per LDS stage
constexpr int MF_PITCH = MF_BK + 8;    // LDS row pitch in elements (144 B)
constexpr int MF_THREADS = 512;        // 8 wavefronts: 4 along M x 2 along N
constexpr int MF_WM = 4, MF_WN = 2;

// DUAL: B0 = gate, B1 = up, BN = 128 columns of each; else B0 only, BN = 256.
template <typename T, bool DUAL>
__global__ __launch_bounds__(MF_THREADS) void grouped_gemm_mfma(const T* __restrict__ A, const T* __restrict__ B0,
                                                                const T* __restrict__ B1, T* __restrict__ C, int K,
                                                                int N, int E, Plan plan) {
    constexpr int BM = MF_BM;
    constexpr int BN = DUAL ? 128 : 256;    // output columns per tile
    constexpr int NB = DUAL ? 2 * BN : BN;  // B rows staged per tile
    constexpr int WTM = BM / MF_WM;         // 64
    constexpr int WTN = BN / MF_WN;         // 64 (DUAL) or 128
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int NSETS = DUAL ? 2 : 1;
    constexpr int A_CHUNKS = BM * (MF_BK / 8) / MF_THREADS;  // 16-byte chunks per thread
    constexpr int B_CHUNKS = NB * (MF_BK / 8) / MF_THREADS;
    typedef typename Mfma<T>::frag frag;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    int* s_mt = reinterpret_cast<int*>(smem_raw);
    Tile tile;
    if (!find_tile<BM, BN>(plan, E, N, s_mt, tile)) return;
    __syncthreads();  // s_mt shares space with the stages
    T* sA = reinterpret_cast<T*>(smem_raw);
    T* sB = sA + 2 * BM * MF_PITCH;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % MF_WM, wn = wave / MF_WM;
    const int e = tile.e, nrows = tile.nrows, n0 = tile.n0;
    const T* Ab = A + (int64_t)tile.row0 * K;
    const T* B0e = B0 + (int64_t)e * N * K;
    const T* B1e = DUAL ? B1 + (int64_t)e * N * K : nullptr;

    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int q = tid + i * MF_THREADS, row = q >> 3, c = q & 7;
            const int kk = k0 + c * 8;
            ra[i] = (row < nrows && kk < K) ? *reinterpret_cast<const uint4*>(Ab + (int64_t)row * K + kk)
                                            : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int q = tid + i * MF_THREADS, row = q >> 3, c = q & 7;
            const int kk = k0 + c * 8;
            const T* src = B0e;
            int n = n0 + row;
            if (DUAL && row >= BN) {
                src = B1e;
                n -= BN;
            }
            rb[i] = (n < N && kk < K) ? *reinterpret_cast<const uint4*>(src + (int64_t)n * K + kk)
                                      : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int stage) {
        T* a = sA + stage * BM * MF_PITCH;
        T* b = sB + stage * NB * MF_PITCH;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int q = tid + i * MF_THREADS, row = q >> 3, c = q & 7;
            *reinterpret_cast<uint4*>(a + row * MF_PITCH + c * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) {
            const int q = tid + i * MF_THREADS, row = q >> 3, c = q & 7;
            *reinterpret_cast<uint4*>(b + row * MF_PITCH + c * 8) = rb[i];
        }
    };

    f32x16 acc[NSETS][FM][FN];
#pragma unroll
    for (int s = 0; s < NSETS; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[s][i][j][v] = 0.f;

    // Rows of this wavefront that hold real tokens: skip the MFMAs of empty 32-row blocks.
    const int wave_rows = min(max(nrows - wm * WTM, 0), WTM);
    const int fr = lane & 31, fh = lane >> 5;

    const int KT = (K + MF_BK - 1) / MF_BK;
    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load((kt + 1) * MF_BK);
        if (wave_rows > 0) {
            const T* a = sA + cur * BM * MF_PITCH + (wm * WTM + fr) * MF_PITCH;
            const T* b = sB + cur * NB * MF_PITCH + (wn * WTN + fr) * MF_PITCH;
#pragma unroll
            for (int ks = 0; ks < MF_BK / 16; ++ks) {
                const int off = (ks * 2 + fh) * 8;
                frag fa[FM], fb[NSETS][FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const frag*>(a + i * 32 * MF_PITCH + off);
#pragma unroll
                for (int s = 0; s < NSETS; ++s)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        fb[s][j] = *reinterpret_cast<const frag*>(b + (s * BN + j * 32) * MF_PITCH + off);
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    if (i * 32 >= wave_rows) continue;
#pragma unroll
                    for (int s = 0; s < NSETS; ++s)
#pragma unroll
                        for (int j = 0; j < FN; ++j) acc[s][i][j] = Mfma<T>::run(fa[i], fb[s][j], acc[s][i][j]);
                }
            }
        }
        if (kt + 1 < KT) store(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 MFMA output: lane l holds column l % 32 and rows
    // 8 * (v / 4) + 4 * (l / 32) + v % 4 for v = 0..15.
    T* Cb = C + (int64_t)tile.row0 * N + n0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = wn * WTN + j * 32 + fr;
            if (n0 + col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * WTM + i * 32 + 8 * (v >> 2) + 4 * fh + (v & 3);
                if (row >= nrows) continue;
                float val;
                if (DUAL)
                    val = silu_f(acc[0][i][j][v]) * acc[NSETS - 1][i][j][v];
                else
                    val = acc[0][i][j][v];
                Cb[(int64_t)row * N + col] = from_f32<T>(val);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// FP32 grouped GEMM (FMA): tile 64 x 64, K staged 16 at a time, 256 threads x (4 x 4) outputs.
// ---------------------------------------------------------------------------------------
constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float* __restrict__ A, const float* __restrict__ B0,
                                                        const float* __restrict__ B1, float* __restrict__ C, int K,
                                                        int N, int E, Plan plan) {
    __shared__ int s_mt[MAX_EXPERTS + 1];
    __shared__ float sA[F_BK][F_BM + 4];
    __shared__ float sB[DUAL ? 2 : 1][F_BK][F_BN + 4];
    Tile tile;
    if (!find_tile<F_BM, F_BN>(plan, E, N, s_mt, tile)) return;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const float* Ab = A + (int64_t)tile.row0 * K;
    const float* B0e = B0 + (int64_t)tile.e * N * K;
    const float* B1e = DUAL ? B1 + (int64_t)tile.e * N * K : nullptr;
    float acc[2][4][4] = {};
    for (int k0 = 0; k0 < K; k0 += F_BK) {
        // 64 rows x 16 k of A and of each B: 4 elements per thread each, stored k-major
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + i * 256, row = q >> 4, kk = q & 15;
            const bool kin = k0 + kk < K;
            sA[kk][row] = (row < tile.nrows && kin) ? Ab[(int64_t)row * K + k0 + kk] : 0.f;
            const int n = tile.n0 + row;
            sB[0][kk][row] = (n < N && kin) ? B0e[(int64_t)n * K + k0 + kk] : 0.f;
            if (DUAL) sB[DUAL ? 1 : 0][kk][row] = (n < N && kin) ? B1e[(int64_t)n * K + k0 + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < F_BK; ++kk) {
            float a[4], b[4], b1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = sB[0][kk][tx * 4 + j];
                b1[j] = DUAL ? sB[DUAL ? 1 : 0][kk][tx * 4 + j] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[0][i][j] = fmaf(a[i], b[j], acc[0][i][j]);
                    if (DUAL) acc[1][i][j] = fmaf(a[i], b1[j], acc[1][i][j]);
                }
        }
        __syncthreads();
    }
    float* Cb = C + (int64_t)tile.row0 * N + tile.n0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = ty * 4 + i;
        if (row >= tile.nrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = tx * 4 + j;
            if (tile.n0 + col >= N) continue;
            float v = acc[0][i][j];
            if (DUAL) v = (v / (1.0f + expf(-v))) * acc[1][i][j];
            Cb[(int64_t)row * N + col] = v;
        }
    }
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static int64_t max_mtiles(int64_t rows, int64_t E, int BM) { return rows / BM + (E < rows ? E : rows); }

size_t experts_workspace_bytes(int64_t E, int64_t H, int64_t I, rudnn_moe_dtype dt, int64_t rows) {
    (void)H;
    return align_up((size_t)rows * I * dtype_size(dt)) + align_up(sizeof(int32_t) * (3 * E + 1));
}

static size_t mfma_smem_bytes(bool dual, size_t es, int64_t E) {
    const size_t stages = 2 * (size_t)(MF_BM + (dual ? 256 : 256)) * MF_PITCH * es;
    const size_t mt = sizeof(int) * (size_t)(E + 1);
    return stages > mt ? stages : mt;
}

template <typename T>
static void launch_mfma(const rudnn_moe_experts* ex, const void* disp, int64_t rows, void* out, void* h, Plan plan,
                        hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate;
    const int64_t mt = max_mtiles(rows, E, MF_BM);
    auto grid_for = [&](int N, int BN) {
        const int64_t tiles = mt * ((N + BN - 1) / BN);
        return (unsigned)((tiles + 7) / 8 * 8);
    };
    const size_t es = sizeof(T);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    grouped_gemm_mfma<T, true><<<grid_for(I, 128), MF_THREADS, mfma_smem_bytes(true, es, E), s>>>(
        (const T*)disp, (const T*)ex->gate, (const T*)ex->up, (T*)h, H, I, E, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
    grouped_gemm_mfma<T, false><<<grid_for(H, 256), MF_THREADS, mfma_smem_bytes(false, es, E), s>>>(
        (const T*)h, (const T*)ex->down, nullptr, (T*)out, I, H, E, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
}

static void launch_f32(const rudnn_moe_experts* ex, const void* disp, int64_t rows, void* out, void* h, Plan plan,
                       hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate;
    const int64_t mt = max_mtiles(rows, E, F_BM);
    auto grid_for = [&](int N) { return (unsigned)((mt * ((N + F_BN - 1) / F_BN) + 7) / 8 * 8); };
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    grouped_gemm_f32<true><<<grid_for(I), 256, 0, s>>>((const float*)disp, (const float*)ex->gate,
                                                       (const float*)ex->up, (float*)h, H, I, E, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
    grouped_gemm_f32<false><<<grid_for(H), 256, 0, s>>>((const float*)h, (const float*)ex->down, nullptr,
                                                        (float*)out, I, H, E, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
}

static bool smem_configured = false;

hipError_t launch_experts(const rudnn_moe_experts* ex, const void* disp, const int32_t* offsets, int64_t rows,
                          void* out, void* workspace, hipStream_t s) {
    const int64_t E = ex->num_experts, I = ex->intermediate;
    const size_t es = dtype_size(ex->dtype);
    unsigned char* ws = (unsigned char*)workspace;
    void* h = ws;
    int32_t* ints = (int32_t*)(ws + align_up((size_t)rows * I * es));
    Plan plan{ints, ints + E, ints + 2 * E};
    if (!smem_configured) {
        // LDS beyond 64 KiB per block must be requested explicitly.
        hipFuncSetAttribute((const void*)grouped_gemm_mfma<bf16, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
        hipFuncSetAttribute((const void*)grouped_gemm_mfma<bf16, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
        hipFuncSetAttribute((const void*)grouped_gemm_mfma<f16, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
        hipFuncSetAttribute((const void*)grouped_gemm_mfma<f16, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
        smem_configured = true;
    }
    const int BM = ex->dtype == RUDNN_MOE_F32 ? F_BM : MF_BM;
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_PLAN, s);
    experts_plan_kernel<<<1, 1024, 0, s>>>(offsets, (int)E, (int)rows, BM, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_PLAN, s);
    switch (ex->dtype) {
    case RUDNN_MOE_F32: launch_f32(ex, disp, rows, out, h, plan, s); break;
    case RUDNN_MOE_F16: launch_mfma<f16>(ex, disp, rows, out, h, plan, s); break;
    default: launch_mfma<bf16>(ex, disp, rows, out, h, plan, s); break;
    }
    return hipGetLastError();
}

}  // namespace rudnn
