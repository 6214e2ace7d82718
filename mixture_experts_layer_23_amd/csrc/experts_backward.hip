// experts_backward.hip -- backward of the bias-free SwiGLU experts on the dispatched rows (ruDNN
// user guide, section 12 step 2: cache.backward(dexpert) -> dinput for the dispatched rows and
// FP32 dgate, dup, ddown).  For the rows r of expert e (x = dispatched, dy = dexpert):
//   [g | u] = x [gate_e; up_e]^T          FP32, recomputed (the forward's inputs are the cache)
//   dh      = dy down_e                    FP32, fused epilogue:
//             dg = dtype(dh u silu'(g)), du = dtype(dh silu(g)), h = dtype(silu(g) u)
//   dx      = [dg | du] [gate_e; up_e]     -> grad_dispatched (dtype)
//   dgate_e = dg^T x,  dup_e = du^T x,  ddown_e = dy^T h     (FP32, sums over the expert's rows)
// silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).
//
// One MFMA kernel serves all five products: C[m, n] = sum_k A(m, k) B(n, k), 128 x 128 tiles,
// K staged 64 bytes per row, four wavefronts of 64 x 64 (v_mfma_f32_32x32x16 for BF16/F16,
// 32x32x2f32 for FP32).  An operand is either "K-major" (k contiguous: staged as 16-byte pieces)
// or "X-major" (its row/column index contiguous: 16-byte pieces of 8 (or 4) consecutive x at
// one k, scattered into the [x][k] LDS tile by element stores).  The operand tiles go through
// registers: step k+1 is loaded while step k computes, then written to the other LDS stage.
// Two operand sources may be stacked along the operand's outer index (gate over up).
// Grouping: ROWS tiles the expert's rows along M (a device-side plan of m-tiles per expert);
// KROWS uses the expert's rows as the contraction axis, every (expert, m, n) tile (an expert
// without rows gets zeros).
#include "device.hpp"
#include "internal.hpp"

namespace rudnn {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, ROWB = 64, THREADS = 256;

template <typename T>
struct Mma;
template <>
struct Mma<bf16> {
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<f16> {
    typedef f16x8 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mma<float> {  // four 32x32x2 steps over one 16-byte chunk per lane half (see route_projected)
    typedef float4 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
    }
};

// 64-byte staged rows: chunk c of row r at slot c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// An operand: element (outer o, inner i) at src(o) + e * estride + o' * ld + i, with src = p0 and
// o' = o for o < split, else p1 and o' = o - split.  K-major: outer = the operand's row (m or n),
// inner = k.  X-major: outer = k, inner = the row.
struct Opnd {
    const void* p0;
    const void* p1;
    int64_t ld, estride;
    int split;
};

template <typename T>
__device__ __forceinline__ const T* opnd_row(const Opnd& o, int e, int64_t outer) {
    const bool hi = outer >= o.split;
    const T* base = reinterpret_cast<const T*>(hi ? o.p1 : o.p0);
    return base + (int64_t)e * o.estride + (hi ? outer - o.split : outer) * o.ld;
}

enum { EPI_F32 = 0, EPI_DT = 1, EPI_SWIGLU = 2 };
enum { ROWS = 0, KROWS = 1 };

struct Plan {
    const int32_t* row_begin;  // [E]
    const int32_t* row_count;  // [E]
    const int32_t* mt_begin;   // [E + 1]
};

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int rows,
                                                    int32_t* __restrict__ row_begin, int32_t* __restrict__ row_count,
                                                    int32_t* __restrict__ mt_begin) {
    __shared__ int scratch[17];
    int tiles = 0;
    for (int e0 = 0, carry = 0; e0 < E; e0 += blockDim.x) {
        const int e = e0 + (int)threadIdx.x;
        tiles = 0;
        if (e < E) {
            const int a = min(max(offsets[e], 0), rows), b = min(max(offsets[e + 1], 0), rows);
            const int n = max(b - a, 0);
            row_begin[e] = a;
            row_count[e] = n;
            tiles = (n + BM - 1) / BM;
        }
        int total;
        const int excl = block_exclusive_scan(tiles, scratch, &total);
        if (e < E) mt_begin[e] = carry + excl;
        carry += total;
        if (threadIdx.x == 0 && e0 + (int)blockDim.x >= E) mt_begin[E] = carry;
    }
}

struct Epi {
    void* c;              // output: FP32 or dtype, [rows or E*M, N] row-major
    int64_t ldc;          // row stride of the output
    const float* gu;      // EPI_SWIGLU: [rows, 2 I] FP32 (g | u)
    void* dgu;            // EPI_SWIGLU: [rows, 2 I] dtype (dg | du)
    void* h;              // EPI_SWIGLU: [rows, I] dtype
};

// C = A B^T on 128 x 128 tiles; see the file comment.
template <typename T, int MODE, int EPI, bool AK, bool BK>
__global__ __launch_bounds__(THREADS) void gemm_kernel(Opnd A, Opnd B, int M, int N, int K, int E, Plan plan,
                                                       const int32_t* __restrict__ offsets, int rows, int NT, int MT,
                                                       Epi ep) {
    constexpr int CE = 16 / (int)sizeof(T);  // elements per 16-byte chunk
    constexpr int BKE = ROWB / (int)sizeof(T);  // K elements per step
    typedef typename Mma<T>::frag frag;
    __shared__ __align__(16) unsigned char lds[2][(BM + BN) * ROWB];

    // ---- which tile ----
    int e, m0, n0, mlim, kb, kn;  // expert, tile origin, valid rows, K origin and length
    int64_t row0 = 0;             // ROWS: first dispatched row of the tile
    if (MODE == ROWS) {
        const int64_t L = blockIdx.x, Mt = L / NT;
        if (Mt >= plan.mt_begin[E]) return;
        int lo = 0, hi = E - 1;  // largest e with mt_begin[e] <= Mt
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (plan.mt_begin[mid] <= Mt)
                lo = mid;
            else
                hi = mid - 1;
        }
        e = lo;
        const int mt = (int)(Mt - plan.mt_begin[e]);
        n0 = (int)(L % NT) * BN;
        m0 = 0;
        row0 = plan.row_begin[e] + (int64_t)mt * BM;
        mlim = min(BM, plan.row_count[e] - mt * BM);
        kb = 0, kn = K;
    } else {
        const int64_t L = blockIdx.x;
        e = (int)(L / ((int64_t)MT * NT));
        const int r = (int)(L % ((int64_t)MT * NT));
        m0 = (r / NT) * BM, n0 = (r % NT) * BN;
        mlim = min(BM, M - m0);
        const int a = min(max(offsets[e], 0), rows), b = min(max(offsets[e + 1], 0), rows);
        kb = a, kn = max(b - a, 0);
    }
    const int nlim = min(BN, N - n0);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- staging: two 16-byte pieces per thread per operand per step ----
    uint4 ra[2], rb[2];
    auto load_k = [&](const Opnd& o, bool is_a, int xlim, int k0, uint4 (&r)[2]) __attribute__((always_inline)) {
        // K-major: piece c -> row x = c / 4, chunk c % 4
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + q * THREADS, x = c >> 2, kc = c & 3;
            const int k = k0 + kc * CE;
            r[q] = make_uint4(0, 0, 0, 0);
            if (x < xlim && k < kn) {
                const int64_t outer = is_a ? (MODE == ROWS ? row0 + x : (int64_t)(m0 + x)) : (int64_t)(n0 + x);
                const T* p = opnd_row<T>(o, MODE == ROWS && is_a ? 0 : e, outer) + kb + k;
                r[q] = *reinterpret_cast<const uint4*>(p);
            }
        }
    };
    auto load_x = [&](const Opnd& o, bool is_a, int xlim, int k0, uint4 (&r)[2]) __attribute__((always_inline)) {
        // X-major: piece c -> k row kk = c / (128 / CE), x chunk c % (128 / CE)
        constexpr int CPK = 128 / CE;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + q * THREADS, kk = c / CPK, x = (c % CPK) * CE;
            const int k = k0 + kk;
            r[q] = make_uint4(0, 0, 0, 0);
            if (x < xlim && k < kn) {
                const int64_t outer = kb + k;
                const int64_t xo = is_a ? (MODE == ROWS ? row0 + x : (int64_t)(m0 + x)) : (int64_t)(n0 + x);
                const T* p = opnd_row<T>(o, MODE == KROWS ? 0 : e, outer) + xo;
                r[q] = *reinterpret_cast<const uint4*>(p);
            }
        }
    };
    auto store_k = [&](unsigned char* st, const uint4 (&r)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + q * THREADS, x = c >> 2, kc = c & 3;
            *reinterpret_cast<uint4*>(st + x * ROWB + ((kc ^ swz(x)) * 16)) = r[q];
        }
    };
    auto store_x = [&](unsigned char* st, const uint4 (&r)[2]) __attribute__((always_inline)) {
        constexpr int CPK = 128 / CE;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + q * THREADS, kk = c / CPK, x0 = (c % CPK) * CE;
            const T* v = reinterpret_cast<const T*>(&r[q]);
#pragma unroll
            for (int i = 0; i < CE; ++i) {
                const int x = x0 + i;
                *reinterpret_cast<T*>(st + x * ROWB + (((kk / CE) ^ swz(x)) * 16) + (kk % CE) * (int)sizeof(T)) = v[i];
            }
        }
    };
    auto load_step = [&](int kt) __attribute__((always_inline)) {
        const int k0 = kt * BKE;
        if (AK)
            load_k(A, true, mlim, k0, ra);
        else
            load_x(A, true, mlim, k0, ra);
        if (BK)
            load_k(B, false, nlim, k0, rb);
        else
            load_x(B, false, nlim, k0, rb);
    };
    auto store_step = [&](int kt) __attribute__((always_inline)) {
        unsigned char* st = lds[kt & 1];
        if (AK)
            store_k(st, ra);
        else
            store_x(st, ra);
        if (BK)
            store_k(st + BM * ROWB, rb);
        else
            store_x(st + BM * ROWB, rb);
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int fr = lane & 31, fh = lane >> 5;
    const int KT = (kn + BKE - 1) / BKE;
    if (KT > 0) {
        load_step(0);
        store_step(0);
    }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load_step(kt + 1);  // into registers, under this step's MFMAs
        const unsigned char* st = lds[kt & 1];
        const unsigned char* sa = st + (wm * 64 + fr) * ROWB;
        const unsigned char* sb = st + BM * ROWB + (wn * 64 + fr) * ROWB;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int off = ((ks * 2 + fh) ^ swz(fr)) * 16;
            frag fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = *reinterpret_cast<const frag*>(sa + i * 32 * ROWB + off);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const frag*>(sb + j * 32 * ROWB + off);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = Mma<T>::run(fb[j], fa[i], acc[i][j]);
        }
        if (kt + 1 < KT) store_step(kt + 1);  // the other stage: last read in step kt - 1
        __syncthreads();
    }

    // ---- epilogue: lane holds row m = fr of each 32-row block, columns 8 (v / 4) + 4 fh + v % 4 ----
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ml = wm * 64 + i * 32 + fr;
        if (ml >= mlim) continue;
        const int64_t crow = MODE == ROWS ? row0 + ml : (int64_t)e * M + m0 + ml;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 64 + j * 32 + 8 * q + 4 * fh;
                if (nl >= nlim) continue;  // N is a multiple of 4: a run of 4 is wholly in or out
                const int n = n0 + nl;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                            v3 = acc[i][j][4 * q + 3];
                if (EPI == EPI_F32) {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.c) + crow * ep.ldc + n) =
                        make_float4(v0, v1, v2, v3);
                } else if (EPI == EPI_DT) {
                    T* c = reinterpret_cast<T*>(ep.c) + crow * ep.ldc + n;
                    c[0] = from_f32<T>(v0), c[1] = from_f32<T>(v1), c[2] = from_f32<T>(v2), c[3] = from_f32<T>(v3);
                } else {  // dh -> dg, du, h; N = I
                    const float dh[4] = {v0, v1, v2, v3};
                    const float* gr = ep.gu + crow * 2 * (int64_t)N + n;
                    T* dg = reinterpret_cast<T*>(ep.dgu) + crow * 2 * (int64_t)N + n;
                    T* hh = reinterpret_cast<T*>(ep.h) + crow * (int64_t)N + n;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float g = gr[t], u = gr[N + t];
                        const float s = 1.f / (1.f + expf(-g));
                        dg[t] = from_f32<T>(dh[t] * u * (s * (1.f + g * (1.f - s))));
                        dg[N + t] = from_f32<T>(dh[t] * (g * s));
                        hh[t] = from_f32<T>(g * s * u);
                    }
                }
            }
    }
}

}  // namespace bwd

// ---- host side ----

size_t experts_backward_workspace_bytes(int64_t E, int64_t I, rudnn_moe_dtype dt, int64_t rows) {
    const size_t es = dtype_size(dt);
    return align_up((size_t)rows * 2 * I * 4) + align_up((size_t)rows * 2 * I * es) + align_up((size_t)rows * I * es) +
           align_up(sizeof(int32_t) * (size_t)(3 * E + 1));
}

namespace {

template <typename T, int MODE, int EPI, bool AK, bool BK>
void gemm(bwd::Opnd A, bwd::Opnd B, int M, int N, int K, int E, bwd::Plan plan, const int32_t* offsets, int rows,
          bwd::Epi ep, rudnn_moe_kernel kid, hipStream_t s) {
    const int NT = (N + bwd::BN - 1) / bwd::BN, MT = (M + bwd::BM - 1) / bwd::BM;
    const int64_t blocks = MODE == bwd::ROWS ? ((int64_t)rows / bwd::BM + E) * NT : (int64_t)E * MT * NT;
    if (blocks <= 0) return;
    timing_before(kid, s);
    bwd::gemm_kernel<T, MODE, EPI, AK, BK><<<dim3((unsigned)blocks), dim3(bwd::THREADS), 0, s>>>(
        A, B, M, N, K, E, plan, offsets, rows, NT, MT, ep);
    timing_after(kid, s);
}

template <typename T>
void run(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets, int64_t rows, const void* dy, void* dx,
         float* dgate, float* dup, float* ddown, void* workspace, hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate, R = (int)rows;
    const size_t es = sizeof(T);
    unsigned char* ws = (unsigned char*)workspace;
    float* gu = (float*)ws;
    T* dgu = (T*)(ws + align_up((size_t)rows * 2 * I * 4));
    T* hbuf = (T*)((unsigned char*)dgu + align_up((size_t)rows * 2 * I * es));
    int32_t* pl = (int32_t*)((unsigned char*)hbuf + align_up((size_t)rows * I * es));
    bwd::Plan plan{pl, pl + E, pl + 2 * E};
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_PLAN, s);
    bwd::plan_kernel<<<1, 1024, 0, s>>>(offsets, E, R, pl, pl + E, pl + 2 * E);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_PLAN, s);
    const int NOSPLIT = 0x7fffffff;
    const int64_t IH = (int64_t)I * H;
    // [g | u] = x [gate; up]^T  (B K-major, gate rows then up rows)
    gemm<T, bwd::ROWS, bwd::EPI_F32, true, true>({x, x, H, 0, NOSPLIT}, {ex->gate, ex->up, H, IH, I}, R, 2 * I, H, E,
                                                 plan, offsets, R, {gu, 2 * (int64_t)I, nullptr, nullptr, nullptr},
                                                 RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_GU, s);
    // dh = dy down_e (B(n = i, k = c) = down[e, c, i]: X-major), epilogue -> dg | du, h
    gemm<T, bwd::ROWS, bwd::EPI_SWIGLU, true, false>({dy, dy, H, 0, NOSPLIT}, {ex->down, ex->down, I, IH, NOSPLIT}, R, I,
                                                     H, E, plan, offsets, R, {nullptr, 0, gu, dgu, hbuf},
                                                     RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DH, s);
    // dx = [dg | du] [gate; up]  (B(n = c, k = i') = gate[e, i', c] or up[e, i' - I, c]: X-major)
    gemm<T, bwd::ROWS, bwd::EPI_DT, true, false>({dgu, dgu, 2 * (int64_t)I, 0, NOSPLIT}, {ex->gate, ex->up, H, IH, I}, R,
                                                 H, 2 * I, E, plan, offsets, R, {dx, H, nullptr, nullptr, nullptr},
                                                 RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DX, s);
    // dgate_e = dg^T x, dup_e = du^T x  (both X-major, K = the expert's rows)
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dgu, dgu, 2 * (int64_t)I, 0, NOSPLIT}, {x, x, H, 0, NOSPLIT}, I, H,
                                                    0, E, plan, offsets, R, {dgate, H, nullptr, nullptr, nullptr},
                                                    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dgu + I, dgu + I, 2 * (int64_t)I, 0, NOSPLIT},
                                                    {x, x, H, 0, NOSPLIT}, I, H, 0, E, plan, offsets, R,
                                                    {dup, H, nullptr, nullptr, nullptr},
                                                    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
    // ddown_e = dy^T h
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dy, dy, H, 0, NOSPLIT}, {hbuf, hbuf, I, 0, NOSPLIT}, H, I, 0, E,
                                                    plan, offsets, R, {ddown, I, nullptr, nullptr, nullptr},
                                                    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
}

}  // namespace

hipError_t launch_experts_backward(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets, int64_t rows,
                                   const void* dy, void* dx, float* dgate, float* dup, float* ddown, void* workspace,
                                   hipStream_t s) {
    switch (ex->dtype) {
    case RUDNN_MOE_F32: run<float>(ex, x, offsets, rows, dy, dx, dgate, dup, ddown, workspace, s); break;
    case RUDNN_MOE_F16: run<f16>(ex, x, offsets, rows, dy, dx, dgate, dup, ddown, workspace, s); break;
    default: run<bf16>(ex, x, offsets, rows, dy, dx, dgate, dup, ddown, workspace, s); break;
    }
    return hipGetLastError();
}

}  // namespace rudnn
