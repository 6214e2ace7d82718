// experts_backward.hip -- backward of the bias-free SwiGLU experts on the dispatched rows (ruDNN
// user guide, section 12 step 2: cache.backward(dexpert) -> dinput for the dispatched rows and
// FP32 dgate, dup, ddown).  For the rows r of expert e (x = dispatched, dy = dexpert):
//   [g | u] = x [gate_e; up_e]^T          FP32: the training forward's cache, or recomputed
//   dh      = dy down_e                    FP32, fused epilogue:
//             dg = dtype(dh u silu'(g)), du = dtype(dh silu(g)), h = dtype(silu(g) u)
//   dx      = [dg | du] [gate_e; up_e]     -> grad_dispatched (dtype)
//   dgate_e = dg^T x,  dup_e = du^T x,  ddown_e = dy^T h     (FP32, sums over the expert's rows)
// silu'(z) = s (1 + z (1 - s)), s = 1 / (1 + e^-z).
//
// Two MFMA kernels serve the five products, C[m, n] = sum_k A(m, k) B(n, k) on BM x BN tiles
// (256 x 256, eight wavefronts of 128 x 64), K staged 128 bytes per row (v_mfma_f32_32x32x16 for
// BF16/F16, 32x32x2f32 for FP32): for 16-bit types the DMA form below (operands copied straight
// into LDS; fragments of an operand that is not K-major read with the LDS transpose read), and
// for FP32 (or operands beyond 2 GiB) the register-staged kernel described next.  An operand is either "K-major" (k contiguous: staged as
// 16-byte pieces) or "X-major" (its row/column index contiguous): a thread then loads 4 rows of k
// by CE consecutive x (CE = elements per 16 bytes), transposes them in registers and stores CE
// runs of 4 k values into the [x][k] LDS tile.  The operand tiles go through registers (two
// sets): during step k, step k+1 (loaded during step k-2) is written to the other LDS stage
// between the first MFMA groups, and the loads of step k+3 go out into the registers it freed.
// Two operand sources may be stacked along the operand's outer index (gate over up).
// Grouping: ROWS tiles the expert's rows along M (a device-side plan of m-tiles per expert);
// KROWS uses the expert's rows as the contraction axis, every (expert, m, n) tile (an expert
// without rows gets zeros).  In the DMA form the ROWS products with a plain epilogue split the
// tiles of a last, partial round along K (see BSplit); split_reduce finishes them.
#include <atomic>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace rudnn {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int ROWB = 128;  // bytes of K per staged row and step

// Block tile BM x BN, WM x WN wavefronts (each (BM / WM) x (BN / WN), whole 32 x 32 MFMA blocks).
template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, THREADS = 64 * WM_ * WN_;
    static constexpr int LDS_BYTES = 2 * (BM_ + BN_) * ROWB;  // two stages
};

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

// 128-byte staged rows: chunk c (16 bytes) of row r at slot c ^ swz(r); the MFMA operand reads
// (one chunk from each of 32 consecutive rows) then spread over all LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 4 rows of 8 16-bit elements -> 8 runs of 4: out[x] holds element x of in[0..4).
__device__ __forceinline__ void transpose_quad(const uint4 (&in)[4], uint2 (&out)[8]) {
#pragma unroll
    for (int x = 0; x < 8; ++x) {
        uint32_t d[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t a = reinterpret_cast<const uint32_t*>(&in[2 * j])[x >> 1];
            const uint32_t b = reinterpret_cast<const uint32_t*>(&in[2 * j + 1])[x >> 1];
            d[j] = (x & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        out[x] = make_uint2(d[0], d[1]);
    }
}
// 4 x 4 transpose of 32-bit elements: out[x] holds element x of in[0..4).
__device__ __forceinline__ void transpose_block(const uint4 (&in)[4], uint4 (&out)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = reinterpret_cast<const uint32_t*>(&in[j])[x];
        out[x] = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

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

// Four adjacent outputs rounded to T, one store (8 bytes for 16-bit T, 16 for FP32); p is
// aligned to four elements (N and the column are multiples of 4).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    } else {
        T v[4] = {from_f32<T>(a), from_f32<T>(b), from_f32<T>(c), from_f32<T>(d)};
        uint2 q;
        __builtin_memcpy(&q, v, 8);
        *reinterpret_cast<uint2*>(p) = q;
    }
}
enum { ROWS = 0, KROWS = 1 };

struct Plan {
    const int32_t* row_begin;  // [E]
    const int32_t* row_count;  // [E]
    const int32_t* mt_begin;   // [E + 1]
};

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int rows, int BM,
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

// Tail split of the products over the dispatched rows: tiles run one per CU in rounds; when the
// tile count leaves a last, partial round of R tiles, each of those is cut along K into S
// segments (S = CUs / R, at most SPLIT_SLOTS / R, each at least SPLIT_MIN_STEPS K steps), so the
// last round fills the machine; the grid has SPLIT_SLOTS units beyond the tiles for them.
constexpr int SPLIT_SLOTS = 256, SPLIT_MIN_STEPS = 8;
struct BSplit {
    int64_t full;  // tiles run whole (they come first)
    int R, S;      // split tiles, segments each (R = 0, S = 1: no split)
};
__device__ __forceinline__ BSplit bsplit_plan(int64_t tiles, int KT, int cus) {
    BSplit sp;
    int64_t R = tiles >= cus ? tiles % cus : tiles;
    int S = R > 0 ? (int)min((int64_t)cus / R, (int64_t)SPLIT_SLOTS / R) : 1;
    S = min(S, KT / SPLIT_MIN_STEPS);
    if (S < 2) S = 1, R = 0;
    sp.full = tiles - R;
    sp.R = (int)R;
    sp.S = S;
    return sp;
}

// Tile L of a product: ROWS tiles the experts' dispatched rows (m-tiles from the
// device-side plan) by N; KROWS takes every (expert, m-tile, n-tile) with the expert's rows as K.
// False if the workgroup has no tile.
struct TileSel {
    int e, m0, n0, mlim, nlim, kb, kn;  // expert, tile origin, valid rows and columns, K origin and length
    int64_t row0;                       // ROWS: first dispatched row of the tile
};
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool pick_tile(const Plan& plan, const int32_t* __restrict__ offsets, int rows, int M,
                                          int N, int K, int E, int NT, int MT, int64_t L, TileSel& t) {
    t.row0 = 0;
    if (MODE == ROWS) {
        const int64_t Mt = L / NT;
        if (Mt >= plan.mt_begin[E]) return false;
        int lo = 0, hi = E - 1;  // largest e with mt_begin[e] <= Mt
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (plan.mt_begin[mid] <= Mt)
                lo = mid;
            else
                hi = mid - 1;
        }
        t.e = lo;
        const int mt = (int)(Mt - plan.mt_begin[t.e]);
        t.n0 = (int)(L % NT) * BN;
        t.m0 = 0;
        t.row0 = plan.row_begin[t.e] + (int64_t)mt * BM;
        t.mlim = min(BM, plan.row_count[t.e] - mt * BM);
        t.kb = 0, t.kn = K;
    } else {
        t.e = (int)(L / ((int64_t)MT * NT));
        const int r = (int)(L % ((int64_t)MT * NT));
        t.m0 = (r / NT) * BM, t.n0 = (r % NT) * BN;
        t.mlim = min(BM, M - t.m0);
        const int a = min(max(offsets[t.e], 0), rows), b = min(max(offsets[t.e + 1], 0), rows);
        t.kb = a, t.kn = max(b - a, 0);
    }
    t.nlim = min(BN, N - t.n0);
    return true;
}

// The products' epilogue, shared by both GEMM kernels.  The accumulator blocks hold C^T (the
// operands went in B fragment first) in ROWS mode and C in KROWS mode; see the two branches.
template <typename T, int MODE, int EPI, int FM, int FN, int TM, int TN>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[FM][FN], int wm, int wn, int lane, int mlim, int nlim,
                                         int e, int M, int m0, int n0, int64_t row0, int N, const Epi& ep) {
    const int fr = lane & 31, fh = lane >> 5;
    if constexpr (MODE == KROWS) {
        // Weight gradients (FP32): the operands went in token fragment first, so lane l holds
        // column l % 32 and rows 8 (v / 4) + 4 fh + v % 4 of each block; a store instruction writes
        // two whole 128-byte row pieces.
        static_assert(EPI == EPI_F32, "weight gradients are FP32");
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int nl = wn * TN + j * 32 + fr;
                if (nl >= nlim) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int ml = wm * TM + i * 32 + 8 * (v / 4) + 4 * fh + v % 4;
                    if (ml < mlim)
                        reinterpret_cast<float*>(ep.c)[((int64_t)e * M + m0 + ml) * ep.ldc + n0 + nl] = acc[i][j][v];
                }
            }
        return;
    }
    // ---- epilogue: lane holds row m = fr of each 32-row block, columns 8 (v / 4) + 4 fh + v % 4 ----
    if constexpr (EPI == EPI_SWIGLU) {
        // dh -> dg, du, h (N = I).  Per 32-row block, all of the lane's g | u loads go out before any
        // store (the stores could alias the loads, so the compiler would otherwise wait for each
        // run's loads in turn: one memory round trip per four outputs).
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int ml = wm * TM + i * 32 + fr;
            if (ml >= mlim) continue;
            const int64_t crow = MODE == ROWS ? row0 + ml : (int64_t)e * M + m0 + ml;
            const float* gr = ep.gu + crow * 2 * (int64_t)N + n0;
            float4 g4[FN][4], u4[FN][4];
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * TN + j * 32 + 8 * q + 4 * fh;
                    if (nl < nlim) {  // N is a multiple of 4: a run of 4 is wholly in or out
                        g4[j][q] = *reinterpret_cast<const float4*>(gr + nl);
                        u4[j][q] = *reinterpret_cast<const float4*>(gr + N + nl);
                    }
                }
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * TN + j * 32 + 8 * q + 4 * fh;
                    if (nl >= nlim) continue;
                    const int n = n0 + nl;
                    const float gv[4] = {g4[j][q].x, g4[j][q].y, g4[j][q].z, g4[j][q].w};
                    const float uv[4] = {u4[j][q].x, u4[j][q].y, u4[j][q].z, u4[j][q].w};
                    float dgv[4], duv[4], hv[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float dh = acc[i][j][4 * q + t], g = gv[t], u = uv[t];
                        // hardware exp and reciprocal, as the forward's silu (a few FP32 ulps)
                        const float s = __builtin_amdgcn_rcpf(1.f + __expf(-g));
                        dgv[t] = dh * u * (s * (1.f + g * (1.f - s)));
                        duv[t] = dh * (g * s);
                        hv[t] = g * s * u;
                    }
                    T* dg = reinterpret_cast<T*>(ep.dgu) + crow * 2 * (int64_t)N + n;
                    store4<T>(dg, dgv[0], dgv[1], dgv[2], dgv[3]);
                    store4<T>(dg + N, duv[0], duv[1], duv[2], duv[3]);
                    store4<T>(reinterpret_cast<T*>(ep.h) + crow * (int64_t)N + n, hv[0], hv[1], hv[2], hv[3]);
                }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int ml = wm * TM + i * 32 + fr;
        if (ml >= mlim) continue;
        const int64_t crow = MODE == ROWS ? row0 + ml : (int64_t)e * M + m0 + ml;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * TN + j * 32 + 8 * q + 4 * fh;
                if (nl >= nlim) continue;  // N is a multiple of 4: a run of 4 is wholly in or out
                const int n = n0 + nl;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                            v3 = acc[i][j][4 * q + 3];
                if (EPI == EPI_F32) {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.c) + crow * ep.ldc + n) =
                        make_float4(v0, v1, v2, v3);
                } else {
                    store4<T>(reinterpret_cast<T*>(ep.c) + crow * ep.ldc + n, v0, v1, v2, v3);
                }
            }
    }
}

// C = A B^T on BM x BN tiles; see the file comment.
template <typename T, typename C, int MODE, int EPI, bool AK, bool BK>
__global__ __launch_bounds__(C::THREADS) void gemm_kernel(Opnd A, Opnd B, int M, int N, int K, int E, Plan plan,
                                                          const int32_t* __restrict__ offsets, int rows, int NT,
                                                          int MT, Epi ep) {
    constexpr int BM = C::BM, BN = C::BN, THREADS = C::THREADS;
    constexpr int TM = BM / C::WM, TN = BN / C::WN;  // wavefront tile
    constexpr int FM = TM / 32, FN = TN / 32;        // 32 x 32 MFMA blocks per wavefront
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront tiles are whole MFMA blocks");
    constexpr int CE = 16 / (int)sizeof(T);     // elements per 16-byte chunk
    constexpr int BKE = ROWB / (int)sizeof(T);  // K elements per step
    constexpr int NCH = ROWB / 16;              // chunks per staged row
    constexpr int KQA = BM * NCH / THREADS, KQB = BN * NCH / THREADS;  // K-major pieces per thread
    static_assert(BM * NCH % THREADS == 0 && BN * NCH % THREADS == 0, "K-major pieces split evenly");
    // X-major pieces: 4 rows of k x CE consecutive x
    constexpr int NKQ = BKE / 4;                                     // k quads per step
    constexpr int NPA = NKQ * (BM / CE), NPB = NKQ * (BN / CE);      // pieces per operand tile
    constexpr int XQA = (NPA + THREADS - 1) / THREADS, XQB = (NPB + THREADS - 1) / THREADS;  // per thread
    static_assert(NKQ % 8 == 0 && (BM / CE) % 8 == 0 && (BN / CE) % 8 == 0, "pieces come in 8 x 8 groups");
    typedef typename Mma<T>::frag frag;
    extern __shared__ __align__(1024) unsigned char lds[];

    // ---- which tile ----
    TileSel ts;
    if (!pick_tile<MODE, BM, BN>(plan, offsets, rows, M, N, K, E, NT, MT, blockIdx.x, ts)) return;
    const int e = ts.e, m0 = ts.m0, n0 = ts.n0, mlim = ts.mlim, nlim = ts.nlim, kb = ts.kb, kn = ts.kn;
    const int64_t row0 = ts.row0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;

    // The outer index of an operand's tile row x (A: a dispatched row or m, B: n).
    auto x_outer = [&](bool is_a, int x) -> int64_t {
        return is_a ? (MODE == ROWS ? row0 + x : (int64_t)(m0 + x)) : (int64_t)(n0 + x);
    };
    // K-major staging: piece c -> row x = c / NCH, chunk c % NCH.
    auto load_k = [&](const Opnd& o, bool is_a, int xlim, int k0, auto& r) __attribute__((always_inline)) {
        constexpr int NQ = sizeof(r) / sizeof(uint4);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int c = tid + q * THREADS, x = c / NCH, k = k0 + (c % NCH) * CE;
            r[q] = make_uint4(0, 0, 0, 0);
            if (x < xlim && k < kn)
                r[q] = *reinterpret_cast<const uint4*>(
                    opnd_row<T>(o, MODE == ROWS && is_a ? 0 : e, x_outer(is_a, x)) + kb + k);
        }
    };
    auto store_k = [&](unsigned char* st, const auto& r) __attribute__((always_inline)) {
        constexpr int NQ = sizeof(r) / sizeof(uint4);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int c = tid + q * THREADS, x = c / NCH, kc = c % NCH;
            *reinterpret_cast<uint4*>(st + x * ROWB + ((kc ^ swz(x)) * 16)) = r[q];
        }
    };
    // X-major staging.  Piece p covers k rows 4 kq .. 4 kq + 3 of the step and x group xg (CE
    // consecutive x): lanes take x groups fastest in runs of 8, then 8 k quads, so one load
    // instruction of a wavefront reads eight full 128-byte lines, and each store step writes 4 k
    // values (8 bytes; 16 for FP32) to rows x whose swizzled positions cover every LDS bank.
    // Thread tid takes pieces tid + j THREADS.
    auto piece = [&](int p, int& kq, int& xg) __attribute__((always_inline)) {
        constexpr int KH = NKQ / 8;
        const int rest = p >> 6;
        kq = ((p >> 3) & 7) + 8 * (rest % KH);
        xg = (p & 7) + 8 * (rest / KH);
    };
    auto load_x = [&](const Opnd& o, bool is_a, int xlim, int k0, auto& r) __attribute__((always_inline)) {
        constexpr int NQ = sizeof(r) / sizeof(r[0]);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int p = tid + j * THREADS;
            if ((is_a ? NPA : NPB) % THREADS != 0 && p >= (is_a ? NPA : NPB)) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) r[j][i] = make_uint4(0, 0, 0, 0);
            int kq, xg;
            piece(p, kq, xg);
            const int x = xg * CE;
            if (x >= xlim) continue;
            const int64_t xo = x_outer(is_a, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = k0 + kq * 4 + i;
                if (k < kn)
                    r[j][i] = *reinterpret_cast<const uint4*>(opnd_row<T>(o, MODE == KROWS ? 0 : e, kb + k) + xo);
            }
        }
    };
    auto store_x = [&](unsigned char* st, bool is_a, const auto& r) __attribute__((always_inline)) {
        constexpr int NQ = sizeof(r) / sizeof(r[0]);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int p = tid + j * THREADS;
            if ((is_a ? NPA : NPB) % THREADS != 0 && p >= (is_a ? NPA : NPB)) continue;
            int kq, xg;
            piece(p, kq, xg);
            const int x0 = xg * CE;
            if constexpr (CE == 8) {
                uint2 t[8];
                transpose_quad(r[j], t);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int x = x0 + i;
                    *reinterpret_cast<uint2*>(st + x * ROWB + (((kq >> 1) ^ swz(x)) * 16) + (kq & 1) * 8) = t[i];
                }
            } else {
                uint4 t[4];
                transpose_block(r[j], t);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int x = x0 + i;
                    *reinterpret_cast<uint4*>(st + x * ROWB + ((kq ^ swz(x)) * 16)) = t[i];
                }
            }
        }
    };

    // One step's operand pieces in registers; two sets, so that the loads of a step are issued
    // two steps before they are written to LDS.
    struct Regs {
        uint4 ka[AK ? KQA : 1], kb[BK ? KQB : 1];
        uint4 xa[AK ? 1 : XQA][4], xb[BK ? 1 : XQB][4];
    };
    auto load_a = [&](int kt, Regs& r) __attribute__((always_inline)) {
        if constexpr (AK)
            load_k(A, true, mlim, kt * BKE, r.ka);
        else
            load_x(A, true, mlim, kt * BKE, r.xa);
    };
    auto load_b = [&](int kt, Regs& r) __attribute__((always_inline)) {
        if constexpr (BK)
            load_k(B, false, nlim, kt * BKE, r.kb);
        else
            load_x(B, false, nlim, kt * BKE, r.xb);
    };
    auto store_a = [&](int kt, const Regs& r) __attribute__((always_inline)) {
        unsigned char* st = lds + (kt & 1) * (BM + BN) * ROWB;
        if constexpr (AK)
            store_k(st, r.ka);
        else
            store_x(st, true, r.xa);
    };
    auto store_b = [&](int kt, const Regs& r) __attribute__((always_inline)) {
        unsigned char* st = lds + (kt & 1) * (BM + BN) * ROWB + BM * ROWB;
        if constexpr (BK)
            store_k(st, r.kb);
        else
            store_x(st, false, r.xb);
    };
    auto load_step = [&](int kt, Regs& r) __attribute__((always_inline)) {
        load_a(kt, r);
        load_b(kt, r);
    };
    auto store_step = [&](int kt, const Regs& r) __attribute__((always_inline)) {
        store_a(kt, r);
        store_b(kt, r);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int fr = lane & 31, fh = lane >> 5;
    const int KT = (kn + BKE - 1) / BKE;
    Regs even, odd;  // steps 0, 2, 4, ... and 1, 3, 5, ...
    if (KT > 0) {
        load_step(0, even);
        store_step(0, even);
    }
    if (KT > 1) load_step(1, odd);
    if (KT > 2) load_step(2, even);
    __syncthreads();
    // Step kt: MFMAs from LDS stage kt & 1; step kt + 1 (in `next`, loaded two steps ago) goes to
    // the other stage (last read in step kt - 1) between the MFMA groups -- A after the first, B
    // after the second -- each followed by the loads of step kt + 3 into the registers it freed,
    // so that the staging work overlaps the matrix cores instead of following them.
    auto step = [&](int kt, Regs& next) __attribute__((always_inline)) {
        const unsigned char* st = lds + (kt & 1) * (BM + BN) * ROWB;
        const unsigned char* sa = st + (wm * TM + fr) * ROWB;
        const unsigned char* sb = st + BM * ROWB + (wn * TN + fr) * ROWB;
#pragma unroll
        for (int ks = 0; ks < NCH / 2; ++ks) {
            const int off = ((ks * 2 + fh) ^ swz(fr)) * 16;
            frag fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) fa[i] = *reinterpret_cast<const frag*>(sa + i * 32 * ROWB + off);
#pragma unroll
            for (int j = 0; j < FN; ++j) fb[j] = *reinterpret_cast<const frag*>(sb + j * 32 * ROWB + off);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = MODE == ROWS ? Mma<T>::run(fb[j], fa[i], acc[i][j]) : Mma<T>::run(fa[i], fb[j], acc[i][j]);
            if (ks == 0) {
                if (kt + 1 < KT) store_a(kt + 1, next);
                if (kt + 3 < KT) load_a(kt + 3, next);
            } else if (ks == 1) {
                if (kt + 1 < KT) store_b(kt + 1, next);
                if (kt + 3 < KT) load_b(kt + 3, next);
            }
        }
        __syncthreads();
    };
    for (int kt = 0; kt < KT; kt += 2) {
        step(kt, odd);
        if (kt + 1 < KT) step(kt + 1, even);
    }

    epilogue<T, MODE, EPI, FM, FN, TM, TN>(acc, wm, wn, lane, mlim, nlim, e, M, m0, n0, row0, N, ep);
}


// ---------------------------------------------------------------------------------------
// DMA form (16-bit types).  Both operand tiles go straight from global memory into LDS with
// buffer_load_dwordx4 ... lds (no register staging), K 64 elements per step, two stages:
//   K-major tile (k contiguous in memory): [x][k], 256 rows of 128 bytes, chunk c of row x at
//   slot c ^ swz(x) -- the forward GEMM's layout; an MFMA fragment is one 16-byte LDS read.
//   X-major tile (x contiguous in memory): kept as it lies, [k][x], 64 k rows of 512 bytes (256
//   x values), chunk c (8 x values) of row k at slot c ^ sxm(k).  Its MFMA fragments are read
//   with the LDS transpose read ds_read_b64_tr_b16: in each group of 16 lanes, lane i reads 4
//   16-bit values at its own address (row i of a 16 x 4 block) and lane j receives column
//   j % 4 of rows j / 4, j / 4 + 4, j / 4 + 8, j / 4 + 12 (measured on gfx950).  Lane i naming
//   (k0 + i / 4, x0 + 4 (i % 4)) therefore gives lane j the values (k0 .. k0 + 3, x0 + j): two
//   such reads make the 8 consecutive k of one x that an MFMA operand lane holds.
// One wavefront copy moves 1 KiB: 8 rows of a K-major tile or 2 k rows of an X-major one; a
// step is 32 copies per operand, dealt to the wavefronts round-robin.  A copy reads rows of one
// operand part only (the part boundary is a multiple of 8 rows), so its buffer is uniform.
// Rows or x past the tile's valid range re-read its last valid row or chunk (their outputs are
// never stored); k past the end is zero-filled.
constexpr int XROWB = 512;  // bytes of one staged X-major k row

// A transpose read touches, per group of 16 lanes, 4 consecutive k rows and 4 consecutive
// chunks, the wavefront's other groups the next 4 chunks or the k rows 8 further on; with this
// swizzle those 32 pieces sit in 32 different slots.
__device__ __forceinline__ int sxm(int k) { return 4 * (k & 3) + 16 * ((k >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-byte LDS-direct copy per lane: the wavefront's 64 pieces land at dst + 16 lane; base and
// dst are wavefront-uniform.  Written as inline asm (buffer_load_dwordx4 ... lds, M0 = the LDS
// address) rather than the builtin: after a builtin LDS-direct copy the compiler treats every
// later LDS transpose read as possibly reading the copy's destination and waits for all of the
// wavefront's outstanding copies (vmcnt 0) before it, which put the next step's copy latency
// inside every step (Mixtral-shaped layer: dinput 2.49 -> 2.23 ms, each weight gradient 1.24 ->
// 1.17 ms, dh 1.61 -> 1.56 ms without those waits).  Nothing else in these kernels uses M0.  The
// copies of a step always go to the stage that no wavefront reads during it, and the explicit
// vmcnt wait plus the barrier at the top of the next step order them before their reads.  (A
// __device__ function, not a lambda: the buffer intrinsics exist only in device code.)
__device__ __forceinline__ void dma16(const void* base, uint32_t off, unsigned char* dst) {
    constexpr int GFX9_RSRC_WORD3 = 0x00020000;  // 32-bit data format, no swizzle
    // the base is wavefront-uniform: read it into SGPRs (as unsigned words: readfirstlane returns
    // int, and a sign-extended low word would corrupt the high word)
    const uint64_t bp = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bp);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bp >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo), (short)0, 0x7fffffff, GFX9_RSRC_WORD3);
    const uint32_t la = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(la), "v"(off), "s"(rs)
                 : "memory", "m0");
}

typedef short v4s __attribute__((ext_vector_type(4)));
// The LDS transpose read (ds_read_b64_tr_b16) of the 8 bytes at p; see the DMA form's comment.
__device__ __forceinline__ v4s read_tr(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
}

template <typename T, typename C, int MODE, int EPI, bool AK, bool BK, bool SPLIT>
__global__ __launch_bounds__(C::THREADS) void gemm_dma_kernel(Opnd A, Opnd B, int M, int N, int K, int E, Plan plan,
                                                              const int32_t* __restrict__ offsets, int rows, int NT,
                                                              int MT, Epi ep, int cus, float* __restrict__ partials) {
    static_assert(sizeof(T) == 2, "the DMA form stages 16-bit operands");
    constexpr int BM = C::BM, BN = C::BN, THREADS = C::THREADS, NWAVES = THREADS / 64;
    constexpr int TM = BM / C::WM, TN = BN / C::WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int BKE = ROWB / 2;              // K elements per step (64)
    constexpr int TILE = 256 * ROWB;           // bytes of one operand tile per stage
    // Copying wavefronts: only the first half (one per SIMD: wavefronts w and w + 4 share one), all at
    // the first MFMA substep, so each SIMD's other wavefront keeps its matrix core busy while the
    // copies queue for issue (Mixtral-shaped layer, against every wavefront copying over the first
    // two substeps: dinput 3.02 -> 2.76 ms, each weight gradient 1.41 -> 1.25 ms, dh 1.62 -> 1.61).
    constexpr int CW = NWAVES / 2;
    constexpr int SLOTS = 64 / CW;             // copies per copying wavefront per step (32 per operand)
    constexpr int SPREAD = 1;                  // MFMA substeps the copies go out under
    static_assert(BM == 256 && BN == 256 && 64 % CW == 0, "operand tiles of 256 x 64, whole copies per wave");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront tiles are whole MFMA blocks");
    typedef typename Mma<T>::frag frag;
    extern __shared__ __align__(1024) unsigned char lds[];

    TileSel ts;
    // Tail split (SPLIT, ROWS mode): the tiles of a last, partial round of CU-count tiles are cut
    // along K into S segments whose FP32 partial sums split_reduce adds up (see BSplit).
    int64_t L = blockIdx.x;
    int ks0 = 0, ks1 = -1, slot = -1;  // K steps [ks0, ks1) of this unit (ks1 < 0: the whole K)
    if constexpr (SPLIT) {
        static_assert(MODE == ROWS, "only products over the dispatched rows are split");
        const int KTall = (K + BKE - 1) / BKE;
        const BSplit sp = bsplit_plan((int64_t)plan.mt_begin[E] * NT, KTall, cus);
        if (L >= sp.full) {
            const int64_t v = L - sp.full;
            if (v >= (int64_t)sp.R * sp.S) return;
            const int seg = (int)(v % sp.S);
            L = sp.full + v / sp.S;
            ks0 = (int)((int64_t)seg * KTall / sp.S), ks1 = (int)((int64_t)(seg + 1) * KTall / sp.S);
            slot = (int)v;
        }
    }
    // The tile's work.  The products over the rows with a plain epilogue (dinput, the recomputed
    // g | u; the ones with the tail split) run it inside a one-pass loop: in that form the compiler
    // keeps the copy addresses of the K loop in scalar registers (per step about 80 vector
    // instructions in a copying wavefront instead of 225, and no readfirstlane per copy; 243 -> 214
    // VGPRs), and dinput takes 1.95-1.97 ms instead of 2.25-2.29 on the Mixtral-shaped layer.  The
    // others keep the straight form (the wrapper made dh slower).
    auto body = [&]() __attribute__((always_inline)) {
        if (!pick_tile<MODE, BM, BN>(plan, offsets, rows, M, N, K, E, NT, MT, L, ts)) return;
        const int e = ts.e, m0 = ts.m0, n0 = ts.n0, mlim = ts.mlim, nlim = ts.nlim, kb = ts.kb, kn = ts.kn;
        const int64_t row0 = ts.row0;
        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = wave / C::WN, wn = wave % C::WN;

        // The first element of operand part `part` of expert ee (copy offsets are bytes from it).
        auto part_base = [&](const Opnd& o, int part, int ee) __attribute__((always_inline)) {
            return (void*)(reinterpret_cast<const T*>(part ? o.p1 : o.p0) + (int64_t)ee * o.estride);
        };
        // Copy q of this wavefront for step kt of operand `is_a` into stage st.
        auto copy = [&](const Opnd& o, bool is_a, bool kmajor, int xlim, unsigned char* st, int gi, int kt)
            __attribute__((always_inline)) {
            unsigned char* dst = st + gi * 1024;
            const int k0 = kt * BKE;
            if (kmajor) {
                // rows x = 8 gi + lane / 8 of the tile, chunk slot lane % 8
                const int x = 8 * gi + lane / 8, xc = min(x, xlim - 1);
                const int xf = min(8 * gi, xlim - 1);  // the copy's first row: its part
                const int64_t of = is_a ? (MODE == ROWS ? row0 + xf : (int64_t)(m0 + xf)) : (int64_t)(n0 + xf);
                const int part = of >= o.split;
                const int64_t oc = is_a ? (MODE == ROWS ? row0 + xc : (int64_t)(m0 + xc)) : (int64_t)(n0 + xc);
                const int kk = k0 + ((lane & 7) ^ swz(x)) * 8;
                if (kk < kn) {
                    const uint32_t off = (uint32_t)((oc - (part ? o.split : 0)) * o.ld + kb + kk) * 2u;
                    dma16(part_base(o, part, MODE == ROWS && is_a ? 0 : e), off, dst);
                } else {
                    *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
                }
            } else {
                // k rows 2 gi + lane / 32 of the step, chunk slot lane % 32
                const int kr = 2 * gi + (lane >> 5), k = k0 + kr;
                const int kf = min(k0 + 2 * gi, max(kn - 1, 0));  // the copy's first row: its part
                const int part = (kb + kf) >= o.split;
                const int c = min((lane & 31) ^ sxm(kr), (xlim - 1) >> 3);
                const int64_t xo = is_a ? (int64_t)(m0 + 8 * c) : (int64_t)(n0 + 8 * c);
                if (k < kn) {
                    const uint32_t off = (uint32_t)((kb + k - (part ? o.split : 0)) * o.ld + xo) * 2u;
                    dma16(part_base(o, part, MODE == KROWS ? 0 : e), off, dst);
                } else {
                    *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
                }
            }
        };

        f32x16 acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

        // Per-lane fragment offsets.  K-major: row fr of a 32-row block, chunk (2 ks + fh) ^ swz(fr).
        // X-major: the transpose read of lane l (group g = l / 16, i = l % 16) for 32-x block xb and
        // half r of substep ks: k = 16 ks + 8 (g / 2) + 4 r + i / 4, x = 32 xb + 16 (g % 2) + 4 (i % 4),
        // at byte k * 512 + ((x / 8) ^ sxm(k)) * 16 + (x % 8) * 2 = tr_base + (16 ks + 4 r) * 512 +
        // ((xb ^ tr_sw) << 6).
        const int fr = lane & 31, fh = lane >> 5;
        const int tg = lane >> 4, ti = lane & 15;
        const int tr_base = (8 * (tg >> 1) + (ti >> 2)) * XROWB + (2 * (tg & 1) + ((ti & 3) >> 1)) * 16 + 8 * (ti & 1);
        const int tr_sw = (ti >> 2) + 4 * (tg >> 1);
        auto frag_k = [&](const unsigned char* t, int row, int ks) __attribute__((always_inline)) {
            return *reinterpret_cast<const frag*>(t + (row + fr) * ROWB + (((ks * 2 + fh) ^ swz(fr)) * 16));
        };
        auto frag_x = [&](const unsigned char* t, int xb, int ks) __attribute__((always_inline)) {
            const unsigned char* p = t + tr_base + ks * 16 * XROWB + ((xb ^ tr_sw) << 6);
            const v4s lo = read_tr(p), hi = read_tr(p + 4 * XROWB);
            frag f;
            __builtin_memcpy(&f, &lo, 8);
            __builtin_memcpy(reinterpret_cast<unsigned char*>(&f) + 8, &hi, 8);
            return f;
        };

        // Step kt: the copies of step kt + 1 go out over the first SPREAD MFMA substeps (into the stage
        // read in step kt - 1), and the fragments of substep ks + 1 are read while the MFMAs of
        // substep ks run.
        auto issue_part = [&](int kt, int q0, int q1) __attribute__((always_inline)) {
            unsigned char* st = lds + (kt & 1) * 2 * TILE;
            if (wave >= CW) return;
#pragma unroll
            for (int q = q0; q < q1; ++q) {
                const int g = wave + q * CW;  // 0..63: A copies, then B copies
                if (g < 32)
                    copy(A, true, AK, mlim, st, g, kt);
                else
                    copy(B, false, BK, nlim, st + TILE, g - 32, kt);
            }
        };
        const int KT = ks1 >= 0 ? ks1 : (kn + BKE - 1) / BKE;
        if (ks0 < KT) issue_part(ks0, 0, SLOTS);
        for (int kt = ks0; kt < KT; ++kt) {
            wait_vmcnt<0>();  // this wavefront's copies of step kt have landed
            __syncthreads();  // everyone's have; everyone is done with the other stage (step kt - 1)
            const unsigned char* ta = lds + (kt & 1) * 2 * TILE;
            const unsigned char* tb = ta + TILE;
            frag fa[2][FM], fb[2][FN];
            auto fetch = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    fa[buf][i] = AK ? frag_k(ta, wm * TM + i * 32, ks) : frag_x(ta, (wm * TM) / 32 + i, ks);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[buf][j] = BK ? frag_k(tb, wn * TN + j * 32, ks) : frag_x(tb, (wn * TN) / 32 + j, ks);
            };
            fetch(0, 0);
#pragma unroll
            for (int ks = 0; ks < BKE / 16; ++ks) {
                if (kt + 1 < KT && ks < SPREAD) issue_part(kt + 1, ks * SLOTS / SPREAD, (ks + 1) * SLOTS / SPREAD);
                if (ks + 1 < BKE / 16) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = MODE == ROWS ? Mma<T>::run(fb[ks & 1][j], fa[ks & 1][i], acc[i][j])
                                                 : Mma<T>::run(fa[ks & 1][i], fb[ks & 1][j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (SPLIT && slot >= 0) {  // a segment: FP32 partial sums of the tile, [slot][BM][BN]
            const Epi pe{partials + (int64_t)slot * BM * BN, BN, nullptr, nullptr, nullptr};
            epilogue<T, MODE, EPI_F32, FM, FN, TM, TN>(acc, wm, wn, lane, mlim, nlim, e, M, m0, 0, 0, N, pe);
            return;
        }
        epilogue<T, MODE, EPI, FM, FN, TM, TN>(acc, wm, wn, lane, mlim, nlim, e, M, m0, n0, row0, N, ep);
    };
    if constexpr (MODE == ROWS && EPI != EPI_SWIGLU) {
#pragma unroll 1
        for (int pass = 0; pass < 1; ++pass) body();
    } else {
        body();
    }
}

// Adds the S partial sums of every split tile in segment order (deterministic) and stores the
// product in the dtype (EPI_DT) or FP32: a thread takes four adjacent columns of one row.
template <typename T, int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void split_reduce(const float* __restrict__ partials, int K, int N, int E, Plan plan,
                                                    const int32_t* __restrict__ offsets, int rows, int NT, int cus,
                                                    Epi ep) {
    static_assert(EPI == EPI_DT || EPI == EPI_F32, "plain epilogues only");
    constexpr int BKE = ROWB / (int)sizeof(T);
    const int KTall = (K + BKE - 1) / BKE;
    const BSplit sp = bsplit_plan((int64_t)plan.mt_begin[E] * NT, KTall, cus);
    constexpr int Q = BN / 4;  // column quads per row
    const int64_t items = (int64_t)sp.R * BM * Q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < items; i += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / (BM * Q)), row = (int)(i / Q % BM), col = (int)(i % Q) * 4;
        TileSel t;
        pick_tile<ROWS, BM, BN>(plan, offsets, rows, 0, N, K, E, NT, 0, sp.full + r, t);
        if (row >= t.mlim || col >= t.nlim) continue;
        const float* p = partials + ((int64_t)r * sp.S * BM + row) * BN + col;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sg = 0; sg < sp.S; ++sg) {
            const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)sg * BM * BN);
            a.x += v.x, a.y += v.y, a.z += v.z, a.w += v.w;
        }
        const int64_t crow = t.row0 + row;
        if (EPI == EPI_F32)
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(ep.c) + crow * ep.ldc + t.n0 + col) = a;
        else
            store4<T>(reinterpret_cast<T*>(ep.c) + crow * ep.ldc + t.n0 + col, a.x, a.y, a.z, a.w);
    }
}

}  // namespace bwd

// ---- host side ----

// Workspace: [dg | du] [rows, 2I] dtype, h [rows, I] dtype, the plan (3E + 1 ints), (without a
// cache) the recomputed pre-activations [g | u] [rows, 2I] FP32, then (16-bit types) the tail
// split's partial-sum slots, SPLIT_SLOTS x 256 x 256 FP32.
static size_t bwd_split_bytes(rudnn_moe_dtype dt) {
    return dt == RUDNN_MOE_F32 ? 0 : align_up((size_t)bwd::SPLIT_SLOTS * 256 * 256 * sizeof(float));
}

size_t experts_backward_workspace_bytes(int64_t E, int64_t I, rudnn_moe_dtype dt, int64_t rows, bool cached) {
    const size_t es = dtype_size(dt);
    return align_up((size_t)rows * 2 * I * es) + align_up((size_t)rows * I * es) +
           align_up(sizeof(int32_t) * (size_t)(3 * E + 1)) + (cached ? 0 : align_up((size_t)rows * 2 * I * 4)) +
           bwd_split_bytes(dt);
}

namespace {

#ifndef RUDNN_BWD_DMA
#define RUDNN_BWD_DMA 1
#endif
constexpr bool bwd_dma_enabled() { return RUDNN_BWD_DMA != 0; }

// Tiles: products over the dispatched rows (ROWS) and the weight gradients (KROWS).
#ifndef RUDNN_BWD_ROWS_TILE
#define RUDNN_BWD_ROWS_TILE 256, 256, 2, 4
#endif
#ifndef RUDNN_BWD_KROWS_TILE
#define RUDNN_BWD_KROWS_TILE 256, 256, 2, 4
#endif
typedef bwd::Cfg<RUDNN_BWD_ROWS_TILE> RowsCfg;
typedef bwd::Cfg<RUDNN_BWD_KROWS_TILE> KRowsCfg;

// Compute units of the current device (one round of tiles), cached per device.
static int bwd_device_cus() {
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// C = A B^T for one product; a_rows / b_rows: rows of each part of A / B in memory (their byte
// extents decide whether the 16-bit DMA form's 32-bit buffer offsets reach every element).
// partials: the tail split's FP32 slots (products over the rows with a plain epilogue, DMA form).
template <typename T, int MODE, int EPI, bool AK, bool BK>
void gemm(bwd::Opnd A, bwd::Opnd B, int M, int N, int K, int E, bwd::Plan plan, const int32_t* offsets, int rows,
          bwd::Epi ep, int64_t a_rows, int64_t b_rows, rudnn_moe_kernel kid, hipStream_t s, float* partials = nullptr) {
    typedef typename std::conditional<MODE == bwd::ROWS, RowsCfg, KRowsCfg>::type C;
    const int NT = (N + C::BN - 1) / C::BN, MT = (M + C::BM - 1) / C::BM;
    const int64_t blocks = MODE == bwd::ROWS ? ((int64_t)rows / C::BM + E) * NT : (int64_t)E * MT * NT;
    if (blocks <= 0) return;
    timing_before(kid, s);
    constexpr int64_t OFFSET_LIMIT = 0x7fffffff;
    if constexpr (sizeof(T) == 2) {
        if (bwd_dma_enabled() && a_rows * A.ld * 2 <= OFFSET_LIMIT && b_rows * B.ld * 2 <= OFFSET_LIMIT) {
            constexpr int LDS = 4 * 256 * bwd::ROWB;  // two stages of two 32 KiB operand tiles
            constexpr bool SPLIT = MODE == bwd::ROWS && EPI != bwd::EPI_SWIGLU;
            static const hipError_t attr = hipFuncSetAttribute(
                (const void*)bwd::gemm_dma_kernel<T, C, MODE, EPI, AK, BK, SPLIT>,
                hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
            (void)attr;
            const int cus = bwd_device_cus();
            const int64_t units = blocks + (SPLIT ? bwd::SPLIT_SLOTS : 0);
            bwd::gemm_dma_kernel<T, C, MODE, EPI, AK, BK, SPLIT><<<dim3((unsigned)units), dim3(C::THREADS), LDS, s>>>(
                A, B, M, N, K, E, plan, offsets, rows, NT, MT, ep, cus, partials);
            if constexpr (SPLIT)
                bwd::split_reduce<T, EPI, C::BM, C::BN><<<1024, 256, 0, s>>>(partials, K, N, E, plan, offsets, rows, NT,
                                                                          cus, ep);
            timing_after(kid, s);
            return;
        }
    }
    static const hipError_t attr = hipFuncSetAttribute((const void*)bwd::gemm_kernel<T, C, MODE, EPI, AK, BK>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    (void)attr;
    bwd::gemm_kernel<T, C, MODE, EPI, AK, BK><<<dim3((unsigned)blocks), dim3(C::THREADS), C::LDS_BYTES, s>>>(
        A, B, M, N, K, E, plan, offsets, rows, NT, MT, ep);
    timing_after(kid, s);
}

template <typename T>
void run(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets, int64_t rows, const float* cache,
         const void* dy, void* dx, float* dgate, float* dup, float* ddown, void* workspace, hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate, R = (int)rows;
    const size_t es = sizeof(T);
    unsigned char* ws = (unsigned char*)workspace;
    T* dgu = (T*)ws;
    T* hbuf = (T*)(ws + align_up((size_t)rows * 2 * I * es));
    int32_t* pl = (int32_t*)((unsigned char*)hbuf + align_up((size_t)rows * I * es));
    unsigned char* after_plan = (unsigned char*)pl + align_up(sizeof(int32_t) * (size_t)(3 * E + 1));
    float* gu = cache ? const_cast<float*>(cache) : (float*)after_plan;
    float* partials = (float*)(after_plan + (cache ? 0 : align_up((size_t)rows * 2 * I * 4)));
    bwd::Plan plan{pl, pl + E, pl + 2 * E};
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_PLAN, s);
    bwd::plan_kernel<<<1, 1024, 0, s>>>(offsets, E, R, RowsCfg::BM, pl, pl + E, pl + 2 * E);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_PLAN, s);
    const int NOSPLIT = 0x7fffffff;
    const int64_t IH = (int64_t)I * H;
    // [g | u] = x [gate; up]^T  (B K-major, gate rows then up rows), unless the forward cached it
    if (!cache)
        gemm<T, bwd::ROWS, bwd::EPI_F32, true, true>({x, x, H, 0, NOSPLIT}, {ex->gate, ex->up, H, IH, I}, R, 2 * I, H,
                                                     E, plan, offsets, R,
                                                     {gu, 2 * (int64_t)I, nullptr, nullptr, nullptr}, R, I,
                                                     RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_GU, s, partials);
    // dh = dy down_e (B(n = i, k = c) = down[e, c, i]: X-major), epilogue -> dg | du, h
    gemm<T, bwd::ROWS, bwd::EPI_SWIGLU, true, false>({dy, dy, H, 0, NOSPLIT}, {ex->down, ex->down, I, IH, NOSPLIT}, R, I,
                                                     H, E, plan, offsets, R, {nullptr, 0, gu, dgu, hbuf}, R, H,
                                                     RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DH, s);
    // dx = [dg | du] [gate; up]  (B(n = c, k = i') = gate[e, i', c] or up[e, i' - I, c]: X-major)
    gemm<T, bwd::ROWS, bwd::EPI_DT, true, false>({dgu, dgu, 2 * (int64_t)I, 0, NOSPLIT}, {ex->gate, ex->up, H, IH, I}, R,
                                                 H, 2 * I, E, plan, offsets, R, {dx, H, nullptr, nullptr, nullptr}, R,
                                                 I, RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DX, s, partials);
    // dgate_e = dg^T x, dup_e = du^T x  (both X-major, K = the expert's rows)
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dgu, dgu, 2 * (int64_t)I, 0, NOSPLIT}, {x, x, H, 0, NOSPLIT}, I, H,
                                                    0, E, plan, offsets, R, {dgate, H, nullptr, nullptr, nullptr}, R,
                                                    R, RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dgu + I, dgu + I, 2 * (int64_t)I, 0, NOSPLIT},
                                                    {x, x, H, 0, NOSPLIT}, I, H, 0, E, plan, offsets, R,
                                                    {dup, H, nullptr, nullptr, nullptr}, R, R,
                                                    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
    // ddown_e = dy^T h
    gemm<T, bwd::KROWS, bwd::EPI_F32, false, false>({dy, dy, H, 0, NOSPLIT}, {hbuf, hbuf, I, 0, NOSPLIT}, H, I, 0, E,
                                                    plan, offsets, R, {ddown, I, nullptr, nullptr, nullptr}, R, R,
                                                    RUDNN_MOE_KERNEL_EXPERTS_BACKWARD_DW, s);
}

}  // namespace

hipError_t launch_experts_backward(const rudnn_moe_experts* ex, const void* x, const int32_t* offsets, int64_t rows,
                                   const float* cache, const void* dy, void* dx, float* dgate, float* dup,
                                   float* ddown, void* workspace, hipStream_t s) {
    switch (ex->dtype) {
    case RUDNN_MOE_F32: run<float>(ex, x, offsets, rows, cache, dy, dx, dgate, dup, ddown, workspace, s); break;
    case RUDNN_MOE_F16: run<f16>(ex, x, offsets, rows, cache, dy, dx, dgate, dup, ddown, workspace, s); break;
    default: run<bf16>(ex, x, offsets, rows, cache, dy, dx, dgate, dup, ddown, workspace, s); break;
    }
    return hipGetLastError();
}

}  // namespace rudnn
