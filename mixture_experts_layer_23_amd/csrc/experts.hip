// experts.hip -- bias-free SwiGLU experts on the dispatched rows (ruDNN user guide, sections
// 3 and 5: SwiGluExperts::forward_dispatched; gate/up [E,I,H], down [E,H,I]).
//
//   h[r, :] = dtype( silu(X_e gate_e^T) * (X_e up_e^T) )  for the rows r of expert e
//   y[r, :] = dtype( h_e down_e^T )
//
// Both products contract over a contiguous axis of both operands ("TN" GEMMs).  Three kernels:
//   plan     one block: clamps the device-side expert offsets to [0, rows], counts BM-row
//            tiles per expert and their exclusive prefix (no host round trip, no sync);
//   skinny   experts with at most SMALL_ROWS rows when a batch has few rows per expert
//            (decode): weight rows streamed whole, FP32 FMAs (see skinny_gemm);
//   gate_up  grouped GEMM, N = I, fused epilogue silu(g) * u (two accumulator sets per tile);
//   down     grouped GEMM, N = H, K = I.
// BF16/F16: v_mfma_f32_32x32x16_{bf16,f16} with FP32 accumulators.  A block of eight wavefronts
// (4 along M x 2 along N, two per SIMD) owns a 256-row tile: gate_up 192 columns of gate + 192 of
// up (384 accumulator columns, 192 registers per lane), down 256 columns.  K is staged 64 at a
// time: tokens and weight rows go straight from global memory into LDS with buffer_load_dwordx4
// ... lds (no register staging), in an XOR-swizzled layout that keeps the MFMA operand reads
// free of bank conflicts.  Two LDS stages: the copies of step k+1 are issued under the MFMAs of
// step k; one barrier per step.
// F32: a plain FP32 FMA tile (64 x 64) on the same tile plan -- no reduced-precision step.
// Training (section 12, forward_dispatched_training): the gate_up epilogue also stores the FP32
// pre-activations [g | u] of every row as the backward's cache (a kernel variant of its own, so
// the plain forward is unchanged).
//
// Tile order.  Tiles of expert e are enumerated in groups of GROUP_N n-tiles, all m-tiles of a
// group together, so tiles that run side by side share both their weight columns and their
// token rows.  Workgroups reach the 8 XCDs round-robin (block b on XCD b % 8); within each
// round of CUs blocks, XCD x takes the contiguous eighth x of the round's units, so the tiles
// that share operands meet in one XCD's L2 (on the Mixtral-shaped layer this cut the gate/up
// fetches from L2 misses by 14% and the down ones by 36%).  (Dealing each XCD a contiguous share
// of the whole list instead measured slower.)  The grid is sized for the worst case
// (floor(rows / BM) + min(E, rows) m-tiles, plus the split units below); blocks beyond the real
// count exit at once.
//
// Tail split.  Tiles run one per CU in rounds; when the tile count leaves a last, partial round
// of R tiles, each of those R tiles is cut along K into S segments (S = CUs / R, at most
// SPLIT_SLOTS / R, each at least SPLIT_MIN_STEPS K steps), so the last round fills the machine.
// A segment stores its FP32 partial sums; a small reduce kernel then adds the S partials of each
// split tile in segment order (deterministic) and applies the epilogue.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace rudnn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef RUDNN_DMA_SPREAD
#define RUDNN_DMA_SPREAD 1
#endif
#ifndef RUDNN_SPLIT_MIN_STEPS
#define RUDNN_SPLIT_MIN_STEPS 8
#endif
#ifndef RUDNN_GROUP_N
#define RUDNN_GROUP_N 4
#endif
constexpr int GROUP_N = RUDNN_GROUP_N;  // n-tiles scheduled together (see "Tile order")
constexpr int SPLIT_SLOTS = 256;        // partial-sum slots of the tail split (see "Tail split")

// ---------------------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------------------
struct Plan {
    int32_t* row_begin;  // [E]
    int32_t* row_count;  // [E]
    int32_t* mt_begin;   // [E + 1]
};

__global__ __launch_bounds__(1024) void experts_plan_kernel(const int32_t* __restrict__ offsets, int E, int rows,
                                                            int BM, int small_rows, Plan plan) {
    __shared__ int scratch[17];
    const int e = threadIdx.x;
    int tiles = 0;
    if (e < E) {
        const int a = min(max(offsets[e], 0), rows);
        const int b = min(max(offsets[e + 1], 0), rows);
        const int n = max(b - a, 0);
        plan.row_begin[e] = a;
        plan.row_count[e] = n;
        tiles = n > small_rows ? (n + BM - 1) / BM : 0;  // experts of <= small_rows rows: skinny_gemm
    }
    int total;
    const int excl = block_exclusive_scan(tiles, scratch, &total);
    if (e < E) plan.mt_begin[e] = excl;
    if (e == 0) plan.mt_begin[E] = total;
}

struct Tile {
    int e, row0, nrows, n0;
};

// Loads the tile plan into LDS (`s_mt` is __shared__ int[E+1]) and returns the tile count.
__device__ __forceinline__ int64_t load_plan(const Plan& plan, int E, int NT, int* s_mt) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_mt[i] = plan.mt_begin[i];
    __syncthreads();
    return (int64_t)s_mt[E] * NT;
}

// Tile L of the list (see "Tile order").
template <int BM, int BN>
__device__ __forceinline__ void decode_tile(const Plan& plan, const int* s_mt, int E, int NT, int64_t L, Tile& t) {
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
}

// The tail split (see "Tail split"): the last R tiles of the list are cut into S segments each.
struct Split {
    int64_t full;  // tiles run whole
    int R, S;      // split tiles, segments per split tile (R = 0, S = 1: no split)
};

__device__ __forceinline__ Split split_plan(int64_t tiles, int KT, int cus) {
    Split sp;
    int64_t R = tiles >= cus ? tiles % cus : tiles;
    int S = R > 0 ? (int)min((int64_t)cus / R, (int64_t)SPLIT_SLOTS / R) : 1;
    S = min(S, KT / RUDNN_SPLIT_MIN_STEPS);
    if (S < 2) S = 1, R = 0;
    sp.full = tiles - R;
    sp.R = (int)R;
    sp.S = S;
    return sp;
}

// This block's work: a whole tile (slot -1) or segment `seg` of a split tile, which leaves its
// partial sums in partial slot `slot`.  False if the block has no work.
struct Unit {
    int kb, ke;  // K steps [kb, ke)
    int slot;    // partial slot, -1 for a whole tile
};

template <int BM, int BN>
__device__ __forceinline__ bool find_unit(const Plan& plan, int E, int N, int KT, int cus, int* s_mt, Tile& t,
                                          Unit& u) {
    const int NT = (N + BN - 1) / BN;
    const int64_t tiles = load_plan(plan, E, NT, s_mt);
    const Split sp = split_plan(tiles, KT, cus);
    int64_t U = blockIdx.x;
    {
        // XCD x runs blocks x, x + 8, ...; within each full round of `cus` blocks it takes the
        // contiguous slice [x * cus/8, (x+1) * cus/8) of the round's units (a bijection on the
        // round; a last, partial round keeps block order).
        const int64_t units = sp.full + (int64_t)sp.R * sp.S;
        if (cus % 8 == 0 && U < units / cus * cus) {
            const int64_t r = U / cus;
            const int j = (int)(U - r * cus);
            U = r * cus + (int64_t)(j % 8) * (cus / 8) + j / 8;
        }
    }
    int64_t L;
    if (U < sp.full) {
        L = U, u.kb = 0, u.ke = KT, u.slot = -1;
    } else {
        const int64_t v = U - sp.full;
        if (v >= (int64_t)sp.R * sp.S) return false;
        const int seg = (int)(v % sp.S);
        L = sp.full + v / sp.S;
        u.kb = (int)((int64_t)seg * KT / sp.S);
        u.ke = (int)((int64_t)(seg + 1) * KT / sp.S);
        u.slot = (int)v;
    }
    decode_tile<BM, BN>(plan, s_mt, E, NT, L, t);
    return true;
}

// Whole tiles only (the FP32 path).
template <int BM, int BN>
__device__ __forceinline__ bool find_tile(const Plan& plan, int E, int N, int* s_mt, Tile& t) {
    const int NT = (N + BN - 1) / BN;
    const int64_t tiles = load_plan(plan, E, NT, s_mt);
    if ((int64_t)blockIdx.x >= tiles) return false;
    decode_tile<BM, BN>(plan, s_mt, E, NT, blockIdx.x, t);
    return true;
}

// silu(z) = z / (1 + e^-z) from the hardware exp and reciprocal (v_exp_f32, v_rcp_f32): a few FP32
// ulps from the exact value, far below the 16-bit rounding of h that follows, and about 20 fewer
// VALU instructions per output than an IEEE division -- the epilogue runs while the matrix cores
// idle (Mixtral-shaped gate/up 1.77 -> 1.73 ms, skewed 0.56-0.58 -> 0.54 ms on one box).
// e^-z = inf for z < -88 gives -0 (z * 0), as the division does; z = -inf gives NaN either way.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

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

// Tile shapes: block rows BM, output columns BN per weight set, WM x WN wavefronts, K elements
// per LDS stage BK (32 or 64), STAGES LDS buffers.  gate_up stages 2*BN weight rows (gate then
// up) per tile.
#ifndef RUDNN_GATE_UP_TILE
#define RUDNN_GATE_UP_TILE 256, 192, 4, 2, 64, 2
#endif
#ifndef RUDNN_DOWN_TILE
#define RUDNN_DOWN_TILE 256, 256, 4, 2, 64, 2
#endif

template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_, int OCC_ = 1>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, STAGES = STAGES_;
    static constexpr int OCC = OCC_;  // wavefronts per SIMD the register budget is sized for
    static constexpr int THREADS = WM * WN * 64;
    static constexpr int ROWB = BK * 2;     // bytes of one staged row (16-bit elements)
    static constexpr int CPR = ROWB / 16;   // 16-byte chunks per staged row
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
};
typedef TileCfg<RUDNN_GATE_UP_TILE> GateUpCfg;
typedef TileCfg<RUDNN_DOWN_TILE> DownCfg;

// Staged rows hold CPR 16-byte chunks; chunk c of row r is stored at c ^ swz(r).  MFMA operand
// reads take one chunk from each of 32 consecutive rows.  With 128-byte rows the swizzle gives
// any 8 consecutive aligned rows, and the even and the odd rows of any 16, eight different
// chunk slots; with 64-byte rows the four rows of any 16 that share an LDS bank offset get
// four different slots.  Either way the reads spread over all LDS banks.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    return CPR == 8 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Staging.  A tile step copies BM rows of tokens and NB = NSETS * BN weight rows, BK elements
// each, straight from global memory into swizzled LDS (buffer_load_dwordx4 ... lds: lane i of a
// wave writes 16 bytes at the wave's LDS base + 16 i, so one wave instruction fills 1 KiB =
// 1024 / ROWB rows).  The buffer form, not global_load_lds, because the compiler counts the
// global form against the LDS-read counter as well and then waits for every outstanding LDS
// read (lgkmcnt 0) before each MFMA group; with buffer copies it waits for exactly the operand
// fragments each MFMA needs.  The copies of one step are numbered as slots (token groups first, then
// weight groups) and dealt round-robin to the first half of the wavefronts only, one per SIMD
// (wavefronts w and w + 4 of the eight share a SIMD): a copying wavefront stalls while its
// copies queue for issue, and its SIMD's other wavefront keeps the matrix core busy meanwhile.
// With every wavefront copying, all eight stalled together at the start of each step (measured:
// Mixtral-shaped experts 2.521-2.523 ms with half the wavefronts copying, 2.557-2.561 ms with all).
// A row past the end of its region reads zeros through the buffer's range check (or, in the
// general form, re-reads the last row); such rows are never stored.  In the last step of a K that
// is not a multiple of BK, chunks at k >= K are zeroed instead of copied.
// Offsets from a tile's base pointers are 32-bit: a tile spans at most a few MB of a matrix.
struct StageSrc {
    __amdgpu_buffer_rsrc_t ra;   // token rows of the tile
    __amdgpu_buffer_rsrc_t rb0;  // weight rows (gate, or down)
    __amdgpu_buffer_rsrc_t rb1;  // up weight rows (gate_up only)
    int ld_bytes, last_a, last_b, K, esize;
    int voff;  // 128-byte rows: this lane's byte offset within any copy (row lane / 8, swizzled chunk)
};

template <typename Cfg, int NSETS, int NWAVES, bool TAIL>
__device__ __forceinline__ void stage_slot(int slot, unsigned char* st, const StageSrc& src, int k0, int wave,
                                           int lane) {
    constexpr int CPR = Cfg::CPR, RPG = 64 / CPR;  // rows per 1 KiB wave copy
    constexpr int GA = Cfg::BM / RPG, GB = Cfg::BN / RPG;  // groups per region
    static_assert(GA % NWAVES == 0 && GB % NWAVES == 0, "each region splits evenly over the wavefronts");
    const int gi = wave + slot * NWAVES;  // global group index over A, B0, B1
    // the region depends on the slot only (a constant once the slot loop is unrolled)
    __amdgpu_buffer_rsrc_t rs;
    int g, last;
    if (slot < GA / NWAVES) {
        rs = src.ra, g = gi, last = src.last_a;
    } else if (NSETS == 1 || slot < (GA + GB) / NWAVES) {
        rs = src.rb0, g = gi - GA, last = src.last_b;
    } else {
        rs = src.rb1, g = gi - GA - GB, last = src.last_b;
    }
    // A group of token rows wholly past the tile's last row is not copied: those LDS rows only
    // feed output rows that are never stored (each output row depends on its own token row).
    // Only with two stages, whose steps wait for every copy (vmcnt 0): with deeper pipelines
    // the per-step copy counts that the waits assume must not vary.
    if (Cfg::STAGES == 2 && slot < GA / NWAVES && g * RPG > last) return;
    unsigned char* const dst0 = st + gi * 1024;
    if constexpr (CPR == 8 && !TAIL) {
        // Row g * 8 + lane / 8 and chunk (lane % 8) ^ swz(row), where swz(row) = lane / 8 ^ (g & 1)
        // and g has the parity of the wavefront (the region offsets and the wavefront stride are
        // even): a per-lane offset fixed for the tile (src.voff) plus a uniform part, so a copy costs
        // one vector add.  Rows past the region's last valid row read zeros through the buffer's
        // range check (the range covers exactly the rows a tile may read); their outputs are never
        // stored.
        static_assert(GA % 2 == 0 && GB % 2 == 0 && NWAVES % 2 == 0, "copy groups keep the wavefront's parity");
        const uint32_t off = (uint32_t)src.voff + (uint32_t)(g * RPG * src.ld_bytes + k0 * src.esize);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst0, 16, off, 0, 0, 0);
        return;
    }
    const int r = g * RPG + lane / CPR;
    const int kk = k0 + ((lane % CPR) ^ swz<CPR>(r)) * 8;
    const int rr = r < last ? r : last;
    unsigned char* dst = st + gi * 1024;
    if (!TAIL || kk < src.K)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                                                 rr * src.ld_bytes + kk * src.esize, 0, 0, 0);
    else
        *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
}

// Grouped GEMM on MFMA: for the tile's expert e, C[r, n] = sum_k A[r, k] B_e[n, k] over the
// tile's rows; DUAL computes gate and up together and stores silu(gate) * up.  CACHE (with DUAL)
// also stores the FP32 pre-activations, cache[r] = [gate . x_r | up . x_r] ([rows, 2N]).
template <typename T, bool DUAL, typename Cfg, bool CACHE = false>
__global__ __launch_bounds__(Cfg::THREADS, Cfg::OCC) void grouped_gemm_mfma(const T* __restrict__ A,
                                                                            const T* __restrict__ B0,
                                                                            const T* __restrict__ B1,
                                                                            T* __restrict__ C, int K, int N, int E,
                                                                            Plan plan, int cus,
                                                                            float* __restrict__ partials,
                                                                            float* __restrict__ cache) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, WM = Cfg::WM, WN = Cfg::WN, STAGES = Cfg::STAGES;
    constexpr int BK = Cfg::BK, ROWB = Cfg::ROWB, CPR = Cfg::CPR;
    constexpr int NWAVES = WM * WN;
    constexpr int NSETS = DUAL ? 2 : 1;
    constexpr int NB = NSETS * BN;          // weight rows staged per tile
    constexpr bool ROLL = DUAL;             // weight-fragment-outer MFMA order (see step)
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int KS = BK / 16;             // MFMA steps per staged tile
    constexpr int A_BYTES = BM * ROWB, STAGE_BYTES = (BM + NB) * ROWB;
    constexpr int CW = NWAVES / 2;                           // copying wavefronts, one per SIMD
    constexpr int SLOTS = (BM + NB) * ROWB / 1024 / CW;      // copies per copying wave per stage
    static_assert((BM + NB) * ROWB % (1024 * CW) == 0, "copies must split evenly over the wavefronts");
    static_assert(BM * ROWB % 1024 == 0 && BN * ROWB % 1024 == 0, "regions are whole 1 KiB copies");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles are made of 32x32 MFMA blocks");
    typedef typename Mfma<T>::frag frag;

    extern __shared__ __align__(1024) unsigned char smem_raw[];
    int* s_mt = reinterpret_cast<int*>(smem_raw);
    const int KT = (K + BK - 1) / BK;
    Tile tile;
    Unit unit;
    if (!find_unit<BM, BN>(plan, E, N, KT, cus, s_mt, tile, unit)) return;
    __syncthreads();  // s_mt shares space with the stages

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
    // Wavefronts go to the four SIMDs of the CU round-robin (wave w on SIMD w % 4).  Neighbouring
    // waves share a row band, so a tile with few rows still spreads its MFMAs over several SIMDs
    // instead of stacking them on one (rows <= 64: two SIMDs, rows <= 128: all four).
    const int wm = wave / WN, wn = wave % WN;
    const int nrows = tile.nrows, n0 = tile.n0;
    StageSrc src;
    src.ld_bytes = K * (int)sizeof(T);
    src.last_a = nrows - 1;
    src.last_b = N - 1 - n0;
    src.K = K;
    src.esize = (int)sizeof(T);
    src.voff = (lane / CPR) * src.ld_bytes + (((lane % CPR) ^ (lane / CPR) ^ (wave & 1)) * 8) * src.esize;
    {
        // raw buffers over exactly the rows a tile may read (the copies clamp to them anyway)
        constexpr int GFX9_RSRC_WORD3 = 0x00020000;  // 32-bit data format, no swizzle
        const int b_bytes = min(src.last_b + 1, BN) * src.ld_bytes;
        src.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)tile.row0 * K), (short)0,
                                                   nrows * src.ld_bytes, GFX9_RSRC_WORD3);
        src.rb0 = __builtin_amdgcn_make_buffer_rsrc((void*)(B0 + ((int64_t)tile.e * N + n0) * K), (short)0, b_bytes,
                                                    GFX9_RSRC_WORD3);
        src.rb1 = DUAL ? __builtin_amdgcn_make_buffer_rsrc((void*)(B1 + ((int64_t)tile.e * N + n0) * K), (short)0,
                                                           b_bytes, GFX9_RSRC_WORD3)
                       : src.rb0;
    }
    const bool ragged_k = (K % BK) != 0;

    // all copies of step kt (the tail form zeroes chunks past K)
    auto issue_all = [&](int kt) __attribute__((always_inline)) {
        unsigned char* st = smem_raw + (kt % STAGES) * STAGE_BYTES;
        if (wave >= CW) return;
        if (ragged_k && kt == KT - 1) {
#pragma unroll
            for (int q = 0; q < SLOTS; ++q) stage_slot<Cfg, NSETS, CW, true>(q, st, src, kt * BK, wave, lane);
        } else {
#pragma unroll
            for (int q = 0; q < SLOTS; ++q) stage_slot<Cfg, NSETS, CW, false>(q, st, src, kt * BK, wave, lane);
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

    // Rows of this wavefront that hold real tokens (a wavefront without any skips its MFMAs).
    const int wave_rows = min(max(nrows - wm * WTM, 0), WTM);
    const int fr = lane & 31, fh = lane >> 5;
    int lane_off[KS];  // byte offset of this lane's 16-byte operand chunk in a 32-row block
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) lane_off[ks] = fr * ROWB + (((ks * 2 + fh) ^ swz<CPR>(fr)) * 16);

    // The MFMAs of one staged step.  Operand fragments of MFMA step ks+1 are read from LDS while
    // the MFMAs of step ks run; with ISSUE, the copies of step kt_next are spread over the MFMA
    // steps.  gate_up (ROLL) has no registers left for a second set of weight fragments: its
    // MFMAs run weight-fragment-outer and each weight fragment is reloaded for step ks+1 right
    // after its FM MFMAs (a fence after each group keeps that order).  down double-buffers all
    // fragments, with a fence after each MFMA step.
    auto step = [&](int kt, auto with_mfma, auto with_issue, int kt_next) __attribute__((always_inline)) {
        const unsigned char* st = smem_raw + (kt % STAGES) * STAGE_BYTES;
        unsigned char* st_next = smem_raw + (kt_next % STAGES) * STAGE_BYTES;
        const unsigned char* a = st + (wm * WTM) * ROWB;
        const unsigned char* b = st + A_BYTES + (wn * WTN) * ROWB;
        if constexpr (ROLL) {
        // Weight-fragment-outer order: each weight fragment feeds its FM MFMAs and its register is
        // then reloaded with the next MFMA step's fragment at once, so every LDS read has about a
        // whole MFMA step to land while only the token fragments are double-buffered (the
        // accumulators leave no room for a second set of weight fragments).
        frag fa[2][FM], fb[NSETS][FN];
        auto fetch_a = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[buf][i] = *reinterpret_cast<const frag*>(a + i * 32 * ROWB + lane_off[ks]);
        };
        auto fetch_b = [&](int ks, int s, int j) __attribute__((always_inline)) {
            fb[s][j] = *reinterpret_cast<const frag*>(b + (s * BN + j * 32) * ROWB + lane_off[ks]);
        };
        if constexpr (decltype(with_mfma)::value) {
            fetch_a(0, 0);
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
#pragma unroll
                for (int j = 0; j < FN; ++j) fetch_b(0, s, j);
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (decltype(with_issue)::value) {
                // copies for the next step go out at once, from the copying wavefronts: spread over
                // the first DMA_SPREAD MFMA steps (one by default)
                constexpr int SP = RUDNN_DMA_SPREAD < KS ? RUDNN_DMA_SPREAD : KS;
                if (ks < SP && wave < CW) {
#pragma unroll
                    for (int q = ks * SLOTS / SP; q < (ks + 1) * SLOTS / SP; ++q)
                        stage_slot<Cfg, NSETS, CW, false>(q, st_next, src, kt_next * BK, wave, lane);
                }
            }
            if constexpr (decltype(with_mfma)::value) {
                if (ks + 1 < KS) fetch_a(ks + 1, (ks + 1) & 1);
#pragma unroll
                for (int s = 0; s < NSETS; ++s)
#pragma unroll
                    for (int j = 0; j < FN; ++j) {
#pragma unroll
                        for (int i = 0; i < FM; ++i)
                            acc[s][i][j] = Mfma<T>::run(fb[s][j], fa[ks & 1][i], acc[s][i][j]);
                        if (ks + 1 < KS) fetch_b(ks + 1, s, j);
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        } else {
        frag fa[2][FM], fb[2][NSETS][FN];
        auto fetch = [&](int ks, int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[buf][i] = *reinterpret_cast<const frag*>(a + i * 32 * ROWB + lane_off[ks]);
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    fb[buf][s][j] = *reinterpret_cast<const frag*>(b + (s * BN + j * 32) * ROWB + lane_off[ks]);
        };
        if constexpr (decltype(with_mfma)::value) fetch(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (decltype(with_issue)::value) {
                // copies for the next step go out at once, from the copying wavefronts: spread over
                // the first DMA_SPREAD MFMA steps (one by default)
                constexpr int SP = RUDNN_DMA_SPREAD < KS ? RUDNN_DMA_SPREAD : KS;
                if (ks < SP && wave < CW) {
#pragma unroll
                    for (int q = ks * SLOTS / SP; q < (ks + 1) * SLOTS / SP; ++q)
                        stage_slot<Cfg, NSETS, CW, false>(q, st_next, src, kt_next * BK, wave, lane);
                }
            }
            if constexpr (decltype(with_mfma)::value) {
                if (ks + 1 < KS) fetch(ks + 1, (ks + 1) & 1);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int s = 0; s < NSETS; ++s)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
                            acc[s][i][j] = Mfma<T>::run(fb[ks & 1][s][j], fa[ks & 1][i], acc[s][i][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
    };

    // The K loop over this unit's steps [kb, ke); a wavefront without rows only helps stage the
    // tiles.  Three straight-line loops, so the accumulators stay in place: the steady state
    // (copies of step kt+STAGES-1 under the MFMAs of step kt), the step that issues a ragged last
    // K tile, and the drain.
    const int kb = unit.kb, ke = unit.ke;
    const bool last_ragged = ragged_k && ke == KT;
    auto kloop = [&](auto with_mfma) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (kb + s < ke) issue_all(kb + s);
        const int steady = ke - (STAGES - 1) - (last_ragged ? 1 : 0);
        int kt = kb;
        for (; kt < steady; ++kt) {
            wait_vmcnt<(STAGES - 2) * SLOTS>();  // this wavefront's copies of step kt have landed
            __syncthreads();  // everyone's copies of step kt landed; everyone is done with step kt-1
            step(kt, with_mfma, std::true_type{}, kt + STAGES - 1);
        }
        if (last_ragged && ke - kb >= STAGES) {  // kt == ke - STAGES: stage the ragged last tile
            wait_vmcnt<(STAGES - 2) * SLOTS>();
            __syncthreads();
            issue_all(ke - 1);
            step(kt, with_mfma, std::false_type{}, kt);
            ++kt;
        }
        for (; kt < ke; ++kt) {
            wait_vmcnt<0>();
            __syncthreads();
            step(kt, with_mfma, std::false_type{}, kt);
        }
    };
    if (wave_rows > 0)
        kloop(std::true_type{});
    else
        kloop(std::false_type{});

    // Epilogue.  The MFMAs take the weight fragment as their first operand, so each 32 x 32
    // accumulator block is the transposed output: lane l holds token row l % 32 and output
    // columns 8 * (v / 4) + 4 * (l / 32) + v % 4 for v = 0..15, i.e. four runs of four adjacent
    // columns.  Each run goes to LDS as one 8-byte write into a row-major [BM][BN] tile (rows
    // padded by 16 bytes), which is then stored to global memory in 16-byte pieces, whole rows per
    // wavefront instruction.  N is a multiple of 8, so a piece lies wholly inside or outside it.
    if (unit.slot >= 0) {
        // a segment of a split tile: FP32 partial sums, [slot][BM][NSETS * BN], rows past the
        // tile and columns past N left unwritten (the reduce kernel never reads them)
        float* P = partials + (int64_t)unit.slot * BM * NB;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 32 + fr;
            if (row >= nrows) continue;
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * WTN + j * 32 + 8 * q + 4 * fh;
                        if (n0 + col >= N) continue;
                        float4 v4 = make_float4(acc[s][i][j][4 * q], acc[s][i][j][4 * q + 1], acc[s][i][j][4 * q + 2],
                                                acc[s][i][j][4 * q + 3]);
                        *reinterpret_cast<float4*>(P + (int64_t)row * NB + s * BN + col) = v4;
                    }
        }
        return;
    }
    if constexpr (DUAL && CACHE) {
        // each lane's runs of four adjacent columns, straight from the accumulators
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * WTM + i * 32 + fr;
            if (row >= nrows) continue;
            float* crow = cache + (int64_t)(tile.row0 + row) * 2 * N + n0;
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * WTN + j * 32 + 8 * q + 4 * fh;
                        if (n0 + col >= N) continue;
                        *reinterpret_cast<float4*>(crow + s * N + col) =
                            make_float4(acc[s][i][j][4 * q], acc[s][i][j][4 * q + 1], acc[s][i][j][4 * q + 2],
                                        acc[s][i][j][4 * q + 3]);
                    }
        }
    }
    constexpr int PITCH = BN * (int)sizeof(T) + 16;  // bytes per staged output row
    constexpr int CHUNKS = BN * (int)sizeof(T) / 16;  // 16-byte pieces per row
    constexpr int LDS_MAX = 160 * 1024;
    constexpr int PASSES = (BM * PITCH + LDS_MAX - 1) / LDS_MAX;  // row bands staged one at a time
    constexpr int PROWS = BM / PASSES;                            // rows per band
    static_assert(WM % PASSES == 0 && PROWS * PITCH <= LDS_MAX, "output bands follow the wavefront rows");
    T* Cb = C + (int64_t)tile.row0 * N + n0;
    const int ncols = min(BN, N - n0);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        __syncthreads();  // the stages (or the previous band) are no longer read
        if (wm / (WM / PASSES) == pass) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WTM + i * 32 + fr - pass * PROWS;
#pragma unroll
                for (int j = 0; j < FN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = wn * WTN + j * 32 + 8 * q + 4 * fh;
                        T out[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int v = 4 * q + u;
                            const float val =
                                DUAL ? silu_f(acc[0][i][j][v]) * acc[NSETS - 1][i][j][v] : acc[0][i][j][v];
                            out[u] = from_f32<T>(val);
                        }
                        uint2 packed;
                        __builtin_memcpy(&packed, out, sizeof(packed));
                        *reinterpret_cast<uint2*>(smem_raw + row * PITCH + col * (int)sizeof(T)) = packed;
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int p = tid; p < PROWS * CHUNKS; p += Cfg::THREADS) {
            const int r = p / CHUNKS, ch = p % CHUNKS, row = pass * PROWS + r;
            if (row < nrows && ch * 8 < ncols)
                *reinterpret_cast<uint4*>(Cb + (int64_t)row * N + ch * 8) =
                    *reinterpret_cast<const uint4*>(smem_raw + r * PITCH + ch * 16);
        }
    }
}

// Adds the S partials of every split tile in segment order and applies the epilogue (silu(g) * u
// for gate_up).  A block takes a slab of 2048 / BN rows of one split tile (the tile is decoded
// once per slab); a thread takes 8 output columns of one row.
template <typename T, bool DUAL, typename Cfg, bool CACHE = false>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ partials, T* __restrict__ C, int K,
                                                     int N, int E, Plan plan, int cus, float* __restrict__ cache) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, NSETS = DUAL ? 2 : 1, NB = NSETS * BN;
    constexpr int CPRW = BN / 8, SLAB = 256 / CPRW;  // 8-column chunks per row, rows per slab
    constexpr int SLABS = (BM + SLAB - 1) / SLAB;     // slabs per tile
    __shared__ int s_mt[MAX_EXPERTS + 1];
    const int NT = (N + BN - 1) / BN;
    const int KT = (K + Cfg::BK - 1) / Cfg::BK;
    const Split sp = split_plan(load_plan(plan, E, NT, s_mt), KT, cus);
    const int slabs = sp.R * SLABS;
    for (int b = blockIdx.x; b < slabs; b += gridDim.x) {
        const int r = b / SLABS;
        Tile t;
        decode_tile<BM, BN>(plan, s_mt, E, NT, sp.full + r, t);
        const int row = (b % SLABS) * SLAB + threadIdx.x / CPRW;
        const int col = (threadIdx.x % CPRW) * 8;
        if (threadIdx.x >= SLAB * CPRW || row >= min(t.nrows, BM) || t.n0 + col >= N) continue;
        const float* P = partials + ((int64_t)r * sp.S * BM + row) * NB + col;
        const int64_t seg_stride = (int64_t)BM * NB;
        float g[8] = {}, u[8] = {};
        auto add = [&](const float* q, float* acc) __attribute__((always_inline)) {
            const float4 x0 = *reinterpret_cast<const float4*>(q), x1 = *reinterpret_cast<const float4*>(q + 4);
            acc[0] += x0.x, acc[1] += x0.y, acc[2] += x0.z, acc[3] += x0.w;
            acc[4] += x1.x, acc[5] += x1.y, acc[6] += x1.z, acc[7] += x1.w;
        };
#pragma unroll 4
        for (int seg = 0; seg < sp.S; ++seg) {
            add(P + seg * seg_stride, g);
            if (DUAL) add(P + seg * seg_stride + BN, u);
        }
        if constexpr (DUAL && CACHE) {
            float* c = cache + (int64_t)(t.row0 + row) * 2 * N + t.n0 + col;
            *reinterpret_cast<float4*>(c) = make_float4(g[0], g[1], g[2], g[3]);
            *reinterpret_cast<float4*>(c + 4) = make_float4(g[4], g[5], g[6], g[7]);
            *reinterpret_cast<float4*>(c + N) = make_float4(u[0], u[1], u[2], u[3]);
            *reinterpret_cast<float4*>(c + N + 4) = make_float4(u[4], u[5], u[6], u[7]);
        }
        T out[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) out[q] = from_f32<T>(DUAL ? silu_f(g[q]) * u[q] : g[q]);
        uint4 packed;
        __builtin_memcpy(&packed, out, sizeof(packed));
        *reinterpret_cast<uint4*>(C + (int64_t)(t.row0 + row) * N + t.n0 + col) = packed;
    }
}

// ---------------------------------------------------------------------------------------
// FP32 grouped GEMM (FMA): tile 64 x 64, K staged 16 at a time, 256 threads x (4 x 4) outputs.
// ---------------------------------------------------------------------------------------
constexpr int F_BM = 64, F_BN = 64, F_BK = 16;

template <bool DUAL>
__global__ __launch_bounds__(256) void grouped_gemm_f32(const float* __restrict__ A, const float* __restrict__ B0,
                                                        const float* __restrict__ B1, float* __restrict__ C, int K,
                                                        int N, int E, Plan plan, float* __restrict__ cache) {
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
            if (DUAL && cache) {
                float* c = cache + (int64_t)(tile.row0 + row) * 2 * N + tile.n0 + col;
                c[0] = v, c[N] = acc[1][i][j];
            }
            if (DUAL) v = (v / (1.0f + expf(-v))) * acc[1][i][j];
            Cb[(int64_t)row * N + col] = v;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Experts with few rows (decode-shaped batches)
// ---------------------------------------------------------------------------------------
// With one to SMALL_ROWS rows per expert the products are a stream of weight rows.  The MFMA
// tiles read them in 128-byte pieces, one piece per K step from each of hundreds of rows at
// once; here a wavefront reads a weight row 1 KiB at a time (lane l: elements [512 c + 8 l, +8)
// of chunk c), every chunk of its FR rows (per weight set) in flight together, and forms the dot
// products with the expert's n token rows, staged once per block in LDS, in FP32 FMAs.  A
// wavefront sum gives each (token row, output column); lane r stores token row r's value.  A
// block covers FPB = 8 wavefronts x FR x IT output columns of one expert; blocks of other
// experts exit at once.
constexpr int SMALL_ROWS = 4;

template <typename T>
__device__ __forceinline__ void unpack8(uint4 q, float (&v)[8]) {
    T t[8];
    __builtin_memcpy(t, &q, sizeof(q));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_f32(t[i]);
}

template <typename T, bool DUAL, int JMAX, int FR, int IT>
__global__ __launch_bounds__(512) void skinny_gemm(const T* __restrict__ A, const T* __restrict__ B0,
                                                   const T* __restrict__ B1, T* __restrict__ C, int K, int N, int E,
                                                   Plan plan, int blocks_per_expert) {
    constexpr int NSETS = DUAL ? 2 : 1, NW = 8, FPB = NW * FR * IT;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    const int e = blockIdx.x / blocks_per_expert, b = blockIdx.x % blocks_per_expert;
    if (e >= E) return;
    const int n = plan.row_count[e];
    if (n <= 0 || n > SMALL_ROWS) return;  // block-uniform
    const int r0 = plan.row_begin[e];
    const int kv = K / 8;  // 16-byte vectors per row (K is a multiple of 8)
    uint4* xs = reinterpret_cast<uint4*>(smem_raw);  // [n][kv]
    for (int q = threadIdx.x; q < n * kv; q += blockDim.x) {
        const int r = q / kv, c = q - r * kv;
        xs[q] = reinterpret_cast<const uint4*>(A + (int64_t)(r0 + r) * K)[c];
    }
    __syncthreads();
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int J = (K + 511) / 512;  // chunks per row, <= JMAX (checked by the host)
    const T* Bs[2] = {B0, B1};
    for (int it = 0; it < IT; ++it) {
        const int f0 = b * FPB + (it * NW + wave) * FR;  // this wavefront's FR output columns
        if (f0 >= N) break;                             // wave-uniform
        uint4 wv[NSETS][FR][JMAX];
#pragma unroll
        for (int st = 0; st < NSETS; ++st)
#pragma unroll
            for (int fr = 0; fr < FR; ++fr)
#pragma unroll
                for (int j = 0; j < JMAX; ++j) {
                    const int kk = j * 512 + lane * 8;
                    wv[st][fr][j] = make_uint4(0, 0, 0, 0);
                    if (j < J && kk < K && f0 + fr < N)
                        wv[st][fr][j] = *reinterpret_cast<const uint4*>(Bs[st] + ((int64_t)e * N + f0 + fr) * K + kk);
                }
        float acc[NSETS][FR][SMALL_ROWS] = {};
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
            const int kk = j * 512 + lane * 8;
            if (j >= J) break;
            if (kk >= K) continue;  // this lane's chunk is past the row's end (zero)
            float wf[NSETS][FR][8];
#pragma unroll
            for (int st = 0; st < NSETS; ++st)
#pragma unroll
                for (int fr = 0; fr < FR; ++fr) unpack8<T>(wv[st][fr][j], wf[st][fr]);
#pragma unroll
            for (int r = 0; r < SMALL_ROWS; ++r) {
                if (r >= n) break;
                float x[8];
                unpack8<T>(xs[r * kv + kk / 8], x);
#pragma unroll
                for (int st = 0; st < NSETS; ++st)
#pragma unroll
                    for (int fr = 0; fr < FR; ++fr)
#pragma unroll
                        for (int i = 0; i < 8; ++i) acc[st][fr][r] = fmaf(wf[st][fr][i], x[i], acc[st][fr][r]);
            }
        }
#pragma unroll
        for (int fr = 0; fr < FR; ++fr) {
            if (f0 + fr >= N) break;
#pragma unroll
            for (int r = 0; r < SMALL_ROWS; ++r) {
                if (r >= n) break;
                const float g = wave_sum(acc[0][fr][r]);
                const float v = DUAL ? silu_f(g) * wave_sum(acc[NSETS - 1][fr][r]) : g;
                if (lane == r) C[(int64_t)(r0 + r) * N + f0 + fr] = from_f32<T>(v);
            }
        }
    }
}

// Launch shapes: gate_up reads one row per set (two sets) with up to 16 chunks (K <= 8192);
// down reads four rows with up to 4 chunks (K <= 2048) or one row with up to 16.
constexpr int SKINNY_MAX_K = 8192;

template <typename T, bool DUAL, int JMAX, int FR, int IT>
static void launch_skinny_t(const T* A, const T* B0, const T* B1, T* C, int K, int N, int E, Plan plan,
                            hipStream_t s) {
    constexpr int FPB = 8 * FR * IT;
    const int bpe = (N + FPB - 1) / FPB;
    const size_t lds = (size_t)SMALL_ROWS * K * sizeof(T);
    skinny_gemm<T, DUAL, JMAX, FR, IT><<<(unsigned)((int64_t)E * bpe), 512, lds, s>>>(A, B0, B1, C, K, N, E, plan, bpe);
}

template <typename T>
static void launch_skinny(bool dual, const T* A, const T* B0, const T* B1, T* C, int K, int N, int E, Plan plan,
                          hipStream_t s) {
    if (dual)
        launch_skinny_t<T, true, 16, 1, 4>(A, B0, B1, C, K, N, E, plan, s);
    else if (K <= 2048)
        launch_skinny_t<T, false, 4, 4, 2>(A, B0, nullptr, C, K, N, E, plan, s);
    else
        launch_skinny_t<T, false, 16, 1, 8>(A, B0, nullptr, C, K, N, E, plan, s);
}

// ---------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------
static int64_t max_mtiles(int64_t rows, int64_t E, int BM) { return rows / BM + (E < rows ? E : rows); }

// Partial-sum slots of the tail split: SPLIT_SLOTS x BM x (accumulator columns of the wider
// tile) FP32.
static size_t split_partials_bytes(rudnn_moe_dtype dt) {
    constexpr size_t NB = 2 * GateUpCfg::BN > DownCfg::BN ? 2 * GateUpCfg::BN : DownCfg::BN;  // widest tile
    return dt == RUDNN_MOE_F32 ? 0 : (size_t)SPLIT_SLOTS * GateUpCfg::BM * NB * sizeof(float);
}

size_t experts_workspace_bytes(int64_t E, int64_t H, int64_t I, rudnn_moe_dtype dt, int64_t rows) {
    (void)H;
    return align_up((size_t)rows * I * dtype_size(dt)) + align_up(sizeof(int32_t) * (3 * E + 1)) +
           split_partials_bytes(dt);
}

// Compute units of the current device (the size of one round of tiles), cached per device
// (atomics: threads may fill the same entry at once, always with the same value).
static int device_cus() {
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

template <typename Cfg, bool DUAL>
static size_t mfma_smem_bytes(int64_t E) {
    const size_t stages = (size_t)Cfg::STAGES * (Cfg::BM + (DUAL ? 2 : 1) * Cfg::BN) * Cfg::ROWB;
    const size_t band = (size_t)Cfg::BM * (Cfg::BN * 2 + 16);  // staged 16-bit output rows
    const size_t out_tile = band > 160 * 1024 ? band / 2 : band;
    const size_t mt = sizeof(int) * (size_t)(E + 1);
    size_t bytes = stages > mt ? stages : mt;
    return bytes > out_tile ? bytes : out_tile;
}

template <typename T, bool CACHE>
static void launch_mfma(const rudnn_moe_experts* ex, const void* disp, int64_t rows, void* out, void* h, Plan plan,
                        float* partials, float* cache, bool skinny, hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate;
    const int64_t mt = max_mtiles(rows, E, GateUpCfg::BM);
    const int cus = device_cus();
    // every tile, plus at most SPLIT_SLOTS segments of split tiles
    auto grid_for = [&](int N, int BN) {
        const int64_t units = mt * ((N + BN - 1) / BN) + SPLIT_SLOTS;
        return (unsigned)((units + 7) / 8 * 8);
    };
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    if (skinny) launch_skinny<T>(true, (const T*)disp, (const T*)ex->gate, (const T*)ex->up, (T*)h, H, I, E, plan, s);
    grouped_gemm_mfma<T, true, GateUpCfg, CACHE><<<grid_for(I, GateUpCfg::BN), GateUpCfg::THREADS,
                                                   mfma_smem_bytes<GateUpCfg, true>(E), s>>>(
        (const T*)disp, (const T*)ex->gate, (const T*)ex->up, (T*)h, H, I, E, plan, cus, partials, cache);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP_REDUCE, s);
    splitk_reduce<T, true, GateUpCfg, CACHE><<<1024, 256, 0, s>>>(partials, (T*)h, H, I, E, plan, cus, cache);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP_REDUCE, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
    if (skinny) launch_skinny<T>(false, (const T*)h, (const T*)ex->down, nullptr, (T*)out, I, H, E, plan, s);
    grouped_gemm_mfma<T, false, DownCfg><<<grid_for(H, DownCfg::BN), DownCfg::THREADS,
                                           mfma_smem_bytes<DownCfg, false>(E), s>>>(
        (const T*)h, (const T*)ex->down, nullptr, (T*)out, I, H, E, plan, cus, partials, nullptr);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_DOWN_REDUCE, s);
    splitk_reduce<T, false, DownCfg><<<1024, 256, 0, s>>>(partials, (T*)out, I, H, E, plan, cus, nullptr);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_DOWN_REDUCE, s);
}

static void launch_f32(const rudnn_moe_experts* ex, const void* disp, int64_t rows, void* out, void* h, Plan plan,
                       float* cache, hipStream_t s) {
    const int E = (int)ex->num_experts, H = (int)ex->hidden, I = (int)ex->intermediate;
    const int64_t mt = max_mtiles(rows, E, F_BM);
    auto grid_for = [&](int N) { return (unsigned)((mt * ((N + F_BN - 1) / F_BN) + 7) / 8 * 8); };
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    grouped_gemm_f32<true><<<grid_for(I), 256, 0, s>>>((const float*)disp, (const float*)ex->gate,
                                                       (const float*)ex->up, (float*)h, H, I, E, plan, cache);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_GATE_UP, s);
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
    grouped_gemm_f32<false><<<grid_for(H), 256, 0, s>>>((const float*)h, (const float*)ex->down, nullptr,
                                                        (float*)out, I, H, E, plan, nullptr);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_DOWN, s);
}

// Dynamic LDS above 64 KiB per block has to be allowed per kernel (once per process).
static std::once_flag g_smem_once;
static void allow_large_lds() {
    const int lds = 160 * 1024;

    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<bf16, true, GateUpCfg>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<bf16, false, DownCfg>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<f16, true, GateUpCfg>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<f16, false, DownCfg>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<bf16, true, GateUpCfg, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    (void)hipFuncSetAttribute((const void*)grouped_gemm_mfma<f16, true, GateUpCfg, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    // skinny_gemm stages SMALL_ROWS rows of up to SKINNY_MAX_K elements (64 KiB at the limit)
    (void)hipFuncSetAttribute((const void*)skinny_gemm<bf16, true, 16, 1, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    (void)hipFuncSetAttribute((const void*)skinny_gemm<bf16, false, 4, 4, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    (void)hipFuncSetAttribute((const void*)skinny_gemm<bf16, false, 16, 1, 8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    (void)hipFuncSetAttribute((const void*)skinny_gemm<f16, true, 16, 1, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    (void)hipFuncSetAttribute((const void*)skinny_gemm<f16, false, 4, 4, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
    (void)hipFuncSetAttribute((const void*)skinny_gemm<f16, false, 16, 1, 8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              lds);
}

hipError_t launch_experts(const rudnn_moe_experts* ex, const void* disp, const int32_t* offsets, int64_t rows,
                          void* out, void* workspace, hipStream_t s, float* cache) {
    const int64_t E = ex->num_experts, I = ex->intermediate;
    const size_t es = dtype_size(ex->dtype);
    unsigned char* ws = (unsigned char*)workspace;
    void* h = ws;
    int32_t* ints = (int32_t*)(ws + align_up((size_t)rows * I * es));
    Plan plan{ints, ints + E, ints + 2 * E};
    std::call_once(g_smem_once, allow_large_lds);
    static_assert(GateUpCfg::BM == DownCfg::BM, "both expert GEMMs share one tile plan");
    const int BM = ex->dtype == RUDNN_MOE_F32 ? F_BM : GateUpCfg::BM;
    // Few rows per expert on average (decode-shaped batches): experts with at most SMALL_ROWS rows
    // stream their weights through skinny_gemm and get no MFMA tiles.  Not with the training
    // cache (skinny_gemm does not store the pre-activations).
    const bool skinny = !cache && ex->dtype != RUDNN_MOE_F32 && ex->hidden <= SKINNY_MAX_K && I <= SKINNY_MAX_K &&
                        rows <= SMALL_ROWS * E;
    timing_before(RUDNN_MOE_KERNEL_EXPERTS_PLAN, s);
    experts_plan_kernel<<<1, 1024, 0, s>>>(offsets, (int)E, (int)rows, BM, skinny ? SMALL_ROWS : 0, plan);
    timing_after(RUDNN_MOE_KERNEL_EXPERTS_PLAN, s);
    float* partials = (float*)(ws + align_up((size_t)rows * I * es) + align_up(sizeof(int32_t) * (3 * E + 1)));
    switch (ex->dtype) {
    case RUDNN_MOE_F32: launch_f32(ex, disp, rows, out, h, plan, cache, s); break;
    case RUDNN_MOE_F16:
        if (cache)
            launch_mfma<f16, true>(ex, disp, rows, out, h, plan, partials, cache, false, s);
        else
            launch_mfma<f16, false>(ex, disp, rows, out, h, plan, partials, nullptr, skinny, s);
        break;
    default:
        if (cache)
            launch_mfma<bf16, true>(ex, disp, rows, out, h, plan, partials, cache, false, s);
        else
            launch_mfma<bf16, false>(ex, disp, rows, out, h, plan, partials, nullptr, skinny, s);
        break;
    }
    return hipGetLastError();
}

}  // namespace rudnn
