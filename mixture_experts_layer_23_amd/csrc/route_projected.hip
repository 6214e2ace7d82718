// route_projected.hip -- the gate projection fused with softmax routing.
//
// The guide leaves the gate projection that produces the logits to the caller (ruDNN user
// guide, section 5: forward takes precomputed logits); here it runs inside the router:
//   logits[t, e] = dtype( sum_h x[t, h] * W_r[e, h] ),   x [T, H], W_r [E, H], one dtype,
// accumulated in FP32 and rounded once to the token dtype, then routed exactly as section 4
// routes logits of that dtype (route_row in route_select.hpp).  The [T, E] logits stay on chip
// unless the caller asks for a copy.
//
// project_route: a block owns BM = 32 WM token rows and every expert (E padded to EP, a multiple
// of 32).  Its wavefronts (4 or 8) split the tile WM x WN x WK ways: WM bands of 32 tokens, WN
// bands of EP / WN experts, WK interleaved parts of each staged K step (WK > 1 when E is small,
// so that all SIMDs work on a small tile).  The K axis is staged 128 bytes at a time (64 16-bit
// or 32 FP32 elements): token rows and router rows go straight from global memory into
// XOR-swizzled LDS (global_load_lds_dwordx4) through a ring of NS stages, the copies of step
// k + NS - 1 issued right after the barrier that opens step k.  The kernel streams the tokens
// from HBM once, so its speed is set by the bytes in flight per CU: the ring depth and BM are
// chosen per expert count within the LDS (see the tile table below).
// BF16/F16 run v_mfma_f32_32x32x16; FP32 runs v_mfma_f32_32x32x2f32, full FP32 products.  The
// router fragment is the first MFMA operand, so lane l of an accumulator block holds token
// l % 32.
// Epilogue: accumulators -> LDS [WK][BM][EP] FP32; the WK slices are added in order, rounded to
// the dtype and routed, G lanes per row, in passes of 256 / G rows.
//
// Few token tiles (T / BM well below the CU count, e.g. decode) would leave most CUs idle while
// one block streams all of W_r, so K is then split over S blocks per token tile
// (projection_split): each stores FP32 partial logits [S][T][EP] in the workspace, and
// route_partials adds the S partials of each logit in a fixed order (deterministic), rounds and
// routes.
//
// HBM traffic per token row: H * sizeof(dtype) read (W_r, E * H elements, is read once per
// block from L2), k * (4 + sizeof(dtype)) written, plus E * sizeof(dtype) for the optional
// logits copy; the split adds 2 * S * EP * 4 bytes of partials.
#include <algorithm>

#include "device.hpp"
#include "internal.hpp"
#include "route_select.hpp"

namespace rudnn {
namespace proj {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int ROWB = 128;           // bytes of one staged row (K step)
constexpr int REDUCE_THREADS = 1024;  // route_partials

// Chunk c (16 bytes) of staged row r sits at slot c ^ swz(r): the MFMA operand reads (one chunk
// from each of 32 consecutive rows) then spread over all LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier of the copy ring.  __syncthreads() would also wait for every outstanding
// global->LDS copy of this wavefront (its release fence covers global memory), draining the
// ring at each step; here the caller first waits for the copies it needs (wait_vmcnt), this
// waits for the wavefront's own LDS accesses, and the "memory" clobber keeps the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte chunk of K per lane: the MFMA step(s) over it.  16-bit types: one 32x32x16 step
// (lane half h holds K elements 8h .. 8h + 7 of the 16).  FP32: four 32x32x2 steps, step q
// taking element q of each lane half's chunk -- a fixed assignment of K elements to steps
// that both operands share, so the dot products are the same.
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
struct Mma<float> {
    typedef float4 frag;
    static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, c, 0, 0, 0);
    }
};

template <typename T>
__device__ __forceinline__ typename RouteBits<T>::raw bits_of(float v) {
    const T t = from_f32<T>(v);
    typename RouteBits<T>::raw b;
    __builtin_memcpy(&b, &t, sizeof(b));
    return b;
}

// This lane's NPER rounded logits of one row (experts e0 ..) to out_row; entries at e >= E are
// not stored.
template <typename T, int NPER>
__device__ __forceinline__ void store_logits(T* out_row, int e0, int E, const typename RouteBits<T>::raw (&raw)[NPER]) {
    typedef typename RouteBits<T>::raw R;
    if (e0 >= E) return;
    R* o = reinterpret_cast<R*>(out_row) + e0;
    constexpr int PER16 = 16 / (int)sizeof(R);
    static_assert(NPER % PER16 == 0, "whole 16-byte pieces per lane");
    if (e0 + NPER <= E && ((uintptr_t)o % 16) == 0) {
#pragma unroll
        for (int c = 0; c < NPER / PER16; ++c) {
            uint4 q;
            __builtin_memcpy(&q, raw + c * PER16, 16);
            *reinterpret_cast<uint4*>(o + c * PER16) = q;
        }
    } else {
#pragma unroll
        for (int s = 0; s < NPER; ++s)
            if (e0 + s < E) o[s] = raw[s];
    }
}

// One staged K step: BM token rows then EP router rows, 128 bytes each, as 1 KiB wave copies
// of 8 rows (lane i writes 16 bytes at the copy's LDS base + 16 i), dealt to the wavefronts
// round-robin, SLOTS copies per wavefront (the ring's waits count them, so every whole step
// issues exactly that many).  Token rows past the tile's last re-read its last row and router
// rows past E re-read row E - 1 (outputs of those rows are never used).  TAIL: chunks at or past
// the row's end (K not a multiple of the step) are zeroed in both operands instead.
template <int BM, int EP, int NWAVES, bool TAIL>
__device__ __forceinline__ void stage(unsigned char* st, const unsigned char* xa, const unsigned char* wa, int nrows,
                                      int E, int kbytes, int k0, int wave, int lane) {
    constexpr int GA = BM / 8, GB = EP / 8, SLOTS = (GA + GB) / NWAVES;
    static_assert((GA + GB) % NWAVES == 0, "copies split evenly over the wavefronts");
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
        const int gi = wave + q * NWAVES;  // wave-uniform
        const unsigned char* base;
        int r, last;
        if (gi < GA) {
            base = xa, r = gi * 8 + lane / 8, last = nrows - 1;
        } else {
            base = wa, r = (gi - GA) * 8 + lane / 8, last = E - 1;
        }
        const int kk = k0 + ((lane & 7) ^ swz(r)) * 16;
        const int rr = r < last ? r : last;
        unsigned char* dst = st + gi * 1024;
        if (!TAIL || kk < kbytes)
            __builtin_amdgcn_global_load_lds((const void*)(base + (uint32_t)(rr * kbytes + kk)),
                                             (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        else
            *reinterpret_cast<uint4*>(dst + lane * 16) = make_uint4(0, 0, 0, 0);
    }
}

template <int EP_, int WM_, int WN_, int WK_, int NS_>
struct Cfg {
    static constexpr int EP = EP_, WM = WM_, WN = WN_, WK = WK_, NS = NS_;
    static constexpr int NWAVES = WM * WN * WK, THREADS = NWAVES * 64;
    static constexpr int BM = WM * 32, WTN = EP / WN, FN = WTN / 32;
    static constexpr int STAGE = (BM + EP) * ROWB;
    static constexpr int SLOTS = (BM + EP) / 8 / NWAVES;     // copies per wavefront per step
    static constexpr int RP = EP + 4;                        // FP32 row pitch of the reduce tile
    static constexpr int RED = WK * BM * RP * 4;             // bytes of the reduce tile
    static_assert(NWAVES == 4 || NWAVES == 8, "four or eight wavefronts");
    static_assert(EP % (32 * WN) == 0 && 4 % WK == 0, "wave tiles of whole 32x32 blocks");
    static_assert(NS >= 2 && (NS - 2) * SLOTS <= 63, "ring waits fit the vmcnt counter");
    static_assert(NS * STAGE <= 160 * 1024, "ring fits the LDS");
};

// Projection of one token tile (or one K segment of it, S > 1) and, with S == 1, its routing.
template <typename T, typename C, int NPER, int G>
__global__ __launch_bounds__(C::THREADS) void project_route(const T* __restrict__ x, const T* __restrict__ wr,
                                                            int64_t Tn, int H, int E, int k, int renorm, int S,
                                                            int rpp, float* __restrict__ partials,
                                                            T* __restrict__ logits_out, uint32_t* __restrict__ idx,
                                                            T* __restrict__ w) {
    constexpr int EP = C::EP, WM = C::WM, WN = C::WN, WK = C::WK, NS = C::NS, NWAVES = C::NWAVES;
    constexpr int THREADS = C::THREADS, BM = C::BM, FN = C::FN, RP = C::RP, STAGE = C::STAGE;
    (void)WM;
    typedef typename RouteBits<T>::raw R;
    typedef typename Mma<T>::frag frag;
    static_assert(G * NPER <= EP, "a row's lanes stay inside the padded tile");
    extern __shared__ __align__(1024) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = wave % WK, wn = (wave / WK) % WN, wm = wave / (WK * WN);
    const int64_t mb = blockIdx.x / S;
    const int seg = (int)(blockIdx.x % S);
    const int64_t row0 = mb * BM;
    const int nrows = (int)min((int64_t)BM, Tn - row0);
    const int kbytes = H * (int)sizeof(T);
    const int KT = (kbytes + ROWB - 1) / ROWB;
    const int kb = (int)((int64_t)seg * KT / S), ke = (int)((int64_t)(seg + 1) * KT / S);
    const bool ragged = kbytes % ROWB != 0;
    const unsigned char* xa = reinterpret_cast<const unsigned char*>(x + row0 * H);
    const unsigned char* wa = reinterpret_cast<const unsigned char*>(wr);

    auto issue = [&](int kt) __attribute__((always_inline)) {
        unsigned char* st = smem + (kt % NS) * STAGE;
        if (ragged && kt == KT - 1)
            stage<BM, EP, NWAVES, true>(st, xa, wa, nrows, E, kbytes, kt * ROWB, wave, lane);
        else
            stage<BM, EP, NWAVES, false>(st, xa, wa, nrows, E, kbytes, kt * ROWB, wave, lane);
    };

    f32x16 acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

    const int fr = lane & 31, fh = lane >> 5;
    // Ring: steps kt + 1 .. kt + NS - 2 are in flight while step kt computes.  The wait before
    // step kt lets exactly the later steps' copies stay outstanding (copies complete in issue
    // order); when one of those is missing or is the ragged last step (fewer copies), it waits
    // for all.
    const int whole_end = ragged ? KT - 1 : KT;  // steps before this one issue SLOTS copies each
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (kb + s < ke) issue(kb + s);
    for (int kt = kb; kt < ke; ++kt) {
        if (NS > 2 && kt + NS - 2 < ke && kt + NS - 2 < whole_end)
            wait_vmcnt<(NS - 2) * C::SLOTS>();  // this wavefront's copies of step kt have landed
        else
            wait_vmcnt<0>();
        ring_barrier();  // everyone's have; everyone is done with step kt - 1
        if (kt + NS - 1 < ke) issue(kt + NS - 1);
        const unsigned char* st = smem + (kt % NS) * STAGE;
        const unsigned char* sx = st + (wm * 32 + fr) * ROWB;
        const unsigned char* sw = st + (BM + wn * C::WTN + fr) * ROWB;
#pragma unroll
        for (int t = 0; t < 4 / WK; ++t) {
            const int off = (((t * WK + wk) * 2 + fh) ^ swz(fr)) * 16;
            const frag fx = *reinterpret_cast<const frag*>(sx + off);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const frag fw = *reinterpret_cast<const frag*>(sw + j * 32 * ROWB + off);
                acc[j] = Mma<T>::run(fw, fx, acc[j]);
            }
        }
    }

    // Accumulators -> LDS: lane l holds token l % 32 and experts 8 (v / 4) + 4 (l / 32) + v % 4
    // of each 32x32 block, i.e. four runs of four adjacent experts.
    __syncthreads();  // the stages are free
    float* red = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int col = wn * C::WTN + j * 32 + 8 * q + 4 * fh;
            *reinterpret_cast<float4*>(red + (wk * BM + wm * 32 + fr) * RP + col) =
                make_float4(acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]);
        }
    __syncthreads();

    if (S > 1) {  // a K segment: FP32 partial logits of the tile's rows, all EP columns
        float* P = partials + ((int64_t)seg * Tn + row0) * EP;
        for (int i = tid; i < nrows * (EP / 4); i += THREADS) {
            const int r = i / (EP / 4), c = (i % (EP / 4)) * 4;
            float4 v = *reinterpret_cast<const float4*>(red + r * RP + c);
#pragma unroll
            for (int s = 1; s < WK; ++s) {
                const float4 u = *reinterpret_cast<const float4*>(red + (s * BM + r) * RP + c);
                v.x += u.x, v.y += u.y, v.z += u.z, v.w += u.w;
            }
            *reinterpret_cast<float4*>(P + (int64_t)r * EP + c) = v;
        }
        return;
    }

    // Routing, G lanes per row, rpp <= THREADS / G rows per pass (the LDS after the reduce tile
    // holds rpp rows of selection scratch).
    const int rb = tid / G, e0 = (lane % G) * NPER;
    const bool active = rb < rpp;
    uint32_t* si = reinterpret_cast<uint32_t*>(smem + C::RED) + (active ? rb : 0) * k;
    float* se = reinterpret_cast<float*>(smem + C::RED) + rpp * k + (active ? rb : 0) * k;
    for (int p = 0; p < BM; p += rpp) {
        const int r = p + rb;
        const bool live = active && r < nrows;
        const float* rr = red + (r < BM ? r : 0) * RP + e0;
        R raw[NPER];
#pragma unroll
        for (int s = 0; s < NPER; ++s) {
            float v = rr[s];
#pragma unroll
            for (int q = 1; q < WK; ++q) v += rr[q * BM * RP + s];
            raw[s] = bits_of<T>(v);
        }
        if (logits_out && live) store_logits<T, NPER>(logits_out + (row0 + r) * E, e0, E, raw);
        route_row<T, NPER, G>(raw, E, k, renorm, live, row0 + r, si, se, idx, w);
        __syncthreads();  // the pass's LDS scratch is read before the next pass writes it
    }
}

// The S partial logits of each row added, rounded, stored (optional) and routed.  A block of
// 1024 threads owns RB rows: thread (part p, row r, column quad c) adds slabs
// [p S / PP, (p + 1) S / PP) of its four logits in slab order (eight slabs loaded ahead), the
// part-0 thread of each column quad then adds the other parts in part order through LDS -- a
// fixed order for given T, H and E -- and G lanes per row route as in the softmax router.  C4 * RB * PP = 1024 with C4 = EP / 4.
template <typename T, int NPER, int G>
__global__ __launch_bounds__(REDUCE_THREADS) void route_partials(const float* __restrict__ P, int64_t Tn, int EP,
                                                                 int S, int PP, int RB, int E, int k, int renorm,
                                                                 T* __restrict__ logits_out,
                                                                 uint32_t* __restrict__ idx, T* __restrict__ w) {
    typedef typename RouteBits<T>::raw R;
    extern __shared__ __align__(16) float sm[];  // sums [PP][RB][EP], then [RB][k] winner ids, [RB][k] e_j
    constexpr int AHEAD = 8;
    const int tid = threadIdx.x, C4 = EP / 4;
    const int c = tid % C4, r = (tid / C4) % RB, p = tid / (C4 * RB);
    const int64_t row0 = (int64_t)blockIdx.x * RB;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + r < Tn) {
        const int s0 = (int)((int64_t)p * S / PP), s1 = (int)((int64_t)(p + 1) * S / PP);
        const float* p0 = P + (row0 + r) * EP + 4 * c;
        const int64_t slab = Tn * EP;
        for (int sg = s0; sg < s1; sg += AHEAD) {
            float4 q[AHEAD];
#pragma unroll
            for (int a = 0; a < AHEAD; ++a)
                if (sg + a < s1) q[a] = *reinterpret_cast<const float4*>(p0 + (sg + a) * slab);
#pragma unroll
            for (int a = 0; a < AHEAD; ++a)
                if (sg + a < s1) acc.x += q[a].x, acc.y += q[a].y, acc.z += q[a].z, acc.w += q[a].w;
        }
    }
    float4* sm4 = reinterpret_cast<float4*>(sm);
    sm4[(p * RB + r) * (EP / 4) + c] = acc;
    __syncthreads();
    if (p == 0) {  // the parts, in part order, into part 0's slot
        for (int q = 1; q < PP; ++q) {
            const float4 u = sm4[(q * RB + r) * (EP / 4) + c];
            acc.x += u.x, acc.y += u.y, acc.z += u.z, acc.w += u.w;
        }
        sm4[r * (EP / 4) + c] = acc;
    }
    __syncthreads();

    const int rb = tid / G, e0 = (lane_id() % G) * NPER;
    const int64_t row = row0 + rb;
    const bool live = rb < RB && row < Tn;
    R raw[NPER];
#pragma unroll
    for (int s = 0; s < NPER; ++s) raw[s] = bits_of<T>(rb < RB ? sm[rb * EP + e0 + s] : 0.f);
    if (logits_out && live) store_logits<T, NPER>(logits_out + row * E, e0, E, raw);
    float* scratch = sm + PP * RB * EP;
    const int sr = rb < RB ? rb : 0;
    route_row<T, NPER, G>(raw, E, k, renorm, live, row, reinterpret_cast<uint32_t*>(scratch) + sr * k,
                          scratch + RB * k + sr * k, idx, w);
}

}  // namespace proj

// ---- host side ----

// Tile shape per expert count: EP, WM, WN, WK, NS (see project_route), the fastest of a sweep on
// the Mixtral-, fine-grained- and 256-expert shapes: E <= 32: 64-token tiles, a 6-step ring, two
// blocks per CU; E <= 64: 64-token tiles, 5 steps, two blocks; E <= 128: 256-token tiles of
// eight wavefronts, 3 steps; E <= 256: 128-token tiles of eight wavefronts, 3 steps.
#ifndef RUDNN_PROJ_E32
#define RUDNN_PROJ_E32 32, 2, 1, 2, 6
#endif
#ifndef RUDNN_PROJ_E64
#define RUDNN_PROJ_E64 64, 2, 1, 2, 5
#endif
#ifndef RUDNN_PROJ_E128
#define RUDNN_PROJ_E128 128, 8, 1, 1, 3
#endif
#ifndef RUDNN_PROJ_E256
#define RUDNN_PROJ_E256 256, 4, 2, 1, 3
#endif
typedef proj::Cfg<RUDNN_PROJ_E32> CfgE32;
typedef proj::Cfg<RUDNN_PROJ_E64> CfgE64;
typedef proj::Cfg<RUDNN_PROJ_E128> CfgE128;
typedef proj::Cfg<RUDNN_PROJ_E256> CfgE256;
static_assert(CfgE32::EP == 32 && CfgE64::EP == 64 && CfgE128::EP == 128 && CfgE256::EP == 256, "expert classes");

namespace {

int64_t padded_experts(int64_t E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }
int64_t block_rows(int64_t E) {
    return E <= 32 ? CfgE32::BM : E <= 64 ? CfgE64::BM : E <= 128 ? CfgE128::BM : CfgE256::BM;
}

constexpr int64_t SPLIT_TARGET_BLOCKS = 256;  // blocks the K split aims for (about one per CU)
constexpr size_t k_max_scratch_rows = 8;       // a routing pass holds at least this many rows at top_k = 64
constexpr int64_t MAX_SPLIT = 64;

}  // namespace

int64_t projection_split(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dt) {
    const int64_t mblocks = (T + block_rows(E) - 1) / block_rows(E);
    const int64_t KT = (H * (int64_t)dtype_size(dt) + proj::ROWB - 1) / proj::ROWB;
    if (mblocks <= 0 || mblocks * 2 > SPLIT_TARGET_BLOCKS) return 1;
    int64_t S = (SPLIT_TARGET_BLOCKS + mblocks - 1) / mblocks;
    S = std::min(S, std::min(MAX_SPLIT, KT / 2));  // each segment at least two K steps
    return S < 2 ? 1 : S;
}

size_t projection_workspace_bytes(int64_t T, int64_t H, int64_t E, rudnn_moe_dtype dt) {
    const int64_t S = projection_split(T, H, E, dt);
    return S > 1 ? align_up((size_t)(S * T * padded_experts(E)) * 4) : 0;
}

namespace {

template <typename T, typename C, int NPER, int G>
hipError_t go(const T* x, const T* wr, int64_t Tn, int64_t H, int64_t E, int64_t k, bool renorm, T* logits_out,
              uint32_t* idx, T* w, float* partials, int64_t S, hipStream_t s) {
    constexpr int RPB = C::THREADS / G;
    static_assert(proj::REDUCE_THREADS % (C::EP / 4) == 0, "column quads tile the reduce block");
    static const hipError_t attr = hipFuncSetAttribute((const void*)proj::project_route<T, C, NPER, G>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)attr;
    const int64_t mblocks = (Tn + C::BM - 1) / C::BM;
    // routing rows per pass: all groups, unless their scratch would not fit beside the reduce tile
    constexpr size_t LDS = 160 * 1024;
    static_assert((size_t)C::RED + (size_t)k_max_scratch_rows * 8 * 64 <= LDS, "room for a routing pass");
    const int64_t rpp = std::min((int64_t)RPB, (int64_t)((LDS - (size_t)C::RED) / ((size_t)k * 8)));
    const size_t smem = std::max((size_t)C::NS * C::STAGE, (size_t)C::RED + (S > 1 ? 0 : (size_t)rpp * k * 8));
    timing_before(RUDNN_MOE_KERNEL_ROUTE_PROJECTED, s);
    proj::project_route<T, C, NPER, G><<<dim3((unsigned)(mblocks * S)), dim3(C::THREADS), smem, s>>>(
        x, wr, Tn, (int)H, (int)E, (int)k, renorm ? 1 : 0, (int)S, (int)rpp, partials, logits_out, idx, w);
    timing_after(RUDNN_MOE_KERNEL_ROUTE_PROJECTED, s);
    if (S > 1) {
        // PP: a power of two <= min(S, 1024 / C4) parts per column quad; RB rows per block
        constexpr int C4 = C::EP / 4;
        int PP = 1;
        while (PP * 2 <= S && PP * 2 <= proj::REDUCE_THREADS / C4) PP *= 2;
        const int RB = proj::REDUCE_THREADS / (C4 * PP);
        const size_t rsmem = ((size_t)PP * RB * C::EP + (size_t)RB * k * 2) * 4;
        timing_before(RUDNN_MOE_KERNEL_ROUTE_PROJECTED_REDUCE, s);
        proj::route_partials<T, NPER, G><<<dim3((unsigned)((Tn + RB - 1) / RB)), dim3(proj::REDUCE_THREADS), rsmem, s>>>(
            partials, Tn, C::EP, (int)S, PP, RB, (int)E, (int)k, renorm ? 1 : 0, logits_out, idx, w);
        timing_after(RUDNN_MOE_KERNEL_ROUTE_PROJECTED_REDUCE, s);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void* xv, const void* wv, int64_t Tn, int64_t H, int64_t E, int64_t k, bool renorm,
                    void* lo, uint32_t* idx, void* wo, float* partials, int64_t S, hipStream_t s) {
    const T* x = (const T*)xv;
    const T* wr = (const T*)wv;
    T* logits_out = (T*)lo;
    T* w = (T*)wo;
    // lanes per row as in the softmax router: the smallest power of two G with G * 16 >= E
    if (E <= 8) return go<T, CfgE32, 8, 1>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 16) return go<T, CfgE32, 16, 1>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 32) return go<T, CfgE32, 16, 2>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 64) return go<T, CfgE64, 16, 4>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 128) return go<T, CfgE128, 16, 8>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    return go<T, CfgE256, 16, 16>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
}

}  // namespace

hipError_t launch_route_projected(const void* x, rudnn_moe_dtype dt, const void* router, int64_t T, int64_t H,
                                  int64_t E, int64_t k, bool renorm, void* logits_out, uint32_t* idx, void* w,
                                  void* workspace, hipStream_t s) {
    const int64_t S = projection_split(T, H, E, dt);
    float* partials = (float*)workspace;
    switch (dt) {
    case RUDNN_MOE_F32: return launch_t<float>(x, router, T, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    case RUDNN_MOE_F16: return launch_t<f16>(x, router, T, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    default: return launch_t<bf16>(x, router, T, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    }
}

}  // namespace rudnn
