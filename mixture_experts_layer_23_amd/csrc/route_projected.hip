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
// of 32).  Its four wavefronts split the tile WM x WN x WK ways: WM bands of 32 tokens, WN bands
// of EP / WN experts, WK interleaved quarters of each staged K step (WK > 1 when E is small, so
// that all four SIMDs work on a 32-token tile).  The K axis is staged 128 bytes at a time
// (64 16-bit or 32 FP32 elements): token rows and router rows go straight from global memory
// into XOR-swizzled LDS (global_load_lds_dwordx4), two stages, the copies of step k+1 issued
// right after the barrier that opens step k.  BF16/F16 run v_mfma_f32_32x32x16; FP32 runs
// v_mfma_f32_32x32x2f32, full FP32 products.  The router fragment is the first MFMA operand, so
// lane l of an accumulator block holds token l % 32.
// Epilogue: accumulators -> LDS [WK][BM][EP] FP32; the WK slices are added in order, rounded to
// the dtype and routed, G lanes per row, in passes of 256 / G rows.
//
// Few token tiles (T / BM well below the CU count, e.g. decode) would leave most CUs idle while
// one block streams all of W_r, so K is then split over S blocks per token tile
// (projection_split): each stores FP32 partial logits [S][T][EP] in the workspace, and
// route_partials adds the S partials of each logit in segment order (deterministic), rounds
// and routes.
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

constexpr int THREADS = 256, NWAVES = 4;
constexpr int ROWB = 128;  // bytes of one staged row (K step)

// Chunk c (16 bytes) of staged row r sits at slot c ^ swz(r): the MFMA operand reads (one chunk
// from each of 32 consecutive rows) then spread over all LDS banks.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// round-robin.  Token rows past the tile's last are not copied when the whole copy lies past
// it (they only feed outputs that are never used) and re-read the last row otherwise; router
// rows past E re-read row E - 1 (logits of padding experts are never used).  TAIL: chunks at
// or past the row's end (K not a multiple of the step) are zeroed in both operands.
template <int BM, int EP, bool TAIL>
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
            if (gi * 8 > nrows - 1) continue;
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

template <int EP, int WM, int WN, int WK>
struct Cfg {
    static constexpr int BM = WM * 32, WTN = EP / WN, FN = WTN / 32;
    static constexpr int STAGE = (BM + EP) * ROWB;
    static constexpr int RP = EP + 4;                        // FP32 row pitch of the reduce tile
    static constexpr int RED = WK * BM * RP * 4;             // bytes of the reduce tile
    static_assert(WM * WN * WK == NWAVES, "four wavefronts");
    static_assert(EP % (32 * WN) == 0 && 4 % WK == 0, "wave tiles of whole 32x32 blocks");
};

// Projection of one token tile (or one K segment of it, S > 1) and, with S == 1, its routing.
template <typename T, int EP, int WM, int WN, int WK, int NPER, int G>
__global__ __launch_bounds__(THREADS) void project_route(const T* __restrict__ x, const T* __restrict__ wr,
                                                         int64_t Tn, int H, int E, int k, int renorm, int S,
                                                         float* __restrict__ partials, T* __restrict__ logits_out,
                                                         uint32_t* __restrict__ idx, T* __restrict__ w) {
    typedef Cfg<EP, WM, WN, WK> C;
    constexpr int BM = C::BM, FN = C::FN, RP = C::RP, STAGE = C::STAGE;
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
        unsigned char* st = smem + (kt & 1) * STAGE;
        if (ragged && kt == KT - 1)
            stage<BM, EP, true>(st, xa, wa, nrows, E, kbytes, kt * ROWB, wave, lane);
        else
            stage<BM, EP, false>(st, xa, wa, nrows, E, kbytes, kt * ROWB, wave, lane);
    };

    f32x16 acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;

    const int fr = lane & 31, fh = lane >> 5;
    issue(kb);
    for (int kt = kb; kt < ke; ++kt) {
        wait_vmcnt0();    // this wavefront's copies of step kt have landed
        __syncthreads();  // everyone's have; everyone is done with step kt - 1
        if (kt + 1 < ke) issue(kt + 1);
        const unsigned char* st = smem + (kt & 1) * STAGE;
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

    // Routing, G lanes per row, 256 / G rows per pass.
    constexpr int RPB = THREADS / G;
    const int rb = tid / G, e0 = (lane % G) * NPER;
    uint32_t* si = reinterpret_cast<uint32_t*>(smem + C::RED) + rb * k;
    float* se = reinterpret_cast<float*>(smem + C::RED) + RPB * k + rb * k;
    for (int p = 0; p < BM; p += RPB) {
        const int r = p + rb;
        const bool live = r < nrows;
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

// The S partial logits of each row added in segment order, rounded, stored (optional) and
// routed; G lanes per row as in the softmax router.
template <typename T, int NPER, int G>
__global__ __launch_bounds__(THREADS) void route_partials(const float* __restrict__ P, int64_t Tn, int EP, int S,
                                                          int E, int k, int renorm, T* __restrict__ logits_out,
                                                          uint32_t* __restrict__ idx, T* __restrict__ w) {
    typedef typename RouteBits<T>::raw R;
    extern __shared__ float s_sel[];  // [rows per block][k] winner ids, then [rows per block][k] e_j
    constexpr int RPB = THREADS / G;
    const int rb = threadIdx.x / G, e0 = (lane_id() % G) * NPER;
    const int64_t row = (int64_t)blockIdx.x * RPB + rb;
    const bool live = row < Tn;
    static_assert(NPER % 4 == 0, "whole float4 pieces per lane");
    float v[NPER];
#pragma unroll
    for (int s = 0; s < NPER; ++s) v[s] = 0.f;
    if (live) {
        for (int sg = 0; sg < S; ++sg) {
            const float* p = P + ((int64_t)sg * Tn + row) * EP + e0;
#pragma unroll
            for (int c = 0; c < NPER / 4; ++c) {
                const float4 q = *reinterpret_cast<const float4*>(p + 4 * c);
                v[4 * c] += q.x, v[4 * c + 1] += q.y, v[4 * c + 2] += q.z, v[4 * c + 3] += q.w;
            }
        }
    }
    R raw[NPER];
#pragma unroll
    for (int s = 0; s < NPER; ++s) raw[s] = bits_of<T>(v[s]);
    if (logits_out && live) store_logits<T, NPER>(logits_out + row * E, e0, E, raw);
    route_row<T, NPER, G>(raw, E, k, renorm, live, row, reinterpret_cast<uint32_t*>(s_sel) + rb * k,
                          s_sel + RPB * k + rb * k, idx, w);
}

}  // namespace proj

// ---- host side ----

namespace {

// Padded experts and token rows per block of the tile shape chosen for E.
int64_t padded_experts(int64_t E) { return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256; }
int64_t block_rows(int64_t E) { return E <= 64 ? 32 : 64; }

constexpr int64_t SPLIT_TARGET_BLOCKS = 256;  // blocks the K split aims for (about one per CU)
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

template <typename T, int EP, int WM, int WN, int WK, int NPER, int G>
hipError_t go(const T* x, const T* wr, int64_t Tn, int64_t H, int64_t E, int64_t k, bool renorm, T* logits_out,
              uint32_t* idx, T* w, float* partials, int64_t S, hipStream_t s) {
    typedef proj::Cfg<EP, WM, WN, WK> C;
    constexpr int RPB = proj::THREADS / G;
    static const hipError_t attr = hipFuncSetAttribute((const void*)proj::project_route<T, EP, WM, WN, WK, NPER, G>,
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    (void)attr;
    const int64_t mblocks = (Tn + C::BM - 1) / C::BM;
    const size_t smem =
        std::max((size_t)2 * C::STAGE, (size_t)C::RED + (S > 1 ? 0 : (size_t)RPB * (size_t)k * 8));
    timing_before(RUDNN_MOE_KERNEL_ROUTE_PROJECTED, s);
    proj::project_route<T, EP, WM, WN, WK, NPER, G><<<dim3((unsigned)(mblocks * S)), dim3(proj::THREADS), smem, s>>>(
        x, wr, Tn, (int)H, (int)E, (int)k, renorm ? 1 : 0, (int)S, partials, logits_out, idx, w);
    timing_after(RUDNN_MOE_KERNEL_ROUTE_PROJECTED, s);
    if (S > 1) {
        timing_before(RUDNN_MOE_KERNEL_ROUTE_PROJECTED_REDUCE, s);
        proj::route_partials<T, NPER, G><<<dim3((unsigned)((Tn + RPB - 1) / RPB)), dim3(proj::THREADS),
                                           (size_t)RPB * (size_t)k * 8, s>>>(
            partials, Tn, EP, (int)S, (int)E, (int)k, renorm ? 1 : 0, logits_out, idx, w);
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
    if (E <= 8) return go<T, 32, 1, 1, 4, 8, 1>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 16) return go<T, 32, 1, 1, 4, 16, 1>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 32) return go<T, 32, 1, 1, 4, 16, 2>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 64) return go<T, 64, 1, 2, 2, 16, 4>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    if (E <= 128) return go<T, 128, 2, 2, 1, 16, 8>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
    return go<T, 256, 2, 2, 1, 16, 16>(x, wr, Tn, H, E, k, renorm, logits_out, idx, w, partials, S, s);
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
