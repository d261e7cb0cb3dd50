// router.hip -- linear router scores with the top-k fused behind them (moe_router_topk).
//
// The TritonMoE abstract (Daily Papers listing): the forward pass starts with router scoring,
// fused with what follows.  A linear router scores token t against expert e with the dot
// product of x[t] and the router row W_r[e]; MegaFlux §1: the k best-scoring experts take the
// token, mixed by routing weights; the top-k renormalisation abstract: the weights are the
// picks' probabilities over the mass of a reference set (moe_topk.h).
//
// bf16: one workgroup (4 waves; 8 for 128-token tiles) per tile of TM tokens against all E
// router rows, E <= 32 NB.
// K (= H) is staged in 64-wide slices (128-byte rows) through an LDS ring of up to 8 stages
// filled by gfx950 direct-to-LDS copies (a stage holds the TM token rows and the 32 NB router
// rows); v_mfma_f32_32x32x16_bf16 accumulates the [TM, 32 NB] scores in float32, each wave
// taking all TM rows against every W-th 32-row router block for W waves (with 4 waves a k-step
// reads TM/32 + NB/4 fragments per wave, not 1 + TM NB / 128 as with one row block per wave).
// At 128 tokens x 256 experts the staging bounds the kernel; 8 waves, two per SIMD, keep more
// copies in flight than 4 and were 7.5% faster there.  The score tile is then written to LDS
// (and to `logits` if asked) and each token's top-k is taken from it by 64 W / TM lanes.
// float32: the same tile flow with scalar FMAs (256 threads).  The histogram is kept in LDS and
// flushed with one atomic per nonzero bin; at most 256 workgroups.
#include "moe_launch.h"
#include "moe_lds.h"
#include "moe_topk.h"

namespace {

constexpr int kF32Threads = 256;  // the float32 kernel's workgroup
constexpr int kMaxBlocks = 256;
constexpr int kRingBytes = 144 * 1024;

template <int TM, int NB, int W = 4>
struct Geom {
    static constexpr int kThr = W * 64;                       // threads
    static constexpr int kRowsB = NB * 32;                    // router rows per stage
    static constexpr int kSegs = (TM + kRowsB) / 8;           // 1 KB segments per stage
    static constexpr int kCPW = kSegs / W;                    // copies per wave per stage
    static constexpr int kStageBytes = kSegs * 1024;
    static constexpr int kStagesFit = kRingBytes / kStageBytes;
    static constexpr int kStages = kStagesFit < 8 ? kStagesFit : 8;
    static constexpr int kRB = TM / 32;                       // 32-row blocks
    static constexpr int kCBW = (NB + W - 1) / W;             // column blocks per wave
    static constexpr int kLPT = kThr / TM;                    // top-k lanes per token
    static constexpr int kNE = kRowsB / kLPT;                 // experts per top-k lane
    static constexpr int kLdS = kRowsB + 1;                   // score tile row stride (floats)
    static constexpr int kScoreBytes = TM * kLdS * 4;
    // LDS: the ring, reused for the score tile once the slices are consumed
    static constexpr int kSmem = kStages * kStageBytes > kScoreBytes ? kStages * kStageBytes
                                                                     : kScoreBytes;
    static_assert(kSegs % W == 0, "whole copies per wave");
    static_assert(kStages >= 2, "ring depth");
    static_assert(kSmem <= 144 * 1024, "LDS");
};

// Stage layout: segment g (8 rows of 128 bytes) at g KB; segments 0 .. TM/8 - 1 hold token
// rows 0 .. TM - 1, the rest hold router rows.  Within each side row r's 16-byte chunk c sits
// at physical chunk swz_chunk(r, c).
template <int TM>
__device__ __forceinline__ bf16x8_t stage_frag(const uint8_t* stage, int row, bool router,
                                               int ch) {
    const int seg = (router ? TM / 8 : 0) + (row >> 3);
    const uint4 v = *reinterpret_cast<const uint4*>(stage + seg * 1024 + (row & 7) * 128 +
                                                    (swz_chunk(row, ch) << 4));
    return __builtin_bit_cast(bf16x8_t, v);
}

template <int TM, int NB, int KM, int W = 4>
__global__ void __launch_bounds__(W * 64, 1)
router_bf16_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H,
                   int E, int K, int k_ref, float* __restrict__ logits,
                   int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                   int32_t* __restrict__ counts) {
    using G = Geom<TM, NB, W>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::kSmem];
    __shared__ int hist[256];
    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    for (int e = tid; e < E; e += G::kThr) hist[e] = 0;

    const int nk = H / 64;
    const int seg_row = lane >> 3;
    const int seg_lchunk = swz_chunk((wave & 1) * 8 + seg_row, lane & 7);
    const int ntiles = (T + TM - 1) / TM;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int t0 = tile * TM;
        // copy q of this wave fills segment wave + W q; lane offsets from the side's base
        uint32_t off[G::kCPW];
        bool on_router[G::kCPW];
#pragma unroll
        for (int q = 0; q < G::kCPW; ++q) {
            const int g = wave + W * q;
            on_router[q] = g >= TM / 8;
            int r = (on_router[q] ? g - TM / 8 : g) * 8 + seg_row;
            if (on_router[q])
                r = r < E ? r : E - 1;  // rows past E: read, unused
            else
                r = t0 + r < T ? t0 + r : T - 1;  // tokens past T: read, unused
            off[q] = (uint32_t)r * (uint32_t)H * 2u + seg_lchunk * 16u;
        }
        auto issue = [&](int kt) {
            const uint32_t st = smem_base + (kt % G::kStages) * G::kStageBytes;
            const uint32_t koff = (uint32_t)kt * 128u;
#pragma unroll
            for (int q = 0; q < G::kCPW; ++q)
                one_copy(st + (wave + W * q) * 1024, on_router[q] ? (const void*)wr : (const void*)x,
                         off[q] + koff);
        };

        // wave w: every row block, column blocks w, w + W, ...  Blocks past NB read router
        // block 0 and are never stored; their MFMAs run anyway, since a branch around an MFMA
        // makes the compiler move its accumulators between register files at every slice
        f32x16_t acc[G::kRB][G::kCBW];
#pragma unroll
        for (int i = 0; i < G::kRB; ++i)
#pragma unroll
            for (int c = 0; c < G::kCBW; ++c)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.f;
        bf16x8_t fa[2][G::kRB], fb[2][G::kCBW];
        auto load_frags = [&](int kt, int kk, int buf) {
            const uint8_t* st = smem + (kt % G::kStages) * G::kStageBytes;
            const int ch = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < G::kRB; ++i)
                fa[buf][i] = stage_frag<TM>(st, i * 32 + (lane & 31), false, ch);
#pragma unroll
            for (int c = 0; c < G::kCBW; ++c) {
                const int cb = wave + W * c;
                fb[buf][c] = stage_frag<TM>(st, (cb < NB ? cb : 0) * 32 + (lane & 31), true, ch);
            }
        };

        __syncthreads();  // the previous tile's LDS reads are done
        const int pre = nk < G::kStages ? nk : G::kStages;
        for (int s = 0; s < pre; ++s) issue(s);
        wait_pending_stages<G::kCPW, G::kStages - 1>(pre - 1);
        load_frags(0, 0, 0);
        for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int cur = kk & 1;
                if (kk + 1 < 4) load_frags(kt, kk + 1, cur ^ 1);
#pragma unroll
                for (int c = 0; c < G::kCBW; ++c)
#pragma unroll
                    for (int i = 0; i < G::kRB; ++i)
                        acc[i][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][c],
                                                                            acc[i][c], 0, 0, 0);
                if (kk == 3 && kt + 1 < nk) {
                    const int issued = kt + G::kStages - 1 < nk ? kt + G::kStages - 1 : nk - 1;
                    wait_pending_stages<G::kCPW, G::kStages - 1>(issued - (kt + 1));
                    if (kt + G::kStages < nk) issue(kt + G::kStages);
                    load_frags(kt + 1, 0, cur ^ 1);
                }
            }
        }

        // scores: acc[i][c][r] = S[row 32 i + 8(r/4) + 4(lane/32) + r%4][col 32 (wave + W c) + lane%32]
        __syncthreads();  // every wave is done with the ring
        float* sc = reinterpret_cast<float*>(smem);
#pragma unroll
        for (int c = 0; c < G::kCBW; ++c) {
            if (wave + W * c >= NB) continue;
            const int col = (wave + W * c) * 32 + (lane & 31);
#pragma unroll
            for (int i = 0; i < G::kRB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                    sc[row * G::kLdS + col] = acc[i][c][r];
                    if (logits && col < E && t0 + row < T) logits[(int64_t)(t0 + row) * E + col] = acc[i][c][r];
                }
        }
        __syncthreads();
        const int slot = tid / G::kLPT, q = tid % G::kLPT;
        moe_topk::topk_token<G::kLPT, G::kNE, KM>(sc + slot * G::kLdS, t0 + slot, t0 + slot < T,
                                                  E, K, k_ref, q, topk_ids, topk_w, hist);
    }
    __syncthreads();
    for (int e = tid; e < E; e += G::kThr) {
        const int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

// float32 router: the same tile flow; the score tile [TM = 64, 32 NB] is accumulated from K
// slices of 32 staged in LDS, thread (token row tid / 4, experts tid % 4 + 4 m).
template <int NB, int KM>
__global__ void __launch_bounds__(kF32Threads)
router_f32_kernel(const float* __restrict__ x, const float* __restrict__ wr, int T, int H, int E,
                  int K, int k_ref, float* __restrict__ logits, int32_t* __restrict__ topk_ids,
                  float* __restrict__ topk_w, int32_t* __restrict__ counts) {
    constexpr int TM = 64, TK = 32, RB = NB * 32, NPT = RB / 4, LDS_ = RB + 1;
    __shared__ float xs[TM][TK + 1];
    __shared__ float ws[RB][TK + 1];
    __shared__ float sc[TM * LDS_];
    __shared__ int hist[256];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kF32Threads) hist[e] = 0;
    const int ntiles = (T + TM - 1) / TM;
    const int r = tid / 4, eq = tid % 4;
    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int t0 = tile * TM;
        float acc[NPT];
#pragma unroll
        for (int m = 0; m < NPT; ++m) acc[m] = 0.f;
        for (int k0 = 0; k0 < H; k0 += TK) {
            __syncthreads();
            for (int i = tid; i < TM * TK; i += kF32Threads) {
                const int rr = i / TK, kk = i % TK;
                xs[rr][kk] = (t0 + rr < T && k0 + kk < H) ? x[(int64_t)(t0 + rr) * H + k0 + kk] : 0.f;
            }
            for (int i = tid; i < RB * TK; i += kF32Threads) {
                const int e = i / TK, kk = i % TK;
                ws[e][kk] = (e < E && k0 + kk < H) ? wr[(int64_t)e * H + k0 + kk] : 0.f;
            }
            __syncthreads();
            const int kn = H - k0 < TK ? H - k0 : TK;
            for (int kk = 0; kk < kn; ++kk) {
                const float xv = xs[r][kk];
#pragma unroll
                for (int m = 0; m < NPT; ++m) acc[m] = fmaf(xv, ws[eq + 4 * m][kk], acc[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < NPT; ++m) {
            const int e = eq + 4 * m;
            sc[r * LDS_ + e] = acc[m];
            if (logits && e < E && t0 + r < T) logits[(int64_t)(t0 + r) * E + e] = acc[m];
        }
        __syncthreads();
        moe_topk::topk_token<4, RB / 4, KM>(sc + r * LDS_, t0 + r, t0 + r < T, E, K, k_ref, eq,
                                            topk_ids, topk_w, hist);
        __syncthreads();
    }
    for (int e = tid; e < E; e += kF32Threads) {
        const int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

template <int TM, int NB, int W = 4>
hipError_t launch_bf16(int km, const uint16_t* x, const uint16_t* wr, int T, int H, int E, int K,
                       int k_ref, float* logits, int32_t* ids, float* w, int32_t* counts,
                       hipStream_t stream) {
    const int tiles = (T + TM - 1) / TM;
    const int grid = tiles < kMaxBlocks ? tiles : kMaxBlocks;
    if (km <= 4)
        router_bf16_kernel<TM, NB, 4, W><<<grid, W * 64, 0, stream>>>(x, wr, T, H, E, K, k_ref,
                                                                     logits, ids, w, counts);
    else if (km <= 8)
        router_bf16_kernel<TM, NB, 8, W><<<grid, W * 64, 0, stream>>>(x, wr, T, H, E, K, k_ref,
                                                                     logits, ids, w, counts);
    else
        router_bf16_kernel<TM, NB, 16, W><<<grid, W * 64, 0, stream>>>(x, wr, T, H, E, K, k_ref,
                                                                      logits, ids, w, counts);
    return hipGetLastError();
}

// 128-token tiles (E > 128 only): the router rows are staged once per 128 tokens; 8 waves
hipError_t launch_tm128(int km, const uint16_t* x, const uint16_t* wr, int T, int H, int E, int K,
                        int k_ref, float* logits, int32_t* ids, float* w, int32_t* counts,
                        hipStream_t stream) {
    if ((E + 31) / 32 <= 6)
        return launch_bf16<128, 6, 8>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
    return launch_bf16<128, 8, 8>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
}

template <int TM>
hipError_t launch_tm(int km, const uint16_t* x, const uint16_t* wr, int T, int H, int E, int K,
                     int k_ref, float* logits, int32_t* ids, float* w, int32_t* counts,
                     hipStream_t stream) {
    const int nb = (E + 31) / 32;
    if (nb <= 1) return launch_bf16<TM, 1>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
    if (nb <= 2) return launch_bf16<TM, 2>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
    if (nb <= 4) return launch_bf16<TM, 4>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
    return launch_bf16<TM, 8>(km, x, wr, T, H, E, K, k_ref, logits, ids, w, counts, stream);
}

template <int NB>
hipError_t launch_f32(int km, const float* x, const float* wr, int T, int H, int E, int K,
                      int k_ref, float* logits, int32_t* ids, float* w, int32_t* counts,
                      hipStream_t stream) {
    const int tiles = (T + 63) / 64;
    const int grid = tiles < kMaxBlocks ? tiles : kMaxBlocks;
    if (km <= 4)
        router_f32_kernel<NB, 4><<<grid, kF32Threads, 0, stream>>>(x, wr, T, H, E, K, k_ref, logits,
                                                               ids, w, counts);
    else if (km <= 8)
        router_f32_kernel<NB, 8><<<grid, kF32Threads, 0, stream>>>(x, wr, T, H, E, K, k_ref, logits,
                                                               ids, w, counts);
    else
        router_f32_kernel<NB, 16><<<grid, kF32Threads, 0, stream>>>(x, wr, T, H, E, K, k_ref, logits,
                                                                ids, w, counts);
    return hipGetLastError();
}

}  // namespace

hipError_t moe_launch_router_topk(const void* x, moe_dtype_t dt, const void* w_router, int T,
                                  int H, int E, int K, int k_ref, float* logits,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  hipStream_t stream) {
    hipError_t err = moe_launch_zero_counts(counts, E, stream);
    if (err != hipSuccess) return err;
    const int km = k_ref < E && k_ref > K ? k_ref : K;  // list length the weights need
    if (dt == MOE_F32) {
        const float* xf = static_cast<const float*>(x);
        const float* wf = static_cast<const float*>(w_router);
        const int nb = (E + 31) / 32;
        if (nb <= 1) return launch_f32<1>(km, xf, wf, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
        if (nb <= 2) return launch_f32<2>(km, xf, wf, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
        if (nb <= 4) return launch_f32<4>(km, xf, wf, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
        return launch_f32<8>(km, xf, wf, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
    }
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* wb = static_cast<const uint16_t*>(w_router);
    // the largest token tile that still gives every CU one (128 only pays for E > 128, where
    // router rows dominate the staging), else 32
    if (E > 128 && (T + 127) / 128 >= 256)
        return launch_tm128(km, xb, wb, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
    if ((T + 63) / 64 >= 256)
        return launch_tm<64>(km, xb, wb, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
    return launch_tm<32>(km, xb, wb, T, H, E, K, k_ref, logits, topk_ids, topk_w, counts, stream);
}
