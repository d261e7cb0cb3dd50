// route.hip -- router top-k, routing weights and expert histogram (moe_route).
//
// MegaFlux §1: a router sends each token to k experts whose outputs are mixed by routing
// weights; §4.1: the k experts of a token are distinct.  The top-k renormalisation abstract
// (Daily Papers listing): the picked experts' probabilities are renormalised over the picks.
//
// LPT lanes per token (4, or 16 when there are too few tokens to fill the chip); the per-token
// top-k and weights are moe_topk (moe_topk.h), on rows read through the staged slices below when
// the rows fill the lanes exactly, else straight from HBM.  The expert histogram is counted in
// LDS per workgroup (integer adds: order-independent) and flushed with one global atomic per
// nonzero bin; the grid is capped at 256 workgroups so that a bin's counter takes at most 256
// of them.
#include "moe_launch.h"
#include "moe_topk.h"

namespace {

constexpr int kRouteThreads = 512;
constexpr int kMaxRouteBlocks = 256;

__global__ void __launch_bounds__(kRouteThreads)
zero_i32_kernel(int32_t* __restrict__ p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Staged reads (rows in HBM, E = LPT * NE, logits 16-byte aligned).  A wave's kTokensPerWave
// tokens are consecutive rows, one contiguous block of logits, read in kParts column slices
// (slice p: chunks [p kPiece, (p+1) kPiece) of every row, kPiece 16-byte chunks, contiguous
// within a row), all slices issued before the first is used.  Each slice goes through the
// wave's own LDS tile (one row per token, padded by kRowPad chunks so that a read's lanes spread
// over the banks) into the lanes' registers in the top-k layout (lane q of a token: chunks q,
// q + LPT, ...) and is scanned while the later slices are still arriving, so that the wave's
// compute overlaps its own reads.  Reading each token's row directly in the top-k layout gives a
// load instruction kTokensPerWave separate LPT x 16-byte pieces, which HBM delivers far slower.
// A wave's own LDS reads and writes execute in order, so the tile needs no barrier.
template <int LPT, int NE, int KM>
struct Staged {
    static constexpr int kTokensPerWave = MOE_WAVE / LPT;
    static constexpr int kCpr = LPT * NE / 4;  // 16-byte chunks per row
    static constexpr int kGroups = NE / moe_topk::group_size<KM, NE>();
    static constexpr int kParts = kGroups >= 4 ? 4 : kGroups;
    static constexpr int kPiece = kCpr / kParts;
    static constexpr int kLoads = kTokensPerWave * kPiece / MOE_WAVE;  // per slice
    static constexpr int kRowPad = 4;
    static constexpr int kRow = kCpr + kRowPad;
};

// LPT: lanes per token; NE: experts per lane (E <= LPT * NE); KM: list length, a power of
// two with K <= KM and (k_ref <= KM or k_ref >= E).  kStaged: the staged reads above.
template <int LPT, int NE, int KM, bool kStaged>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const float* __restrict__ logits, int T, int E, int K, int k_ref,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
             int32_t* __restrict__ counts) {
    using S = Staged<LPT, NE, KM>;
    static_assert(!kStaged || (NE % 4 == 0 && S::kParts <= 4 &&
                               S::kLoads * MOE_WAVE == S::kTokensPerWave * S::kPiece &&
                               (S::kPiece & (S::kPiece - 1)) == 0),
                  "whole power-of-two slices");
    constexpr int kTokensPerWave = MOE_WAVE / LPT;
    constexpr int kWaves = kRouteThreads / MOE_WAVE;
    __shared__ int hist[256];
    __shared__ __attribute__((aligned(16))) f32x4_t tile[kStaged ? kWaves * kTokensPerWave * S::kRow : 1];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();

    const int lane = moe_lane_id();
    const int q = lane & (LPT - 1);
    const int slot = lane / LPT;
    const int wave = threadIdx.x / MOE_WAVE;
    const int waves_total = gridDim.x * kWaves;
    const int wave_global = blockIdx.x * kWaves + wave;

    for (int t0 = wave_global * kTokensPerWave; t0 < T; t0 += waves_total * kTokensPerWave) {
        const int t = t0 + slot;
        const bool valid = t < T;
        if constexpr (kStaged) {
            const f32x4_t* src = reinterpret_cast<const f32x4_t*>(logits);
            const bool whole = t0 + kTokensPerWave <= T;  // wave-uniform
            f32x4_t x[S::kParts * S::kLoads];             // slice-major, issued in that order
#pragma unroll
            for (int k = 0; k < S::kParts * S::kLoads; ++k) {
                const int p = k / S::kLoads, f = (k % S::kLoads) * MOE_WAVE + lane;
                int row = t0 + f / S::kPiece;
                if (!whole) row = row < T ? row : T - 1;  // rows past T read the last row
                x[k] = src[(int64_t)row * S::kCpr + p * S::kPiece + f % S::kPiece];
                if ((k + 1) % S::kLoads == 0) __builtin_amdgcn_sched_barrier(0);  // slice order
            }
            f32x4_t* my_tile = tile + wave * kTokensPerWave * S::kRow;
            float v[NE];
            double list[KM];
            // slice P: its loads into the tile, the lane's chunks of the slice into v, their
            // keys into list; the next slice's wait for its loads stays behind this slice's
            // compute
#define MOE_ROUTE_SLICE(P)                                                                     \
    if constexpr (S::kParts > P) {                                                             \
        _Pragma("unroll") for (int i = 0; i < S::kLoads; ++i) {                                \
            const int f = i * MOE_WAVE + lane;                                                 \
            my_tile[(f / S::kPiece) * S::kRow + P * S::kPiece + f % S::kPiece] =               \
                x[P * S::kLoads + i];                                                          \
        }                                                                                      \
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");                                 \
        __builtin_amdgcn_wave_barrier();                                                       \
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");                                 \
        constexpr int J0 = P * NE / S::kParts, J1 = (P + 1) * NE / S::kParts;                  \
        _Pragma("unroll") for (int jc = J0 / 4; jc < J1 / 4; ++jc) {                           \
            const f32x4_t y = my_tile[slot * S::kRow + q + LPT * jc];                          \
            v[4 * jc] = y.x;                                                                   \
            v[4 * jc + 1] = y.y;                                                               \
            v[4 * jc + 2] = y.z;                                                               \
            v[4 * jc + 3] = y.w;                                                               \
        }                                                                                      \
        moe_topk::scan_values<LPT, NE, KM, J0, J1>(v, valid, q, list);                         \
        __builtin_amdgcn_sched_barrier(0);                                                     \
    }
            MOE_ROUTE_SLICE(0)
            MOE_ROUTE_SLICE(1)
            MOE_ROUTE_SLICE(2)
            MOE_ROUTE_SLICE(3)
#undef MOE_ROUTE_SLICE
            moe_topk::finish_values<LPT, NE, KM>(list, v, t, valid, K, k_ref, q, topk_ids, topk_w,
                                                 hist);
        } else {
            moe_topk::topk_token<LPT, NE, KM>(logits + (int64_t)(valid ? t : 0) * E, t, valid, E,
                                              K, k_ref, q, topk_ids, topk_w, hist);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

template <int LPT, int NE, int KM>
void launch_km(int grid, hipStream_t stream, const float* logits, int T, int E, int K,
               int k_ref, int32_t* ids, float* w, int32_t* counts) {
    // staged reads when the rows exactly fill the lanes and the logits are 16-byte aligned
    const bool vec = NE % 4 == 0 && E == LPT * NE && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
    if constexpr (NE % 4 == 0) {
        if (vec) {
            route_kernel<LPT, NE, KM, true><<<grid, kRouteThreads, 0, stream>>>(
                logits, T, E, K, k_ref, ids, w, counts);
            return;
        }
    }
    route_kernel<LPT, NE, KM, false><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, k_ref,
                                                                        ids, w, counts);
}

template <int LPT, int NE>
void launch_ne(int grid, hipStream_t stream, const float* logits, int T, int E, int K,
               int k_ref, int32_t* ids, float* w, int32_t* counts) {
    const int need = k_ref < E && k_ref > K ? k_ref : K;  // list length the weights need
    if (need <= 4)
        launch_km<LPT, NE, 4>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else if (need <= 8)
        launch_km<LPT, NE, 8>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else
        launch_km<LPT, NE, 16>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
}

template <int LPT>
void launch_lpt(hipStream_t stream, const float* logits, int T, int E, int K, int k_ref,
                int32_t* ids, float* w, int32_t* counts) {
    const int tokens_per_block = (MOE_WAVE / LPT) * (kRouteThreads / MOE_WAVE);
    int grid = (T + tokens_per_block - 1) / tokens_per_block;
    if (grid > kMaxRouteBlocks) grid = kMaxRouteBlocks;
    const int ne = (E + LPT - 1) / LPT;
    if (ne <= 2)
        launch_ne<LPT, 2>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else if (ne <= 4)
        launch_ne<LPT, 4>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else if (ne <= 8)
        launch_ne<LPT, 8>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else if (LPT * 16 >= 256 || ne <= 16)  // E <= 256: 16 lanes per token need at most 16
        launch_ne<LPT, 16>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    else if constexpr (LPT * 16 < 256) {
        if (ne <= 32)
            launch_ne<LPT, 32>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
        else
            launch_ne<LPT, 64>(grid, stream, logits, T, E, K, k_ref, ids, w, counts);
    }
}

}  // namespace

hipError_t moe_launch_zero_counts(int32_t* counts, int E, hipStream_t stream) {
    zero_i32_kernel<<<(E + kRouteThreads - 1) / kRouteThreads, kRouteThreads, 0, stream>>>(counts, E);
    return hipGetLastError();
}

hipError_t moe_launch_route(const float* logits, int T, int E, int K, int k_ref,
                            int32_t* topk_ids, float* topk_w, int32_t* counts,
                            hipStream_t stream) {
    zero_i32_kernel<<<(E + kRouteThreads - 1) / kRouteThreads, kRouteThreads, 0, stream>>>(counts, E);
    // 4 lanes per token while that still gives a wave to each of the 1024 SIMDs, else 16
    if ((T + 15) / 16 >= 1024)
        launch_lpt<4>(stream, logits, T, E, K, k_ref, topk_ids, topk_w, counts);
    else
        launch_lpt<16>(stream, logits, T, E, K, k_ref, topk_ids, topk_w, counts);
    return hipGetLastError();
}
