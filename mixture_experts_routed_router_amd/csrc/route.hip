// route.hip -- router top-k, routing weights and expert histogram (moe_route).
//
// MegaFlux §1: a router sends each token to k experts whose outputs are mixed by routing
// weights; §4.1: the k experts of a token are distinct.  The top-k renormalisation abstract
// (Daily Papers listing): the picked experts' probabilities are renormalised over the picks.
//
// LPT lanes per token (4, or 16 when there are too few tokens to fill the chip); the per-token
// top-k and weights are moe_topk::topk_token (moe_topk.h).  The expert histogram is counted in
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

// LPT: lanes per token; NE: experts per lane (E <= LPT * NE); KM: list length, a power of
// two with K <= KM and (k_ref <= KM or k_ref >= E).
template <int LPT, int NE, int KM>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const float* __restrict__ logits, int T, int E, int K, int k_ref,
             int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
             int32_t* __restrict__ counts) {
    constexpr int kTokensPerWave = MOE_WAVE / LPT;
    __shared__ int hist[256];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();

    const int lane = moe_lane_id();
    const int q = lane & (LPT - 1);
    const int slot = lane / LPT;
    const int waves_total = gridDim.x * (kRouteThreads / MOE_WAVE);
    const int wave_global = blockIdx.x * (kRouteThreads / MOE_WAVE) + threadIdx.x / MOE_WAVE;

    for (int t0 = wave_global * kTokensPerWave; t0 < T; t0 += waves_total * kTokensPerWave) {
        const int t = t0 + slot;
        const bool valid = t < T;
        moe_topk::topk_token<LPT, NE, KM>(logits + (int64_t)(valid ? t : 0) * E, t, valid, E, K,
                                          k_ref, q, topk_ids, topk_w, hist);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

template <int LPT, int NE>
void launch_ne(int grid, hipStream_t stream, const float* logits, int T, int E, int K,
               int k_ref, int32_t* ids, float* w, int32_t* counts) {
    const int need = k_ref < E && k_ref > K ? k_ref : K;  // list length the weights need
    if (need <= 4)
        route_kernel<LPT, NE, 4><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, k_ref, ids,
                                                                     w, counts);
    else if (need <= 8)
        route_kernel<LPT, NE, 8><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, k_ref, ids,
                                                                     w, counts);
    else
        route_kernel<LPT, NE, 16><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, k_ref,
                                                                      ids, w, counts);
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
