// route.hip -- router top-k, routing weights and expert histogram (moe_route).
//
// MegaFlux §1: a router sends each token to k experts whose outputs are mixed by routing
// weights; §4.1: the k experts of a token are distinct.  The top-k renormalisation abstract
// (Daily Papers listing): the picked experts' probabilities are renormalised over the picks.
//
// LPT lanes per token (4, or 16 when there are too few tokens to fill the chip).  Lane q of a
// token scans experts q, q+LPT, q+2 LPT, ... and keeps its own top-KM list in registers,
// sorted under the total order "larger logit, then smaller id" (ties resolve to the lower
// id).  A (logit, id) pair is one 64-bit key: the logit's bits mapped to an order-preserving
// signed integer in the high word and ~id in the low word, so one signed 64-bit compare
// decides the order and no two keys are equal.  Inside a lane the ids rise along the scan,
// so a new key beats a listed one exactly when its logit is larger: the insertion compares
// the high words only.  The lane lists are merged by bitonic merges across the token's
// lanes; afterwards every lane of the token holds the token's top-KM.  Weights: a float32
// softmax over the K picks (or over all E logits), shifted by the largest logit.  The expert
// histogram is counted in LDS per workgroup (integer adds: order-independent) and flushed
// with one global atomic per nonzero bin; the grid is capped at 256 workgroups so that a
// bin's counter takes at most 256 of them.
#include "moe_launch.h"

namespace {

constexpr int kRouteThreads = 512;
constexpr int kMaxRouteBlocks = 256;
constexpr int64_t kPadKey = INT64_MIN;  // loses to every real key

__global__ void __launch_bounds__(kRouteThreads)
zero_i32_kernel(int32_t* __restrict__ p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// order-preserving map of a finite float to int32 (-0 and +0 map to the same value)
__device__ __forceinline__ int32_t float_order_key(float v) {
    int32_t b = __float_as_int(v);
    if (b == INT32_MIN) b = 0;
    return b < 0 ? (b ^ 0x7FFFFFFF) : b;
}

__device__ __forceinline__ float key_logit(int64_t key) {
    int32_t b = (int32_t)(key >> 32);
    return __int_as_float(b < 0 ? (b ^ 0x7FFFFFFF) : b);
}

__device__ __forceinline__ int key_id(int64_t key) { return (int)~(uint32_t)key; }

// Top-KM of the union of this lane's list and the list of lane ^ mask (both sorted
// descending): the elementwise larger of a[i] and b[KM-1-i] is the top-KM as a bitonic
// sequence, which a bitonic merge sorts.
template <int KM>
__device__ __forceinline__ void merge_with(int64_t (&a)[KM], int mask) {
    int64_t b[KM];
#pragma unroll
    for (int i = 0; i < KM; ++i) b[i] = __shfl_xor(a[i], mask, MOE_WAVE);
#pragma unroll
    for (int i = 0; i < KM; ++i) {
        const int64_t o = b[KM - 1 - i];
        a[i] = o > a[i] ? o : a[i];
    }
#pragma unroll
    for (int s = KM / 2; s > 0; s >>= 1) {
#pragma unroll
        for (int i = 0; i < KM; ++i) {
            if ((i & s) == 0) {
                const int64_t hi = a[i] > a[i + s] ? a[i] : a[i + s];
                const int64_t lo = a[i] > a[i + s] ? a[i + s] : a[i];
                a[i] = hi;
                a[i + s] = lo;
            }
        }
    }
}

// LPT: lanes per token; NE: experts per lane (E <= LPT * NE); KM: list length (K <= KM),
// a power of two.
template <int LPT, int NE, int KM>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const float* __restrict__ logits, int T, int E, int K, int renormalize,
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
        const float* row = logits + (int64_t)(valid ? t : 0) * E;
        // this lane's top-KM, sorted descending: a new key goes in just above the first
        // listed key it beats and everything from there moves down one place
        int64_t top[KM];
#pragma unroll
        for (int i = 0; i < KM; ++i) top[i] = kPadKey;
#pragma unroll 4
        for (int j = 0; j < NE; ++j) {
            const int e = q + LPT * j;
            const bool real = valid && e < E;
            const int32_t hi = real ? float_order_key(row[e]) : INT32_MIN;
            const int64_t key = real ? (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(~(uint32_t)e))
                                     : kPadKey;
            bool gt[KM];
#pragma unroll
            for (int i = 0; i < KM; ++i) gt[i] = real && hi > (int32_t)(top[i] >> 32);
#pragma unroll
            for (int i = KM - 1; i > 0; --i) top[i] = gt[i - 1] ? top[i - 1] : (gt[i] ? key : top[i]);
            top[0] = gt[0] ? key : top[0];
        }
#pragma unroll
        for (int mask = 1; mask < LPT; mask <<= 1) merge_with<KM>(top, mask);

        const float m = key_logit(top[0]);
        float ex[KM];
        float denom = 0.f;
#pragma unroll
        for (int k = 0; k < KM; ++k) {
            ex[k] = k < K ? expf(key_logit(top[k]) - m) : 0.f;
            denom += ex[k];
        }
        if (!renormalize) {
            float s = 0.f;
            for (int j = 0; j < NE; ++j)
                if (valid && q + LPT * j < E) s += expf(row[q + LPT * j] - m);
#pragma unroll
            for (int mask = 1; mask < LPT; mask <<= 1) s += __shfl_xor(s, mask, MOE_WAVE);
            denom = s;
        }
        if (valid) {
#pragma unroll
            for (int k = 0; k < KM; ++k) {
                if (k < K && (k & (LPT - 1)) == q) {
                    const int id = key_id(top[k]);
                    topk_ids[(int64_t)t * K + k] = id;
                    topk_w[(int64_t)t * K + k] = ex[k] / denom;
                    atomicAdd(&hist[id], 1);
                }
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

template <int LPT, int NE>
void launch_ne(int grid, hipStream_t stream, const float* logits, int T, int E, int K,
               int renormalize, int32_t* ids, float* w, int32_t* counts) {
    if (K <= 4)
        route_kernel<LPT, NE, 4><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K,
                                                                     renormalize, ids, w, counts);
    else if (K <= 8)
        route_kernel<LPT, NE, 8><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K,
                                                                     renormalize, ids, w, counts);
    else
        route_kernel<LPT, NE, 16><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K,
                                                                      renormalize, ids, w, counts);
}

template <int LPT>
void launch_lpt(hipStream_t stream, const float* logits, int T, int E, int K, int renormalize,
                int32_t* ids, float* w, int32_t* counts) {
    const int tokens_per_block = (MOE_WAVE / LPT) * (kRouteThreads / MOE_WAVE);
    int grid = (T + tokens_per_block - 1) / tokens_per_block;
    if (grid > kMaxRouteBlocks) grid = kMaxRouteBlocks;
    const int ne = (E + LPT - 1) / LPT;
    if (ne <= 2)
        launch_ne<LPT, 2>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
    else if (ne <= 4)
        launch_ne<LPT, 4>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
    else if (ne <= 8)
        launch_ne<LPT, 8>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
    else if (LPT * 16 >= 256 || ne <= 16)  // E <= 256: 16 lanes per token need at most 16
        launch_ne<LPT, 16>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
    else if constexpr (LPT * 16 < 256) {
        if (ne <= 32)
            launch_ne<LPT, 32>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
        else
            launch_ne<LPT, 64>(grid, stream, logits, T, E, K, renormalize, ids, w, counts);
    }
}

}  // namespace

hipError_t moe_launch_route(const float* logits, int T, int E, int K, int renormalize,
                            int32_t* topk_ids, float* topk_w, int32_t* counts,
                            hipStream_t stream) {
    zero_i32_kernel<<<(E + kRouteThreads - 1) / kRouteThreads, kRouteThreads, 0, stream>>>(counts, E);
    // 4 lanes per token while that still gives a wave to each of the 1024 SIMDs, else 16
    if ((T + 15) / 16 >= 1024)
        launch_lpt<4>(stream, logits, T, E, K, renormalize, topk_ids, topk_w, counts);
    else
        launch_lpt<16>(stream, logits, T, E, K, renormalize, topk_ids, topk_w, counts);
    return hipGetLastError();
}
