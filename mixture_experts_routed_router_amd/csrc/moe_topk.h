// moe_topk.h -- per-token top-k and routing weights over a logit row, shared by moe_route
// (logits in HBM) and moe_router_topk (logits in LDS).
//
// LPT lanes per token.  Lane q of a token scans experts q, q+LPT, q+2 LPT, ... and keeps its
// own top-KM list in registers, sorted under the total order "larger logit, then smaller id"
// (ties resolve to the lower id).  A (logit, id) pair is one 64-bit key: the logit's bits
// mapped to an order-preserving signed integer in the high word and ~id in the low word, so
// one signed 64-bit compare decides the order and no two keys are equal.  Inside a lane the
// ids rise along the scan, so a new key beats a listed one exactly when its logit is larger:
// the insertion compares the high words only.  The lane lists are merged by bitonic merges
// across the token's lanes; afterwards every lane of the token holds the token's top-KM.
// Weights: exp(l_k - m) for the K picks over a reference mass, m the largest logit: the top
// k_ref experts' exp(l - m) for k_ref < E (k_ref = K: renormalised over the picks), every
// expert's for k_ref = E (plain softmax), float32.
#pragma once
#include "moe_device.h"

namespace moe_topk {

constexpr int64_t kPadKey = INT64_MIN;  // loses to every real key

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


// Top-K of one token (row = its E logits, valid = the token exists) into topk_ids / topk_w
// [t * K + k] and the workgroup histogram `hist` (LDS).  Requires K <= KM, and k_ref <= KM
// unless k_ref >= E.  Called by all LPT lanes of the token with q = their index.
template <int LPT, int NE, int KM>
__device__ __forceinline__ void topk_token(const float* row, int t, bool valid, int E, int K,
                                           int k_ref, int q, int32_t* __restrict__ topk_ids,
                                           float* __restrict__ topk_w, int* hist) {
    // this lane's top-KM, sorted descending: a new key goes in just above the first listed
    // key it beats and everything from there moves down one place
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
        const float v = expf(key_logit(top[k]) - m);
        ex[k] = k < K ? v : 0.f;
        if (k < k_ref) denom += v;  // k_ref <= KM here unless k_ref >= E (below)
    }
    if (k_ref >= E) {
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

}  // namespace moe_topk
