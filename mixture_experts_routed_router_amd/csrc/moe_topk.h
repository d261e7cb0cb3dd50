// moe_topk.h -- per-token top-k and routing weights over a logit row, shared by moe_route
// (logits in HBM) and moe_router_topk (logits in LDS).
//
// LPT lanes per token.  Each lane keeps its own top-KM list in registers, sorted under the total
// order "larger logit, then smaller id" (ties resolve to the lower id), takes its experts G at a
// time (sort the group with a sorting network, merge it into the list with one bitonic merge),
// and the token's lane lists are then merged across the lanes (DPP lane moves, bitonic merges);
// afterwards every lane of the token holds the token's top-KM.  A (logit, id) pair is kept as a
// double whose bit pattern rises with that order (scan_key below), so that each compare-exchange
// is one v_max_f64 and one v_min_f64; the final list is turned into 64-bit integer keys (the
// logit's order-preserving integer in the high word, ~id in the low word) to read logits and ids
// back.  No two keys are equal, so the result does not depend on the order of the comparisons.
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

// Scan keys.  A lane's list is kept as doubles whose bit patterns rise with the key order:
// bit 61 set (exponent in [0x200, 0x3ff]: a positive normal number, never inf or NaN), bits
// 60..29 the logit's order-preserving unsigned image (the high word of the 64-bit key with its
// sign bit flipped) and bits 28..0 (2^29 - 1) - id.  On such doubles the numeric order is the
// bit-pattern order, so max and min of two keys are one v_max_f64 / v_min_f64 each, where the
// 64-bit integer form needs a compare and four selects.  A double with a zero high word is an
// empty slot and loses to every real key.  Requires E <= 2^29.
constexpr uint32_t kIdMask = (1u << 29) - 1;

// the key of logit v and id_term = kIdMask - id; an empty slot (high word 0, below every real
// key) unless real
__device__ __forceinline__ double scan_key(float v, uint32_t id_term, bool real) {
    const int32_t b = __float_as_int(v + 0.f);  // -0 + 0 = +0: both zeros give one key
    const uint32_t u = (uint32_t)b ^ ((uint32_t)(b >> 31) | 0x80000000u);
    const uint32_t hi = __builtin_amdgcn_alignbit(1u, u, 3);  // (1 << 29) | (u >> 3)
    const uint32_t lo = (u << 29) | id_term;
    return __hiloint2double(real ? (int)hi : 0, (int)lo);
}

__device__ __forceinline__ int64_t scan_key_to_key(double d) {
    const uint32_t hi = (uint32_t)__double2hiint(d), lo = (uint32_t)__double2loint(d);
    const uint32_t u = __builtin_amdgcn_alignbit(hi, lo, 29);
    const uint32_t id = kIdMask - (lo & kIdMask);
    const int64_t key = (int64_t)(((uint64_t)(u ^ 0x80000000u) << 32) | (uint64_t)(~id));
    return hi == 0 ? kPadKey : key;
}

// Max and min of two keys.  Written as the instructions themselves: keys are never NaN, and the
// compiler's fmax / fmin would first quiet each freshly built key with one more v_max_f64.
__device__ __forceinline__ double key_max(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ double key_min(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// a keeps the larger key, b the smaller
__device__ __forceinline__ void exchange(double& a, double& b) {
    const double hi = key_max(a, b), lo = key_min(a, b);
    a = hi;
    b = lo;
}

// Sorts G keys descending with Batcher's odd-even merge sort network (G = 2, 4, 8: 1, 5 and 19
// exchanges).
template <int G>
__device__ __forceinline__ void sort_group(double (&s)[G]) {
    static_assert(G == 2 || G == 4 || G == 8, "group of 2, 4 or 8");
    if constexpr (G == 2) {
        exchange(s[0], s[1]);
    } else if constexpr (G == 4) {
        exchange(s[0], s[1]); exchange(s[2], s[3]);
        exchange(s[0], s[2]); exchange(s[1], s[3]);
        exchange(s[1], s[2]);
    } else {
        exchange(s[0], s[1]); exchange(s[2], s[3]); exchange(s[4], s[5]); exchange(s[6], s[7]);
        exchange(s[0], s[2]); exchange(s[1], s[3]); exchange(s[4], s[6]); exchange(s[5], s[7]);
        exchange(s[1], s[2]); exchange(s[5], s[6]);
        exchange(s[0], s[4]); exchange(s[1], s[5]); exchange(s[2], s[6]); exchange(s[3], s[7]);
        exchange(s[2], s[4]); exchange(s[3], s[5]);
        exchange(s[1], s[2]); exchange(s[3], s[4]); exchange(s[5], s[6]);
    }
}

// The top KM of list and s (both sorted descending) back into list, sorted: the elementwise
// larger of list[i] and s[KM-1-i] (s padded with empty slots) holds the top KM as a bitonic
// sequence, which a bitonic merge sorts.
template <int KM, int G>
__device__ __forceinline__ void merge_group(double (&list)[KM], const double (&s)[G]) {
#pragma unroll
    for (int i = 0; i < KM; ++i)
        if (KM - 1 - i < G) list[i] = key_max(list[i], s[KM - 1 - i]);
#pragma unroll
    for (int st = KM / 2; st > 0; st >>= 1) {
#pragma unroll
        for (int i = 0; i < KM; ++i)
            if ((i & st) == 0) exchange(list[i], list[i + st]);
    }
}

// x of the partner lane: kCtrl is a DPP lane pattern that keeps a lane inside its row of 16.
template <int kCtrl>
__device__ __forceinline__ double dpp_key(double x) {
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), kCtrl, 0xF, 0xF, false);
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), kCtrl, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Round r of the merge of a token's lane lists (lanes 0 .. LPT-1 of an aligned group, LPT <= 16):
// every lane pairs with a lane of the other half of its aligned group of 2^(r+1) lanes (quad
// lane xor 1, quad lane xor 2, the mirror lane in its 8, the mirror lane in its 16), whose
// list equals that of every lane of its half after the earlier rounds.  The elementwise larger
// of a[i] and the partner's b[KM-1-i] holds the top KM of both lists as a bitonic sequence,
// which a bitonic merge sorts; afterwards the whole group of 2^(r+1) lanes holds one list.
template <int KM, int kRound>
__device__ __forceinline__ void merge_lanes(double (&a)[KM]) {
    constexpr int kCtrl = kRound == 0 ? 0xB1 : kRound == 1 ? 0x4E : kRound == 2 ? 0x141 : 0x140;
    static_assert(kRound >= 0 && kRound < 4, "at most 16 lanes per token");
    double b[KM];
#pragma unroll
    for (int i = 0; i < KM; ++i) b[i] = dpp_key<kCtrl>(a[i]);
#pragma unroll
    for (int i = 0; i < KM; ++i) a[i] = key_max(a[i], b[KM - 1 - i]);
#pragma unroll
    for (int st = KM / 2; st > 0; st >>= 1) {
#pragma unroll
        for (int i = 0; i < KM; ++i)
            if ((i & st) == 0) exchange(a[i], a[i + st]);
    }
}

// Expert id of the lane's j-th value: kChunks, expert 4c + j % 4 of chunk c = q + LPT (j / 4);
// else expert q + LPT j.
template <int LPT, bool kChunks>
__device__ __forceinline__ int lane_expert(int q, int j) {
    return kChunks ? 4 * (q + LPT * (j / 4)) + (j % 4) : q + LPT * j;
}

// The top KM keys of the lane's experts into list (sorted descending, empty slots last), taken
// G at a time: each group is sorted and merged into the list (for KM = 8 about 9 max / min per
// expert, against 15 for inserting one key at a time).  kChunks: the values are v, in chunk
// order (lane_expert); else the group's G values are read from row (experts q, q + LPT, ...)
// just before use, from indices clamped into the row.  kAll: the token exists and every one of
// the lane's experts is below E, so no key needs emptying.
// Groups j0 in [J0, J1) only (multiples of G; J0 = 0 starts the list).
template <int LPT, int NE, int KM, int G, bool kChunks, bool kAll, int J0 = 0, int J1 = NE>
__device__ __forceinline__ void scan_lane(const float* row, const float (&v)[kChunks ? NE : 1],
                                          bool valid, int E, int q, double (&list)[KM]) {
    static_assert(J0 % G == 0 && J1 % G == 0 && J0 < J1 && J1 <= NE, "whole groups");
#pragma unroll(kChunks ? (J1 - J0) / G : 2)
    for (int j0 = J0; j0 < J1; j0 += G) {
        // the partial scan is rare: keep its per-expert bound checks inside the loop instead
        // of hoisted ahead of it as masks that take registers for the whole kernel
        int E_ = E;
        if constexpr (!kAll) asm volatile("" : "+s"(E_));
        double g[G];
#pragma unroll
        for (int jj = 0; jj < G; ++jj) {
            const int e = lane_expert<LPT, kChunks>(q, j0 + jj);
            float x;
            if constexpr (kChunks) x = v[j0 + jj];
            else x = row[kAll || e < E_ ? e : E_ - 1];
            g[jj] = scan_key(x, kIdMask - e, kAll || (valid && e < E_));
        }
        sort_group<G>(g);
        if (j0 == 0) {
#pragma unroll
            for (int i = 0; i < KM; ++i) list[i] = i < G ? g[i < G ? i : 0] : 0.0;
        } else {
            merge_group<KM, G>(list, g);
        }
    }
}

// The lane lists of a token merged across its LPT lanes, then the K ids and weights written by
// the lanes in turn and counted in `hist`.  lane_sum_exp(m): the lane's sum of exp(l - m) over
// its experts below E (used when k_ref >= E).
template <int LPT, int KM, class LaneSumExp>
__device__ __forceinline__ void finish_token(double (&list)[KM], int t, bool valid, int E,
                                             int K, int k_ref, int q,
                                             int32_t* __restrict__ topk_ids,
                                             float* __restrict__ topk_w, int* hist,
                                             LaneSumExp lane_sum_exp) {
    static_assert(LPT >= 1 && LPT <= 16 && (LPT & (LPT - 1)) == 0, "1 to 16 lanes per token");
    if constexpr (LPT > 1) merge_lanes<KM, 0>(list);
    if constexpr (LPT > 2) merge_lanes<KM, 1>(list);
    if constexpr (LPT > 4) merge_lanes<KM, 2>(list);
    if constexpr (LPT > 8) merge_lanes<KM, 3>(list);
    int64_t top[KM];
#pragma unroll
    for (int i = 0; i < KM; ++i) top[i] = scan_key_to_key(list[i]);

    const float m = key_logit(top[0]);
    float ex[KM];
    float denom = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
        const float x = expf(key_logit(top[k]) - m);
        ex[k] = k < K ? x : 0.f;
        if (k < k_ref) denom += x;  // k_ref <= KM here unless k_ref >= E (below)
    }
    if (k_ref >= E) {
        float s = lane_sum_exp(m);
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

template <int KM, int NE>
constexpr int group_size() {
    return (KM >= 8 ? 8 : 4) < NE ? (KM >= 8 ? 8 : 4) : NE;
}

// Top-K of one token (row = its E logits, valid = the token exists) into topk_ids / topk_w
// [t * K + k] and the workgroup histogram `hist` (LDS).  Requires K <= KM, and k_ref <= KM
// unless k_ref >= E.  Called by all LPT lanes of the token with q = their index; lane q takes
// experts q, q + LPT, ...  row must point at E readable floats also when the token does not
// exist.
template <int LPT, int NE, int KM>
__device__ __forceinline__ void topk_token(const float* row, int t, bool valid, int E, int K,
                                           int k_ref, int q, int32_t* __restrict__ topk_ids,
                                           float* __restrict__ topk_w, int* hist) {
    constexpr int G = group_size<KM, NE>();
    static_assert(NE % G == 0, "whole groups per lane");
    const float none[1] = {0.f};
    double list[KM];
    if (valid && E == LPT * NE)
        scan_lane<LPT, NE, KM, G, false, true>(row, none, valid, E, q, list);
    else
        scan_lane<LPT, NE, KM, G, false, false>(row, none, valid, E, q, list);
    finish_token<LPT, KM>(list, t, valid, E, K, k_ref, q, topk_ids, topk_w, hist, [&](float m) {
        float s = 0.f;
        for (int j = 0; j < NE; ++j)
            if (valid && q + LPT * j < E) s += expf(row[q + LPT * j] - m);
        return s;
    });
}

// The same on values already in registers, in parts: v[j] is the logit of expert
// lane_expert<LPT, true>(q, j), that is 16-byte chunks q, q + LPT, ... of the row, and the row
// is whole (E = LPT * NE).  scan_values<J0, J1> takes groups [J0, J1) of the lane's values into
// list (J0 = 0 first); finish_values then merges the lanes and writes the token.
template <int LPT, int NE, int KM, int J0, int J1>
__device__ __forceinline__ void scan_values(const float (&v)[NE], bool valid, int q,
                                            double (&list)[KM]) {
    constexpr int G = group_size<KM, NE>();
    static_assert(NE % G == 0 && NE % 4 == 0 && G >= 4, "whole chunks and groups per lane");
    if (valid)
        scan_lane<LPT, NE, KM, G, true, true, J0, J1>(nullptr, v, valid, LPT * NE, q, list);
    else
        scan_lane<LPT, NE, KM, G, true, false, J0, J1>(nullptr, v, valid, LPT * NE, q, list);
}

template <int LPT, int NE, int KM>
__device__ __forceinline__ void finish_values(double (&list)[KM], const float (&v)[NE], int t,
                                              bool valid, int K, int k_ref, int q,
                                              int32_t* __restrict__ topk_ids,
                                              float* __restrict__ topk_w, int* hist) {
    finish_token<LPT, KM>(list, t, valid, LPT * NE, K, k_ref, q, topk_ids, topk_w, hist,
                          [&](float m) {
                              float s = 0.f;
#pragma unroll
                              for (int j = 0; j < NE; ++j) s += expf(v[j] - m);
                              return s;
                          });
}

}  // namespace moe_topk
