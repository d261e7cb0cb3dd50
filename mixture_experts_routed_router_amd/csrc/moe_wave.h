// moe_wave.h -- wave-level arg-min / arg-max over the lanes of a wave, shared by the planners.
#pragma once
#include "moe_device.h"

namespace moe_wave {

// value of lane (lane ^ 1), (lane ^ 2), (7 - lane within 8), (15 - lane within 16): after
// reductions over the smaller groups, each step pairs a lane with the other half of its group
template <int kStep>
__device__ __forceinline__ int dpp_partner(int v) {
    constexpr int ctrl = kStep == 0 ? 0xB1 : kStep == 1 ? 0x4E : kStep == 2 ? 0x141 : 0x140;
    return __builtin_amdgcn_update_dpp(v, v, ctrl, 0xF, 0xF, false);
}

// Totally ordered 64-bit keys for arg-best searches over (value, index): the value in the high
// word, so a signed 64-bit compare decides by value first, then by the low word.
//   min_key: smaller value wins, then smaller index;  max_key: larger value, then smaller index.
__device__ __forceinline__ int64_t min_key(int v, int i) {
    return (int64_t)v * 4294967296LL + (int64_t)(uint32_t)i;
}
__device__ __forceinline__ int64_t max_key(int v, int i) {
    return (int64_t)v * 4294967296LL + (int64_t)(uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ int key_value(int64_t k) { return (int)(k >> 32); }
__device__ __forceinline__ int min_key_index(int64_t k) { return (int)(uint32_t)k; }
__device__ __forceinline__ int max_key_index(int64_t k) { return (int)~(uint32_t)k; }

// The best key of all 64 lanes, returned uniform (scalar).  Branch-free: four DPP steps inside
// each 16-lane row, then v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (halves).
// A swap returns the lane's own key and its partner's in some order; the better of the two is
// the same either way, so the order does not matter.  Call with every lane active.
template <bool kMax>
__device__ __forceinline__ int64_t wave_best_key(int64_t k) {
    auto pick = [](int64_t a, int64_t b) { return kMax ? (a > b ? a : b) : (a < b ? a : b); };
    auto join = [](uint32_t lo, uint32_t hi) { return (int64_t)(((uint64_t)hi << 32) | lo); };
    uint32_t lo = (uint32_t)k, hi = (uint32_t)((uint64_t)k >> 32);
    k = pick(k, join(dpp_partner<0>((int)lo), dpp_partner<0>((int)hi)));
    lo = (uint32_t)k; hi = (uint32_t)((uint64_t)k >> 32);
    k = pick(k, join(dpp_partner<1>((int)lo), dpp_partner<1>((int)hi)));
    lo = (uint32_t)k; hi = (uint32_t)((uint64_t)k >> 32);
    k = pick(k, join(dpp_partner<2>((int)lo), dpp_partner<2>((int)hi)));
    lo = (uint32_t)k; hi = (uint32_t)((uint64_t)k >> 32);
    k = pick(k, join(dpp_partner<3>((int)lo), dpp_partner<3>((int)hi)));
    lo = (uint32_t)k; hi = (uint32_t)((uint64_t)k >> 32);
    {
        const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        k = pick(join(l[0], h[0]), join(l[1], h[1]));
    }
    lo = (uint32_t)k; hi = (uint32_t)((uint64_t)k >> 32);
    {
        const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        k = pick(join(l[0], h[0]), join(l[1], h[1]));
    }
    lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)k);
    hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)k >> 32));
    return join(lo, hi);
}

// Best (v, i) over all 64 lanes, returned uniform: larger v wins for kMax, else smaller v;
// equal v: smaller i.  Lanes that do not compete hold a value that loses to every competitor
// (-1 or the type's minimum for kMax, the type's maximum otherwise).  Call with every lane
// active.
template <bool kMax>
__device__ __forceinline__ void wave_best_all(int& v, int& i) {
    const int64_t k = wave_best_key<kMax>(kMax ? max_key(v, i) : min_key(v, i));
    v = key_value(k);
    i = kMax ? max_key_index(k) : min_key_index(k);
}

}  // namespace moe_wave

using moe_wave::wave_best_all;
using moe_wave::wave_best_key;
