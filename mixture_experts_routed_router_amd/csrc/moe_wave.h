// moe_wave.h -- wave-level arg-min / arg-max over groups of lanes, shared by the planners.
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

// Best (v, i) over the aligned group of 2^levels lanes containing this lane (levels <= 6);
// every lane of the group ends with the result.  kMax: larger v wins, else smaller v; equal
// v: smaller i.
template <bool kMax>
__device__ __forceinline__ void group_best(int& v, int& i, int levels) {
    auto take = [&](int ov, int oi) {
        const bool better = kMax ? (ov > v || (ov == v && oi < i)) : (ov < v || (ov == v && oi < i));
        if (better) {
            v = ov;
            i = oi;
        }
    };
    if (levels > 0) take(dpp_partner<0>(v), dpp_partner<0>(i));
    if (levels > 1) take(dpp_partner<1>(v), dpp_partner<1>(i));
    if (levels > 2) take(dpp_partner<2>(v), dpp_partner<2>(i));
    if (levels > 3) take(dpp_partner<3>(v), dpp_partner<3>(i));
    if (levels > 4) take(__shfl_xor(v, 16, MOE_WAVE), __shfl_xor(i, 16, MOE_WAVE));
    if (levels > 5) take(__shfl_xor(v, 32, MOE_WAVE), __shfl_xor(i, 32, MOE_WAVE));
}

__device__ __forceinline__ int ceil_log2(int n) {
    int l = 0;
    while ((1 << l) < n) ++l;
    return l;
}

// group_best over the group of lanes 0 .. 2^levels - 1, broadcast from lane 0 to the whole
// wave, so that every lane takes the same decisions (call with every lane active).
template <bool kMax>
__device__ __forceinline__ void wave_best(int& v, int& i, int levels) {
    group_best<kMax>(v, i, levels);
    v = __builtin_amdgcn_readfirstlane(v);
    i = __builtin_amdgcn_readfirstlane(i);
}

}  // namespace moe_wave

using moe_wave::ceil_log2;
using moe_wave::group_best;
using moe_wave::wave_best;
