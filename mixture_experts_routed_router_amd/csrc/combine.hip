// combine.hip -- routing-weight combine of each token's expert outputs (moe_combine).
//
// MegaFlux §1: expert outputs are mixed by the routing weights; §2.1: the final top-k sum is
// a step of its own; App. A.2: token ids, top-k slots and weights are kept for it.  The
// weighted scatter-add is done in its gather form: each output element reads the K rows its
// token's entries landed in (entry_pos), so every output is written once, with no atomics,
// and the sum runs in a fixed order (ascending k, float32).
//
// One thread per 16 bytes of output (8 bf16 or 4 float32 columns); consecutive threads take
// consecutive columns of a token, so every yp row read and out row write is a coalesced run.
#include "moe_launch.h"

namespace {

constexpr int kThreads = 256;

template <bool kBF16>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const uint8_t* __restrict__ yp, const float* __restrict__ w,
               const int32_t* __restrict__ entry_pos, int T, int H, int K,
               uint8_t* __restrict__ out) {
    constexpr int kVec = kBF16 ? 8 : 4;  // elements per 16 bytes
    const int64_t row_bytes = (int64_t)H * (kBF16 ? 2 : 4);
    const int nv = H / kVec;
    const int64_t total = (int64_t)T * nv;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int t = (int)(idx / nv);
        const int c = (int)(idx - (int64_t)t * nv);
        float acc[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
        for (int k = 0; k < K; ++k) {
            const int p = entry_pos[(int64_t)t * K + k];
            if (p < 0) continue;
            const float wk = w[(int64_t)t * K + k];
            const uint4 v = reinterpret_cast<const uint4*>(yp + (int64_t)p * row_bytes)[c];
            if (kBF16) {
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] = fmaf(wk, moe_bf16_to_f32((uint16_t)(u[e] & 0xFFFFu)), acc[2 * e]);
                    acc[2 * e + 1] = fmaf(wk, moe_bf16_to_f32((uint16_t)(u[e] >> 16)), acc[2 * e + 1]);
                }
            } else {
                acc[0] = fmaf(wk, __uint_as_float(v.x), acc[0]);
                acc[1] = fmaf(wk, __uint_as_float(v.y), acc[1]);
                acc[2] = fmaf(wk, __uint_as_float(v.z), acc[2]);
                acc[3] = fmaf(wk, __uint_as_float(v.w), acc[3]);
            }
        }
        uint4 o;
        if (kBF16) {
            o.x = moe_pack_bf16x2(acc[0], acc[1]);
            o.y = moe_pack_bf16x2(acc[2], acc[3]);
            o.z = moe_pack_bf16x2(acc[4], acc[5]);
            o.w = moe_pack_bf16x2(acc[6], acc[7]);
        } else {
            o.x = __float_as_uint(acc[0]);
            o.y = __float_as_uint(acc[1]);
            o.z = __float_as_uint(acc[2]);
            o.w = __float_as_uint(acc[3]);
        }
        reinterpret_cast<uint4*>(out + (int64_t)t * row_bytes)[c] = o;
    }
}

}  // namespace

hipError_t moe_launch_combine(const void* yp, moe_dtype_t dt, const float* w,
                              const int32_t* entry_pos, int T, int H, int K, void* out,
                              hipStream_t stream) {
    const int vec = dt == MOE_BF16 ? 8 : 4;
    const int64_t total = (int64_t)T * (H / vec);
    int64_t grid = (total + kThreads - 1) / kThreads;
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    if (dt == MOE_BF16)
        combine_kernel<true><<<(int)grid, kThreads, 0, stream>>>(
            static_cast<const uint8_t*>(yp), w, entry_pos, T, H, K, static_cast<uint8_t*>(out));
    else
        combine_kernel<false><<<(int)grid, kThreads, 0, stream>>>(
            static_cast<const uint8_t*>(yp), w, entry_pos, T, H, K, static_cast<uint8_t*>(out));
    return hipGetLastError();
}
