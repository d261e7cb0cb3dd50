// route.hip -- router top-k, routing weights and expert histogram (moe_route).
//
// MegaFlux §1: a router sends each token to k experts whose outputs are mixed by routing
// weights; §4.1: the k experts of a token are distinct.  The top-k renormalisation abstract
// (Daily Papers listing): the picked experts' probabilities are renormalised over the picks.
//
// One wavefront per token.  Lane j holds logits j, j+64, j+128, j+192 (E <= 256) in
// registers; K rounds of a wave-wide arg-max under the total order (larger logit, then
// smaller id) pick the experts, so ties resolve to the lower id and every lane agrees on the
// winner.  Lane k keeps slot k; the weights are a softmax over the K picks (or all E).  The
// expert histogram is counted in LDS per workgroup (integer adds: order-independent) and
// flushed with one global atomic per nonzero bin.
#include "moe_launch.h"

namespace {

constexpr int kRouteThreads = 256;

__global__ void __launch_bounds__(kRouteThreads)
zero_i32_kernel(int32_t* __restrict__ p, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

template <int EPL>
__global__ void __launch_bounds__(kRouteThreads)
route_kernel(const float* __restrict__ logits, int T, int E, int K, int renormalize,
             int tokens_per_block, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
             int32_t* __restrict__ counts) {
    __shared__ int hist[256];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();

    const int lane = moe_lane_id();
    const int wave = threadIdx.x / MOE_WAVE;
    const int nwaves = blockDim.x / MOE_WAVE;
    const int t_begin = blockIdx.x * tokens_per_block;
    const int t_end = min(T, t_begin + tokens_per_block);

    for (int t = t_begin + wave; t < t_end; t += nwaves) {
        const float* row = logits + (size_t)t * E;
        float v[EPL];
        uint32_t taken = 0;  // bit j: logit lane + 64*j already picked (or absent)
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            int e = lane + MOE_WAVE * j;
            if (e < E) {
                v[j] = row[e];
            } else {
                v[j] = -INFINITY;
                taken |= 1u << j;
            }
        }
        float my_v = 0.f;
        int my_e = 0;
        for (int k = 0; k < K; ++k) {
            float bv = -INFINITY;
            int be = 0x7FFFFFFF;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                int e = lane + MOE_WAVE * j;
                if (!((taken >> j) & 1u) && (v[j] > bv || (v[j] == bv && e < be))) {
                    bv = v[j];
                    be = e;
                }
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                float ov = __shfl_xor(bv, off, MOE_WAVE);
                int oe = __shfl_xor(be, off, MOE_WAVE);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            if ((be & (MOE_WAVE - 1)) == lane) taken |= 1u << (be / MOE_WAVE);
            if (lane == k) {
                my_v = bv;
                my_e = be;
            }
        }
        const float m = __shfl(my_v, 0, MOE_WAVE);
        const float ex = lane < K ? expf(my_v - m) : 0.f;
        float denom;
        if (renormalize) {
            denom = moe_wave_sum_f32(ex);
        } else {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (lane + MOE_WAVE * j < E) s += expf(v[j] - m);
            denom = moe_wave_sum_f32(s);
        }
        if (lane < K) {
            topk_ids[(size_t)t * K + lane] = my_e;
            topk_w[(size_t)t * K + lane] = ex / denom;
            atomicAdd(&hist[my_e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int c = hist[e];
        if (c) atomicAdd(&counts[e], c);
    }
}

}  // namespace

hipError_t moe_launch_route(const float* logits, int T, int E, int K, int renormalize,
                            int32_t* topk_ids, float* topk_w, int32_t* counts,
                            hipStream_t stream) {
    zero_i32_kernel<<<(E + kRouteThreads - 1) / kRouteThreads, kRouteThreads, 0, stream>>>(counts, E);
    // about 1024 workgroups: enough to fill the chip, few histogram flushes
    int waves_per_block = kRouteThreads / MOE_WAVE;
    int tpb = (T + 1023) / 1024;
    tpb = (tpb + waves_per_block - 1) / waves_per_block * waves_per_block;
    if (tpb < waves_per_block) tpb = waves_per_block;
    int grid = (T + tpb - 1) / tpb;
    int epl = (E + MOE_WAVE - 1) / MOE_WAVE;
    if (epl == 1)
        route_kernel<1><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, renormalize, tpb,
                                                            topk_ids, topk_w, counts);
    else if (epl == 2)
        route_kernel<2><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, renormalize, tpb,
                                                            topk_ids, topk_w, counts);
    else
        route_kernel<4><<<grid, kRouteThreads, 0, stream>>>(logits, T, E, K, renormalize, tpb,
                                                            topk_ids, topk_w, counts);
    return hipGetLastError();
}
