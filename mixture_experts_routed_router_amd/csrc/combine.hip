// combine.hip -- routing-weight combine of each token's expert outputs (moe_combine).
//
// MegaFlux §1: expert outputs are mixed by the routing weights; §2.1: the final top-k sum is
// a step of its own; App. A.2: token ids, top-k slots and weights are kept for it.  The
// weighted scatter-add is done in its gather form: each output element reads the K rows its
// token's entries landed in (entry_pos), so every output is written once, with no atomics,
// and the sum runs in a fixed order (ascending k, float32).
//
// One wavefront per token (grid-stride): lane k < K loads entry k's row and weight once; the
// wave reads them back uniformly (readlane, scalar registers), skips non-local entries, and
// walks the output row in 16-byte chunks (8 bf16 or 4 float32 per lane, stored non-temporally).
// With four or more local entries it issues the loads of all entries for 2 chunks per lane before
// their FMAs; with fewer it takes 4 chunks per lane at once, entry by entry, so either way a wave
// has several KB of loads in flight.  Rows of yp and out are read / written in coalesced 1 KB
// runs per wave instruction; the sum runs over k in ascending order in both paths.
//
// Direct rows (moe_expert_ffn_fc2_direct + moe_combine_multi): a token with exactly one local
// entry sums one weighted row, bf16(fmaf(w, y, 0)), which the down GEMM's epilogue can store
// itself, bit for bit, into the token's output row.  That removes the reading of its expert
// row and the second writing of its output row from this pass: on one GPU's 32-expert share of
// a 256-expert top-8 layer about half the tokens are such tokens.  direct_rows_kernel marks the
// rows; the combine then skips those tokens (skip_one).
#include "moe_launch.h"

namespace {

constexpr int kThreads = 256;

// out is written once and not read again by the path: 16-byte non-temporal stores (3-4% faster
// on the larger layers, neutral on the OLMoE shape; non-temporal loads of yp were slower there).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt16(uint4 v, uint4* p) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// out chunk (16 bytes) from the weighted entry chunks, ascending k; v[k] holds entry k's chunk
template <bool kBF16>
__device__ __forceinline__ void fma_chunk(float (&acc)[8], const uint4& v, float wk) {
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

template <bool kBF16>
__device__ __forceinline__ uint4 pack_chunk(const float (&acc)[8]) {
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
    return o;
}

// Chunks per lane taken at once when a token has few local entries (one GPU's expert share:
// mostly one), so that a wave keeps 4 KB of loads in flight instead of 1 KB (8 chunks
// measured faster still on the one-entry shape but cost the dense path occupancy).
constexpr int kSparseChunks = 4;
// Chunks per lane with four or more local entries: two keep 2 KB per entry in flight per wave
// (3-22% faster than one chunk after the down GEMM on the workloads' shapes; four chunks were
// no faster on the large-H shapes and slower on the DeepSeek-V3 share).
constexpr int kDenseChunks = 2;

// KM: the top-k bound the kernel is unrolled for (4, 8 or 16 >= K).  kSkipOne: tokens with
// exactly one local entry are left alone (their rows were written by the down GEMM).
template <bool kBF16, int KM, bool kSkipOne>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const uint8_t* __restrict__ yp, const float* __restrict__ w,
               const int32_t* __restrict__ entry_pos, int T, int H, int K,
               uint8_t* __restrict__ out) {
    const int lane = moe_lane_id();
    const int64_t row_bytes = (int64_t)H * (kBF16 ? 2 : 4);
    const int n16 = (int)(row_bytes / 16);
    const int waves = gridDim.x * (kThreads / MOE_WAVE);
    for (int t = blockIdx.x * (kThreads / MOE_WAVE) + threadIdx.x / MOE_WAVE; t < T; t += waves) {
        int my_p = -1;
        float my_w = 0.f;
        if (lane < K) {
            my_p = entry_pos[(int64_t)t * K + lane];
            my_w = w[(int64_t)t * K + lane];
        }
        uint4* orow = reinterpret_cast<uint4*>(out + (int64_t)t * row_bytes);
        const int n_local = __popcll(__ballot(my_p >= 0));
        if (kSkipOne && n_local == 1) continue;  // wave-uniform
        if (n_local >= 4) {
            // many entries: kDenseChunks chunks per lane, the loads of all entries before the FMAs
            for (int c0 = lane; c0 < n16; c0 += MOE_WAVE * kDenseChunks) {
                // wave-uniform entry rows/weights (readlane: loop-invariant scalars)
                uint4 v[KM][kDenseChunks];
#pragma unroll
                for (int k = 0; k < KM; ++k) {
                    if (k < K) {
                        const int p = __builtin_amdgcn_readlane(my_p, k);
                        if (p >= 0) {
                            const uint4* row = reinterpret_cast<const uint4*>(yp + (int64_t)p * row_bytes);
#pragma unroll
                            for (int u = 0; u < kDenseChunks; ++u)
                                if (c0 + u * MOE_WAVE < n16) v[k][u] = row[c0 + u * MOE_WAVE];
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < kDenseChunks; ++u) {
                    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < KM; ++k) {
                        if (k < K && __builtin_amdgcn_readlane(my_p, k) >= 0) {
                            const float wk = __builtin_bit_cast(
                                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), k));
                            fma_chunk<kBF16>(acc, v[k][u], wk);
                        }
                    }
                    if (c0 + u * MOE_WAVE < n16) store_nt16(pack_chunk<kBF16>(acc), orow + c0 + u * MOE_WAVE);
                }
            }
        } else {
            // few entries (or none: zeros): kSparseChunks chunks per lane, entry by entry
            for (int c0 = lane; c0 < n16; c0 += MOE_WAVE * kSparseChunks) {
                float acc[kSparseChunks][8];
#pragma unroll
                for (int u = 0; u < kSparseChunks; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
                for (int k = 0; k < K; ++k) {
                    const int p = __builtin_amdgcn_readlane(my_p, k);
                    if (p < 0) continue;
                    const float wk = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), k));
                    const uint4* row = reinterpret_cast<const uint4*>(yp + (int64_t)p * row_bytes);
                    uint4 v[kSparseChunks];
#pragma unroll
                    for (int u = 0; u < kSparseChunks; ++u) {
                        const int c = c0 + u * MOE_WAVE;
                        if (c < n16) v[u] = row[c];
                    }
#pragma unroll
                    for (int u = 0; u < kSparseChunks; ++u)
                        if (c0 + u * MOE_WAVE < n16) fma_chunk<kBF16>(acc[u], v[u], wk);
                }
#pragma unroll
                for (int u = 0; u < kSparseChunks; ++u) {
                    const int c = c0 + u * MOE_WAVE;
                    if (c < n16) store_nt16(pack_chunk<kBF16>(acc[u]), orow + c);
                }
            }
        }
    }
}

template <bool kBF16, bool kSkipOne>
void launch_km(int grid, hipStream_t stream, const uint8_t* yp, const float* w,
               const int32_t* entry_pos, int T, int H, int K, uint8_t* out) {
    if (K <= 4)
        combine_kernel<kBF16, 4, kSkipOne><<<grid, kThreads, 0, stream>>>(yp, w, entry_pos, T, H, K, out);
    else if (K <= 8)
        combine_kernel<kBF16, 8, kSkipOne><<<grid, kThreads, 0, stream>>>(yp, w, entry_pos, T, H, K, out);
    else
        combine_kernel<kBF16, 16, kSkipOne><<<grid, kThreads, 0, stream>>>(yp, w, entry_pos, T, H, K, out);
}

// dir[p] = t and dir[max_rows + p] = the bits of w[t][k] when row p is the only local entry
// (slot k) of its token t = row_token[p]; dir[p] = -1 (weight word 0) for every other row,
// padding and rows past the permutation included, so that the table describes all max_rows
// rows whatever a block table covers.  One thread per row; the token's K entry_pos words are
// read to count its local entries, as the combine counts them.
__global__ void __launch_bounds__(kThreads)
direct_rows_kernel(const int32_t* __restrict__ row_token, const int32_t* __restrict__ entry_pos,
                   const float* __restrict__ w, int T, int K, int64_t max_rows,
                   int32_t* __restrict__ dir) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < max_rows; p += stride) {
        const int t = row_token[p];
        int tok = -1;
        int wbits = 0;
        if (t >= 0 && t < T) {
            int n = 0, kk = -1;
            for (int k = 0; k < K; ++k) {
                const int e = entry_pos[(int64_t)t * K + k];
                if (e >= 0) {
                    ++n;
                    if (e == p) kk = k;
                }
            }
            if (n == 1 && kk >= 0) {
                tok = t;
                wbits = __float_as_int(w[(int64_t)t * K + kk]);
            }
        }
        dir[p] = tok;
        dir[max_rows + p] = wbits;
    }
}

}  // namespace

hipError_t moe_launch_direct_rows(const int32_t* row_token, const int32_t* entry_pos,
                                  const float* w, int T, int K, int64_t max_rows, int32_t* dir,
                                  hipStream_t stream) {
    int64_t grid = (max_rows + kThreads - 1) / kThreads;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    direct_rows_kernel<<<(int)grid, kThreads, 0, stream>>>(row_token, entry_pos, w, T, K,
                                                           max_rows, dir);
    return hipGetLastError();
}

hipError_t moe_launch_combine(const void* yp, moe_dtype_t dt, const float* w,
                              const int32_t* entry_pos, int T, int H, int K, void* out,
                              hipStream_t stream, bool skip_one) {
    const int waves_per_block = kThreads / MOE_WAVE;
    int64_t grid = ((int64_t)T + waves_per_block - 1) / waves_per_block;
    // grid-stride beyond 32K waves (3% faster than 16K on the 32-expert share of a 256-expert
    // layer, where a token has about one local entry; the same elsewhere)
    if (grid > 8192) grid = 8192;
    const uint8_t* y = static_cast<const uint8_t*>(yp);
    uint8_t* o = static_cast<uint8_t*>(out);
    if (dt == MOE_BF16) {
        if (skip_one)
            launch_km<true, true>((int)grid, stream, y, w, entry_pos, T, H, K, o);
        else
            launch_km<true, false>((int)grid, stream, y, w, entry_pos, T, H, K, o);
    } else {
        if (skip_one)
            launch_km<false, true>((int)grid, stream, y, w, entry_pos, T, H, K, o);
        else
            launch_km<false, false>((int)grid, stream, y, w, entry_pos, T, H, K, o);
    }
    return hipGetLastError();
}
