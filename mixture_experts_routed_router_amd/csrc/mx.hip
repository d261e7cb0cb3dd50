// mx.hip -- quantization into the MX formats (moe_mx_quantize).
//
// MegaFlux §4.1 (Platform and configurations): the forward pass uses MXFP4 weights and MXFP8
// activations; MoonEP's cost model: packed 4-bit elements plus one scale per 32 elements.  The
// encodings are the OCP Microscaling Formats (MX) v1.0 ones: per block of 32 consecutive values
// one E8M0 scale 2^(code - 127) with shared exponent floor(log2 max|v|) - emax (emax 8 for FP8
// E4M3, 2 for FP4 E2M1; -127 for an all-zero block), elements v / scale rounded to nearest,
// ties to even, saturating at the largest value (448 / 6).  FP4 codes pack two per byte, the
// lower-indexed element in the low nibble.
//
// Four lanes per block, eight values per lane: 16- or 32-byte loads, the block maximum from two
// lane swaps, then each lane scales its values (exactly: a power-of-two multiple) and converts
// them -- FP8 with the hardware conversion after a +-448 clamp (moe_mx.h: equal to the integer
// encoder), FP4 with integer rounding -- and stores 8 (FP8) or 4 (FP4) bytes.
#include "moe_launch.h"
#include "moe_mx.h"

namespace {

constexpr int kThreads = 256;

template <bool kBF16, bool kFP4>
__global__ void __launch_bounds__(kThreads)
mx_quantize_kernel(const uint8_t* __restrict__ src, int64_t n8, int64_t gpr, int64_t pitch,
                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    // group g = 8 consecutive values = (row, column group col); tracked incrementally over the
    // grid-stride loop (one 64-bit division at the start)
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t s_row = stride / gpr, s_col = stride - s_row * gpr;
    int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    int64_t row = g / gpr, col = g - row * gpr;
    for (; g < n8; g += stride) {
        float v[8];
        if (kBF16) {
            const uint4 u = reinterpret_cast<const uint4*>(src)[g];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = moe_bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
                v[2 * i + 1] = moe_bf16_to_f32((uint16_t)(w[i] >> 16));
            }
        } else {
            const uint4 u0 = reinterpret_cast<const uint4*>(src)[2 * g];
            const uint4 u1 = reinterpret_cast<const uint4*>(src)[2 * g + 1];
            const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
        // the block is the aligned group of 4 lanes (g % 4 == lane % 4)
        amax = fmaxf(amax, __shfl_xor(amax, 1, MOE_WAVE));
        amax = fmaxf(amax, __shfl_xor(amax, 2, MOE_WAVE));
        const int se = mx_shared_exp(amax, kFP4 ? 2 : 8);
        if ((g & 3) == 0) scales[row * pitch + (col >> 2)] = (uint8_t)(se + 127);
        float sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[i], -se);  // exact: a power-of-two scaling
        if (kFP4) {
            uint32_t packed = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t m = e2m1_code(fabsf(sv[i]));
                const uint32_t c = m | ((sv[i] < 0.f && m != 0) ? 0x8u : 0u);
                packed |= c << (4 * i);
            }
            reinterpret_cast<uint32_t*>(codes)[g] = packed;
        } else {
            uint2 o;
            o.x = e4m3_word(sv[0], sv[1], sv[2], sv[3]);
            o.y = e4m3_word(sv[4], sv[5], sv[6], sv[7]);
            reinterpret_cast<uint2*>(codes)[g] = o;
        }
        col += s_col;
        row += s_row;
        if (col >= gpr) {
            col -= gpr;
            row += 1;
        }
    }
}

}  // namespace

hipError_t moe_launch_mx_quantize(const void* src, moe_dtype_t dt, int64_t rows, int64_t cols,
                                  int fmt, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    const int64_t n8 = rows * cols / 8, gpr = cols / 8, pitch = moe_mx_scale_pitch_impl(cols);
    int64_t grid = (n8 + kThreads - 1) / kThreads;
    if (grid > 8192) grid = 8192;
    if (grid < 1) return hipSuccess;
    const uint8_t* s = static_cast<const uint8_t*>(src);
    if (dt == MOE_BF16) {
        if (fmt == MOE_MX_FP4)
            mx_quantize_kernel<true, true><<<(int)grid, kThreads, 0, stream>>>(s, n8, gpr, pitch, codes, scales);
        else
            mx_quantize_kernel<true, false><<<(int)grid, kThreads, 0, stream>>>(s, n8, gpr, pitch, codes, scales);
    } else {
        if (fmt == MOE_MX_FP4)
            mx_quantize_kernel<false, true><<<(int)grid, kThreads, 0, stream>>>(s, n8, gpr, pitch, codes, scales);
        else
            mx_quantize_kernel<false, false><<<(int)grid, kThreads, 0, stream>>>(s, n8, gpr, pitch, codes, scales);
    }
    return hipGetLastError();
}
