// moe_mx.h -- element encoders of the OCP MX formats (shared by the quantizer and the MX
// expert GEMM's activation epilogue): E2M1 by integer rounding, E4M3 by the hardware
// conversion, and the E8M0 shared exponent.
#pragma once
#include "moe_device.h"

// |a| -> E2M1 magnitude code (values 0, 0.5, 1, 1.5, 2, 3, 4, 6), nearest, ties even, saturating.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
    if (a >= 6.f) return 0x7;
    if (a < 1.f) return (uint32_t)rintf(a * 2.f);  // 0, 0.5 (1), 1.0 (2)
    const int e = ilogbf(a);                          // 0, 1 or 2
    int q = (int)rintf((ldexpf(a, -e) - 1.f) * 2.f);
    int eb = e + 1;
    if (q == 2) {
        q = 0;
        eb += 1;
    }
    const uint32_t c = ((uint32_t)eb << 1) | (uint32_t)q;
    return c > 0x7 ? 0x7 : c;
}

// E8M0 shared exponent of a block whose largest magnitude is amax (finite, float32):
// floor(log2 amax) - emax, clamped to [-127, 127]; -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(float amax, int emax) {
    if (!(amax > 0.f)) return -127;
    const int e = ilogbf(amax) - emax;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four float32 values (already divided by the block scale) -> their E4M3 codes in one word,
// value j in byte j: clamped to +-448 (saturation), then the hardware conversion (nearest,
// ties to even); a zero result loses its sign.  Equal to an integer nearest-even encoder of the
// same rule for every finite input (checked on the GPU over all float32 mantissas at stride 2^9
// across the E4M3 range, and at every code and midpoint, both signs).
__device__ __forceinline__ uint32_t e4m3_word(float v0, float v1, float v2, float v3) {
    v0 = __builtin_amdgcn_fmed3f(v0, -448.f, 448.f);
    v1 = __builtin_amdgcn_fmed3f(v1, -448.f, 448.f);
    v2 = __builtin_amdgcn_fmed3f(v2, -448.f, 448.f);
    v3 = __builtin_amdgcn_fmed3f(v3, -448.f, 448.f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    const uint32_t u = (uint32_t)w;
    const uint32_t nz = ((u & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7: magnitude != 0
    return u & (0x7F7F7F7Fu | nz);
}
