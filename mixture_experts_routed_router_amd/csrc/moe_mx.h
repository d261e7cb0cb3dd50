// moe_mx.h -- element encoders of the OCP MX formats (shared by the quantizer and the MX
// expert GEMM's activation epilogue).
#pragma once
#include "moe_device.h"

// |a| (finite, already divided by the block scale) -> E4M3 magnitude code, nearest, ties even,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_code(float a) {
    if (a >= 448.f) return 0x7E;
    if (a < 0.015625f) return (uint32_t)rintf(a * 512.f);  // subnormal: units of 2^-9 (8 = 2^-6)
    const int e = ilogbf(a);                                // 2^e <= a < 2^(e+1), e in [-6, 8]
    int q = (int)rintf((ldexpf(a, -e) - 1.f) * 8.f);
    int eb = e + 7;
    if (q == 8) {
        q = 0;
        eb += 1;
    }
    const uint32_t c = ((uint32_t)eb << 3) | (uint32_t)q;
    return c > 0x7E ? 0x7E : c;
}

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
