// moe_lds.h -- gfx950 direct-to-LDS staging helpers shared by the GEMM kernels.
#pragma once
#include "moe_device.h"

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

// Row r's logical 16-byte chunk c of a 128-byte row is stored at physical chunk
// c ^ ((r >> 1) & 7): a ds_read_b128 serves 16 lanes at a time over 64 four-byte banks, and
// 16 consecutive rows reading one logical chunk then land in 16 distinct bank groups (r & 1
// picks the 128-byte half of a 256-byte bank line, the XOR the group in it), provided rows
// sit at 128-byte strides in segments that start on multiples of 256 bytes.
__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }

// Four copies of one stage for this wave straight from global memory into LDS (gfx950
// global_load_lds_dwordx4, scalar base + 32-bit lane offset): copy i moves 16 B per lane to
// LDS address M0 + 1024 i + 16 lane from base_i + lane offset + 1024 i (the scalar bases are
// passed pre-biased by -1024 i).  Issued from inline asm so that the compiler does not drain
// every outstanding copy before each LDS access; the kernel waits with explicit vmcnt counts
// and a barrier instead.  M0 is saved and restored.  With `two` false only copies 0 and 1 go.
__device__ __forceinline__ void four_copies(uint32_t m0, const void* b0, const void* b1,
                                            const void* b2, const void* b3, uint32_t o0,
                                            uint32_t o1, uint32_t o2, uint32_t o3, bool two) {
    uint32_t saved;
    if (two)
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %5\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %6\n\t"
            "global_load_lds_dwordx4 %2, %7 offset:1024\n\t"
            "global_load_lds_dwordx4 %3, %8 offset:2048\n\t"
            "global_load_lds_dwordx4 %4, %9 offset:3072\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(o0), "v"(o1), "v"(o2), "v"(o3), "s"(m0), "s"(b0), "s"(b1), "s"(b2), "s"(b3)
            : "memory");
    else
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %3\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %4\n\t"
            "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
            "s_nop 0\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(o0), "v"(o1), "s"(m0), "s"(b0), "s"(b1)
            : "memory");
}

// One copy: 16 B per lane from base + lane offset to LDS address M0 + 16 lane.
__device__ __forceinline__ void one_copy(uint32_t m0, const void* base, uint32_t off) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(m0), "s"(base)
        : "memory");
}

// One 4-byte copy: 4 B per lane from base + lane offset to LDS address M0 + 4 lane.
__device__ __forceinline__ void one_copy_dword(uint32_t m0, const void* base, uint32_t off) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, %3\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(m0), "s"(base)
        : "memory");
}

// Wait until at most n of this wave's copies are outstanding, then meet the workgroup.
// n = pending stages (0, 1 or 2) x copies per stage (8, 7, 6 or 5).
#define MOE_WAIT_CASE(n)                                                                      \
    case n:                                                                                   \
        asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); \
        break;
__device__ __forceinline__ void wait_copies_and_barrier(int n) {
    switch (n) {
        MOE_WAIT_CASE(14)
        MOE_WAIT_CASE(12)
        MOE_WAIT_CASE(10)
        MOE_WAIT_CASE(8)
        MOE_WAIT_CASE(7)
        MOE_WAIT_CASE(6)
        MOE_WAIT_CASE(5)
        default:
            asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            break;
    }
}
#undef MOE_WAIT_CASE

// Wait until at most N of this wave's copies are outstanding, then meet the workgroup
// (N a compile-time constant).
template <int N>
__device__ __forceinline__ void wait_copies_n_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// wait_copies_n_and_barrier<p * CPW> for a runtime p in [0, MAXP].
template <int CPW, int MAXP>
__device__ __forceinline__ void wait_pending_stages(int p) {
    if constexpr (MAXP > 0) {
        if (p >= MAXP) {
            wait_copies_n_and_barrier<MAXP * CPW>();
            return;
        }
        wait_pending_stages<CPW, MAXP - 1>(p);
    } else {
        wait_copies_n_and_barrier<0>();
    }
}
