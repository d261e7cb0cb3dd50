// ffn.hip -- SwiGLU expert FFN over the plan's block table (moe_expert_ffn).
//
// MegaFlux §2.1: FC1 (gate and up projections) then FC2; §4.1: SwiGLU experts, FP32
// accumulation, BF16 outputs; §3.1: the token dimension of the expert GEMM tiles is the
// plan's block of at most beta rows.  The fused gate+up idea (both projections from the same
// input tile, activation applied in registers) is the one the TritonMoE abstract (Daily Papers
// listing) describes.
//
// bf16 path: two grouped GEMMs on v_mfma_f32_32x32x16_bf16.
//   gate/up: per (block, 64 act columns): a 128-row A tile of xp times 128 rows of W1 (64 gate
//            rows n0.. and the 64 up rows I+n0..), then act = SiLU(g) * u in registers.
//   down:    per (block, 128 columns of H): act tile times 128 rows of W2.
// Both operands are K-contiguous (C = A * B^T), so each lane's MFMA fragment is one 16-byte
// LDS read.  Tiles are staged through LDS in 64-wide K slices, double buffered, rows XOR-
// swizzled in 16-byte chunks so the fragment reads of 8 consecutive rows hit distinct banks.
// Four waves per workgroup in a 2 x 2 grid, each owning 64 rows x 64 B-rows (2 x 2 MFMA
// tiles).  The grid is persistent: workgroup w runs on XCD w % 8 and walks a contiguous slice
// of the (block, column tile) items, so items that share A rows run on the same XCD's L2.
// The block count is read on the device; there is no host round trip.
#include "moe_launch.h"

namespace {

constexpr int BM = 128;      // rows per tile (= the plan's block of <= 128 rows)
constexpr int BN = 256;      // B rows per tile (FC1: 128 gate + 128 up; FC2: 256 columns of H)
constexpr int BK = 64;       // K slice per LDS stage
constexpr int STAGES = 3;    // LDS ring depth: two slices in flight while one is consumed
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int A_STAGE_BYTES = BM * BK * 2;                  // 16 KB
constexpr int B_STAGE_BYTES = BN * BK * 2;                  // 32 KB
constexpr int STAGE_BYTES = A_STAGE_BYTES + B_STAGE_BYTES;  // 48 KB
constexpr int LOADS_PER_STAGE = STAGE_BYTES / (kThreads * 16);  // 12 x 16 B per thread

typedef __attribute__((address_space(3))) uint8_t lds_u8_t;

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int row, int ch) {
    // 16-byte chunk `ch` of row `row` in a [rows][64] bf16 tile whose chunks are XOR-swizzled
    // by (row & 7): 8 consecutive rows reading one logical chunk hit 8 different bank groups.
    const uint4 v = *reinterpret_cast<const uint4*>(base + row * (BK * 2) + ((ch ^ (row & 7)) << 4));
    return __builtin_bit_cast(bf16x8_t, v);
}

// 16 bytes per lane from global memory straight into LDS (gfx950 global_load_lds_dwordx4):
// lane i's bytes land at LDS address lds_addr + 16 * i.  Issued from inline asm so that the
// compiler does not drain every outstanding copy before each LDS access; the caller waits
// with vmcnt and a barrier instead.  M0 (the LDS base) is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_addr) {
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(gptr), "s"(lds_addr)
        : "memory");
}

// All but the newest stage's copies of this wave have landed; then the whole workgroup meets.
#define MOE_WAIT_STAGE_AND_BARRIER() \
    asm volatile("s_waitcnt vmcnt(12)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define MOE_WAIT_ALL_AND_BARRIER() \
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// One grouped GEMM over the block table: C[p][n] for rows p of each block (expert l),
//   FC1 (kSwiGLU): act[p][c] = SiLU(A[p].W1[l][c]) * (A[p].W1[l][I + c]), c < I
//   FC2:           yp[p][c]  = A[p].W2[l][c],                              c < H
// A is [a_rows, Kdim], B per expert [b_rows, Kdim]; both K-contiguous.
template <bool kSwiGLU>
__global__ void __launch_bounds__(kThreads, 1)
ffn_bf16_kernel(const uint16_t* __restrict__ A, int64_t a_rows, int Kdim,
                const uint16_t* __restrict__ B, int64_t b_expert_stride, int b_rows,
                uint16_t* __restrict__ C, int ldc, int n_cols, int I, int NT,
                const int32_t* __restrict__ blocks, const int32_t* __restrict__ n_blocks_ptr,
                int max_blocks) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

    static_assert(LOADS_PER_STAGE == 12, "the stage wait below counts 12 copies per thread");
    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_u8_t*)smem;

    int nb = *n_blocks_ptr;
    nb = nb < max_blocks ? nb : max_blocks;
    const int total = nb * NT;
    // persistent grid: XCD x (= blockIdx % 8) walks the x-th eighth of the items in order
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int per_xcd_wgs = gridDim.x / kXcds;
    const int per_xcd_items = (total + kXcds - 1) / kXcds;
    const int it_begin = xcd * per_xcd_items;
    const int it_end = min(total, it_begin + per_xcd_items);

    // Direct-to-LDS loads: each instruction moves 64 lanes x 16 B = 8 rows of a stage.
    // Load i of this wave fills 8-row segment (i * 4 + wave): A segments 0..15, B 16..47.
    // Lane j writes LDS chunk j of its segment: row j/8, physical chunk j%8, which holds
    // logical chunk (j%8) ^ (j/8) (the read-side swizzle).
    const int seg_row = lane >> 3;
    const int seg_lchunk = (lane & 7) ^ (lane >> 3);
    const int nk = Kdim / BK;

    for (int it = it_begin + slot; it < it_end; it += per_xcd_wgs) {
        const int b = it / NT;
        const int nt = it - b * NT;
        const int l = blocks[4 * b + 1];
        const int blk_row0 = blocks[4 * b + 2];
        const int blk_rows = blocks[4 * b + 3];
        const uint16_t* Bexp = B + (int64_t)l * b_expert_stride;

        for (int sub = 0; sub < blk_rows; sub += BM) {  // blocks of 256 rows take two tiles
            const int row0 = blk_row0 + sub;
            const int m = blk_rows - sub < BM ? blk_rows - sub : BM;

            const uint16_t* src[LOADS_PER_STAGE];
#pragma unroll
            for (int i = 0; i < LOADS_PER_STAGE; ++i) {
                const int segm = i * 4 + wave;
                if (segm < BM / 8) {
                    int64_t ar = row0 + segm * 8 + seg_row;
                    if (ar > a_rows - 1) ar = a_rows - 1;  // rows past the block: read, unused
                    src[i] = A + ar * Kdim + seg_lchunk * 8;
                } else {
                    const int rr = (segm - BM / 8) * 8 + seg_row;
                    int br;
                    if (kSwiGLU)
                        br = rr < BN / 2 ? nt * (BN / 2) + rr : I + nt * (BN / 2) + (rr - BN / 2);
                    else
                        br = nt * BN + rr;
                    if (br > b_rows - 1) br = b_rows - 1;  // columns past H: read, not stored
                    src[i] = Bexp + (int64_t)br * Kdim + seg_lchunk * 8;
                }
            }
            auto issue = [&](int kt) {
                const uint32_t stage = smem_base + (kt % STAGES) * STAGE_BYTES;
#pragma unroll
                for (int i = 0; i < LOADS_PER_STAGE; ++i)
                    lds_dma16(src[i] + kt * BK, stage + (i * 4 + wave) * 1024);
            };

            f32x16_t acc[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

            __syncthreads();  // the previous tile's last LDS reads are done
            issue(0);
            if (nk > 1) issue(1);

            for (int kt = 0; kt < nk; ++kt) {
                // slice kt has landed in every wave's share of its stage (kt+1 may be in flight)
                if (kt + 1 < nk)
                    MOE_WAIT_STAGE_AND_BARRIER();
                else
                    MOE_WAIT_ALL_AND_BARRIER();
                if (kt + 2 < nk) issue(kt + 2);   // refills the stage read in iteration kt-1

                const uint8_t* As = smem + (kt % STAGES) * STAGE_BYTES;
                const uint8_t* Bs = As + A_STAGE_BYTES;
#pragma unroll
                for (int kk = 0; kk < BK / 16; ++kk) {
                    const int ch = kk * 2 + (lane >> 5);
                    bf16x8_t bfr[2], af[4];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int br = kSwiGLU ? j * (BN / 2) + wave * 32 + (lane & 31)
                                               : wave * 64 + j * 32 + (lane & 31);
                        bfr[j] = lds_frag(Bs, br, ch);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) af[i] = lds_frag(As, i * 32 + (lane & 31), ch);
                    // D = B-rows x A-rows: lane keeps one A row and 4 consecutive columns per
                    // register group, so the epilogue stores 8 bytes at a time
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                bfr[j], af[i], acc[i][j], 0, 0, 0);
                }
            }

            // epilogue: acc[i][j][4g + e] = C[row i*32 + lane%32][col base + 8g + 4(lane/32) + e]
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = i * 32 + (lane & 31);
                if (rl >= m) continue;
                uint16_t* crow = C + (int64_t)(row0 + rl) * ldc;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c4 = 8 * g + 4 * (lane >> 5);
                    if (kSwiGLU) {
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float gt = acc[i][0][4 * g + e];
                            const float up = acc[i][1][4 * g + e];
                            v[e] = gt / (1.f + expf(-gt)) * up;
                        }
                        const int col = nt * (BN / 2) + wave * 32 + c4;
                        if (col < n_cols) {  // n_cols is a multiple of 64: all 4 or none
                            uint2 o;
                            o.x = moe_pack_bf16x2(v[0], v[1]);
                            o.y = moe_pack_bf16x2(v[2], v[3]);
                            *reinterpret_cast<uint2*>(crow + col) = o;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            const int col = nt * BN + wave * 64 + j * 32 + c4;
                            if (col < n_cols) {  // n_cols is a multiple of 64: all 4 or none
                                uint2 o;
                                o.x = moe_pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
                                o.y = moe_pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                                *reinterpret_cast<uint2*>(crow + col) = o;
                            }
                        }
                    }
                }
            }
        }
    }
}

// float32 path (small layers): one thread per output element, sequential K loop.
__global__ void __launch_bounds__(256)
ffn_f32_gateup_kernel(const float* __restrict__ xp, const float* __restrict__ w1, int H, int I,
                      const int32_t* __restrict__ blocks, const int32_t* __restrict__ n_blocks_ptr,
                      int max_blocks, float* __restrict__ act) {
    int nb = *n_blocks_ptr;
    nb = nb < max_blocks ? nb : max_blocks;
    for (int b = blockIdx.x; b < nb; b += gridDim.x) {
        const int l = blocks[4 * b + 1], row0 = blocks[4 * b + 2], m = blocks[4 * b + 3];
        const float* wg = w1 + (int64_t)l * 2 * I * H;
        for (int idx = threadIdx.x; idx < m * I; idx += blockDim.x) {
            const int r = idx / I, i = idx - r * I;
            const float* x = xp + (int64_t)(row0 + r) * H;
            const float* g_row = wg + (int64_t)i * H;
            const float* u_row = wg + (int64_t)(I + i) * H;
            float g = 0.f, u = 0.f;
            for (int h = 0; h < H; ++h) {
                g = fmaf(x[h], g_row[h], g);
                u = fmaf(x[h], u_row[h], u);
            }
            act[(int64_t)(row0 + r) * I + i] = g / (1.f + expf(-g)) * u;
        }
    }
}

__global__ void __launch_bounds__(256)
ffn_f32_down_kernel(const float* __restrict__ act, const float* __restrict__ w2, int H, int I,
                    const int32_t* __restrict__ blocks, const int32_t* __restrict__ n_blocks_ptr,
                    int max_blocks, float* __restrict__ yp) {
    int nb = *n_blocks_ptr;
    nb = nb < max_blocks ? nb : max_blocks;
    for (int b = blockIdx.x; b < nb; b += gridDim.x) {
        const int l = blocks[4 * b + 1], row0 = blocks[4 * b + 2], m = blocks[4 * b + 3];
        const float* w = w2 + (int64_t)l * H * I;
        for (int idx = threadIdx.x; idx < m * H; idx += blockDim.x) {
            const int r = idx / H, h = idx - r * H;
            const float* a = act + (int64_t)(row0 + r) * I;
            const float* w_row = w + (int64_t)h * I;
            float y = 0.f;
            for (int i = 0; i < I; ++i) y = fmaf(a[i], w_row[i], y);
            yp[(int64_t)(row0 + r) * H + h] = y;
        }
    }
}

int persistent_grid(int wgs_per_cu) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    int g = cus * wgs_per_cu;
    g = g / kXcds * kXcds;
    return g < kXcds ? kXcds : g;
}

}  // namespace

hipError_t moe_launch_ffn_fc1(const void* xp, const void* w1, moe_dtype_t dt, int H, int I,
                              const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                              void* act, int64_t max_rows, hipStream_t stream) {
    if (dt == MOE_F32) {
        int grid = max_blocks < 1024 ? max_blocks : 1024;
        ffn_f32_gateup_kernel<<<grid, 256, 0, stream>>>(
            static_cast<const float*>(xp), static_cast<const float*>(w1), H, I, blocks, n_blocks,
            max_blocks, static_cast<float*>(act));
        return hipGetLastError();
    }
    ffn_bf16_kernel<true><<<persistent_grid(1), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(xp), max_rows, H, static_cast<const uint16_t*>(w1),
        (int64_t)2 * I * H, 2 * I, static_cast<uint16_t*>(act), I, I, I,
        (I + BN / 2 - 1) / (BN / 2), blocks,
        n_blocks, max_blocks);
    return hipGetLastError();
}

hipError_t moe_launch_ffn_fc2(const void* act, const void* w2, moe_dtype_t dt, int H, int I,
                              const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                              void* yp, int64_t max_rows, hipStream_t stream) {
    if (dt == MOE_F32) {
        int grid = max_blocks < 1024 ? max_blocks : 1024;
        ffn_f32_down_kernel<<<grid, 256, 0, stream>>>(
            static_cast<const float*>(act), static_cast<const float*>(w2), H, I, blocks,
            n_blocks, max_blocks, static_cast<float*>(yp));
        return hipGetLastError();
    }
    ffn_bf16_kernel<false><<<persistent_grid(1), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(act), max_rows, I, static_cast<const uint16_t*>(w2),
        (int64_t)H * I, H, static_cast<uint16_t*>(yp), H, H, I, (H + BN - 1) / BN, blocks,
        n_blocks, max_blocks);
    return hipGetLastError();
}
