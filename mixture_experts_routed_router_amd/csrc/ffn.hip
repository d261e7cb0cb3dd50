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

constexpr int BM = 128;  // rows per tile (= max block rows)
constexpr int BN = 128;  // B rows per tile
constexpr int BK = 64;   // K slice per LDS stage
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// LDS element offset of 16-byte chunk `ch` of row `row` in a [rows][64] bf16 tile.
__device__ __forceinline__ int swz(int row, int ch) { return row * BK + ((ch ^ (row & 7)) << 3); }

template <bool kSwiGLU>
__global__ void __launch_bounds__(kThreads, 2)
ffn_bf16_kernel(const uint16_t* __restrict__ A, int64_t a_rows, int Kdim,
                const uint16_t* __restrict__ B, int64_t b_expert_stride, int b_rows,
                uint16_t* __restrict__ C, int ldc, int n_cols, int I, int NT,
                const int32_t* __restrict__ blocks, const int32_t* __restrict__ n_blocks_ptr,
                int max_blocks) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int wave = tid / MOE_WAVE;
    const int wm = wave >> 1, wn = wave & 1;

    int nb = *n_blocks_ptr;
    nb = nb < max_blocks ? nb : max_blocks;
    const int total = nb * NT;
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int per_xcd_wgs = gridDim.x / kXcds;
    const int per_xcd_items = (total + kXcds - 1) / kXcds;
    const int it_begin = xcd * per_xcd_items;
    const int it_end = min(total, it_begin + per_xcd_items);

    // this thread's load slots: rows (tid >> 3) + 32 * i, 16-byte chunk tid & 7
    const int ld_ch = tid & 7;
    const int ld_row0 = tid >> 3;

    for (int it = it_begin + slot; it < it_end; it += per_xcd_wgs) {
        const int b = it / NT;
        const int nt = it - b * NT;
        const int l = blocks[4 * b + 1];
        const int blk_row0 = blocks[4 * b + 2];
        const int blk_rows = blocks[4 * b + 3];
        const uint16_t* Bexp = B + (int64_t)l * b_expert_stride;
      // blocks taller than one tile (block_m = 256) take several 128-row tiles
      for (int sub = 0; sub < blk_rows; sub += BM) {
        const int row0 = blk_row0 + sub;
        const int m = blk_rows - sub < BM ? blk_rows - sub : BM;

        const uint16_t* a_src[4];
        const uint16_t* b_src[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int rr = ld_row0 + 32 * i;
            int64_t ar = row0 + rr;
            if (ar > a_rows - 1) ar = a_rows - 1;
            a_src[i] = A + ar * Kdim + ld_ch * 8;
            int br;
            if (kSwiGLU)
                br = rr < 64 ? nt * 64 + rr : I + nt * 64 + (rr - 64);
            else
                br = nt * BN + rr;
            if (br > b_rows - 1) br = b_rows - 1;
            b_src[i] = Bexp + (int64_t)br * Kdim + ld_ch * 8;
        }

        f32x16_t acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

        uint4 ra[4], rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *reinterpret_cast<const uint4*>(a_src[i]);
            rb[i] = *reinterpret_cast<const uint4*>(b_src[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int rr = ld_row0 + 32 * i;
            *reinterpret_cast<uint4*>(&As[0][swz(rr, ld_ch)]) = ra[i];
            *reinterpret_cast<uint4*>(&Bs[0][swz(rr, ld_ch)]) = rb[i];
        }
        __syncthreads();

        const int nk = Kdim / BK;
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                const int k0 = (kt + 1) * BK;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
                    rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
                }
            }
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int ch = kk * 2 + (lane >> 5);
                bf16x8_t af[2], bfr[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    int row = wm * 64 + i * 32 + (lane & 31);
                    af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&As[cur][swz(row, ch)]));
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    int row = kSwiGLU ? (j == 0 ? wn * 32 : 64 + wn * 32) + (lane & 31)
                                      : wn * 64 + j * 32 + (lane & 31);
                    bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&Bs[cur][swz(row, ch)]));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j],
                                                                            acc[i][j], 0, 0, 0);
            }
            if (more) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int rr = ld_row0 + 32 * i;
                    *reinterpret_cast<uint4*>(&As[cur ^ 1][swz(rr, ld_ch)]) = ra[i];
                    *reinterpret_cast<uint4*>(&Bs[cur ^ 1][swz(rr, ld_ch)]) = rb[i];
                }
            }
            __syncthreads();
        }

        // epilogue: lane holds column (lane & 31), rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (rl >= m) continue;
                uint16_t* crow = C + (int64_t)(row0 + rl) * ldc;
                if (kSwiGLU) {
                    const float g = acc[i][0][r];
                    const float u = acc[i][1][r];
                    const float v = g / (1.f + expf(-g)) * u;
                    crow[nt * 64 + wn * 32 + (lane & 31)] = moe_f32_to_bf16(v);
                } else {
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        int col = nt * BN + wn * 64 + j * 32 + (lane & 31);
                        if (col < n_cols) crow[col] = moe_f32_to_bf16(acc[i][j][r]);
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
    ffn_bf16_kernel<true><<<persistent_grid(2), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(xp), max_rows, H, static_cast<const uint16_t*>(w1),
        (int64_t)2 * I * H, 2 * I, static_cast<uint16_t*>(act), I, I, I, I / 64, blocks,
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
    ffn_bf16_kernel<false><<<persistent_grid(2), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(act), max_rows, I, static_cast<const uint16_t*>(w2),
        (int64_t)H * I, H, static_cast<uint16_t*>(yp), H, H, I, (H + BN - 1) / BN, blocks,
        n_blocks, max_blocks);
    return hipGetLastError();
}
