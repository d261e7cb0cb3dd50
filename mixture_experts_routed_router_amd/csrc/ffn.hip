// ffn.hip -- SwiGLU expert FFN over the plan's block table (moe_expert_ffn).
//
// MegaFlux §2.1: FC1 (gate and up projections) then FC2; §4.1: SwiGLU experts, FP32
// accumulation, BF16 outputs; §3.1: the token dimension of the expert GEMM work is the plan's
// block of at most beta rows.  The fused gate+up idea (both projections from the same input
// tile, activation applied in registers) is the one the TritonMoE abstract (Daily Papers
// listing) describes.
//
// bf16 path: a schedule pass, then two grouped GEMMs on v_mfma_f32_32x32x16_bf16.
//   schedule: each expert's row-contiguous blocks are cut into 128-row pieces and paired into
//             256-row tiles of two halves with independent row bases; an expert with an odd
//             piece count ends with a half tile.  Tiles are listed expert by expert.
//   FC1:      per (tile, 128 act columns): A = the tile's xp rows, B = 128 gate rows of W1[l]
//             and the matching 128 up rows; act = SiLU(g) * u in registers, bf16 store.
//   FC2:      per (tile, 256 columns of H): A = act rows, B = 256 rows of W2[l].
// Why 256 x 256: a CU fills LDS from L2 at roughly 14-20 B/clk (bounded by outstanding L1
// misses times L2 latency), while its four SIMDs consume 4096 flop/clk; a tile must therefore
// do >= ~200 flop per staged byte to approach the MFMA roof.  256 x 256 gives 128 flop/B at
// one workgroup (256 accumulators per lane) per CU; 128 x 256 gave 85.
// Both operands are K-contiguous (C = A * B^T), so an MFMA fragment is one 16-byte LDS read.
// K is staged in 64-wide slices (128-byte rows: whole cache lines) through a 2-deep LDS ring
// filled by gfx950 direct-to-LDS loads, one slice in flight while the other is consumed, with
// one wait + barrier per slice placed behind that slice's last MFMAs.  The grid is
// persistent, one workgroup per CU: workgroup w runs on XCD w % 8 and takes (tile, column
// tile) items from its XCD's contiguous eighth of the item list through an atomic counter,
// so the items in flight on an XCD share A rows and B rows in its L2; a workgroup whose
// eighth is drained takes items from the other XCDs' eighths.
// Block and tile counts are read on the device; there is no host round trip.
#include "moe_launch.h"
#include "moe_lds.h"
#include "moe_ffn_ws.h"

namespace {

using namespace moe_ffn_ws;
static_assert(MOE_FFN_WS_ERR == WS_ERR && MOE_FFN_MAX_BLOCK_ROWS == kMaxBlockRows &&
                  MOE_FFN_ERR_EXPERT == FFN_ERR_EXPERT && MOE_FFN_ERR_ROWS == FFN_ERR_ROWS &&
                  MOE_FFN_ERR_RANGE == FFN_ERR_RANGE && MOE_FFN_ERR_COUNT == FFN_ERR_COUNT,
              "the error word's layout in moe.h");
constexpr int BN = 256;      // B rows per tile (FC1: 128 gate + 128 up; FC2: 256 columns of H)
constexpr int BK = 64;       // K slice per LDS stage: 128-byte rows = whole cache lines
constexpr int kWaves = 8;    // two waves per SIMD
constexpr int kThreads = kWaves * MOE_WAVE;
constexpr int ROW_BYTES = BK * 2;           // 128
constexpr int SEG_ROWS = 1024 / ROW_BYTES;  // 8 rows per 1 KB copy

// An item stages kRowsA rows of A per K slice: 256 (two 128-row halves, a 2-deep ring of
// 64 KB stages), 128 or 64 (one half of at most that many rows, a 3-deep ring of 48 or 40 KB
// stages).  The smaller items keep two slices in flight instead of one, where the kernel is
// mostly streaming weights, and stage only the A rows they use.
template <int kRowsA>
struct Mode {
    static constexpr int kStages = kRowsA == 256 ? 2 : 3;
    static constexpr int kARegion = kRowsA * ROW_BYTES;
    static constexpr int kStageBytes = kARegion + BN * ROW_BYTES;
    static constexpr int kACopies = kRowsA / 64;  // 1 KB A copies per wave per stage
    static constexpr int kBCopies = BN / 64;      // 1 KB B copies per wave per stage
    static constexpr int kCopies = kACopies + kBCopies;
    static constexpr int kRowBlocks = kRowsA / 64;  // 32-row MFMA blocks per wave
};
constexpr int SMEM_BYTES = Mode<128>::kStages * Mode<128>::kStageBytes;  // 144 KB
static_assert(Mode<256>::kStages * Mode<256>::kStageBytes <= SMEM_BYTES, "ring size");
static_assert(Mode<64>::kStages * Mode<64>::kStageBytes <= SMEM_BYTES, "ring size");

// Stage layout.  A stage holds the item's kRowsA A rows and 256 B rows, 128 bytes (64 bf16,
// one cache line) each, in 1 KB segments of 8 rows: A segment g = rows 8g..8g+7, B likewise.
// Wave w fills A segments w, w+8, ... and B segments w, w+8, w+16, w+24, each run placed
// contiguously (A at w * kACopies KB, B at kARegion + w * 4 KB), so the wave needs one M0
// value per run and selects segments with the copy instruction's immediate offset (which
// moves the LDS destination and the global source alike).  Within the tile, row r's logical
// 16-byte chunk c sits at physical chunk c ^ ((r >> 1) & 7): a ds_read_b128 serves 16 lanes
// at a time over 64 four-byte banks, and 16 consecutive rows reading one logical chunk then
// land in 16 distinct bank groups (r & 1 picks the 128-byte half, the XOR the group in it;
// segment bases are multiples of 256 bytes).
template <int kRowsA>
__device__ __forceinline__ uint32_t stage_row_offset(int row, bool b_side) {
    using M = Mode<kRowsA>;
    const int g = row >> 3;  // segment of the row on its side
    const uint32_t in_seg = (uint32_t)(row & 7) * ROW_BYTES;
    if (b_side) return (uint32_t)(M::kARegion + (g & 7) * (M::kBCopies * 1024) + (g >> 3) * 1024) + in_seg;
    return (uint32_t)((g & 7) * (M::kACopies * 1024) + (g >> 3) * 1024) + in_seg;
}

template <int kRowsA>
__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* stage, int row, bool b_side, int ch) {
    const uint4 v = *reinterpret_cast<const uint4*>(stage + stage_row_offset<kRowsA>(row, b_side) +
                                                    (swz_chunk(row, ch) << 4));
    return __builtin_bit_cast(bf16x8_t, v);
}

// ------------------------------------------------------------------ tile schedule ---

// One workgroup.  The blocks of each expert are taken in table order (a stable counting sort
// by expert); consecutive blocks whose rows are contiguous form one run (the plan's shares of
// an expert are consecutive ranges of its segment, so a whole table gives one run per
// expert).  Each run is cut into 128-row pieces from its start, and an expert's pieces are
// paired in order into 256-row tiles (an odd last piece is a half tile).  Experts follow one
// another in ascending local id.  The GEMMs' item and finished counters are cleared too.
// Tables of up to kSchedLds blocks are staged in LDS first, so the per-expert walks (one
// thread per expert) touch LDS only; larger tables are walked in global memory.
constexpr int kSchedLds = 3072;

// FFN_ERR_* bits of table entry (expert l, first row, rows) for E_loc experts and max_rows
// rows.  The schedule takes a block only when this is 0 and rows > 0, which keeps every tile
// inside [0, max_rows) and every expert index inside the weights, whatever the table holds;
// blocks of at most kMaxBlockRows rows also keep the tiles within their 2 * max_blocks
// records (an expert's 128-row pieces number at most twice its blocks).
__device__ __forceinline__ int block_error(int l, int first, int rows, int E_loc, int64_t max_rows) {
    int e = 0;
    if (l < 0 || l >= E_loc) e |= FFN_ERR_EXPERT;
    if (rows < 0 || rows > kMaxBlockRows) e |= FFN_ERR_ROWS;
    if (first < 0 || (int64_t)first + (rows > 0 ? rows : 0) > max_rows) e |= FFN_ERR_RANGE;
    return e;
}

// Exclusive prefix sum of v over the 256 threads of the workgroup (thread order); *total gets
// the sum.  part holds one int per wave.
__device__ __forceinline__ int block_exclusive_scan(int v, int* part, int* total) {
    const int lane = moe_lane_id(), wave = threadIdx.x / MOE_WAVE;
    int incl = v;
#pragma unroll
    for (int d = 1; d < MOE_WAVE; d <<= 1) {
        const int o = __shfl_up(incl, d, MOE_WAVE);
        if (lane >= d) incl += o;
    }
    if (lane == MOE_WAVE - 1) part[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int pw = part[w];
        before += w < wave ? pw : 0;
        all += pw;
    }
    *total = all;
    __syncthreads();  // part may be reused
    return before + incl - v;
}

struct SchedShared {
    int sum_rows[256];
    int min_first[256];
    int max_end[256];
    int cnt[256];
    int bstart[257];
    int npieces[256];
    int tstart[257];
    int running[256];
    unsigned long long mask[4][256];
    int s_l[kSchedLds], s_first[kSchedLds], s_rows[kSchedLds], s_sorted[kSchedLds];
    int scan_part[4];
    int err;
};

// kLds: the table (nb <= kSchedLds blocks) has been staged in sh.s_*; otherwise it is read
// from global memory.  Two instantiations, so that neither path carries the other's loads.
template <bool kLds>
__device__ __forceinline__ void schedule_body(const int32_t* __restrict__ blocks, int nb,
                                              int max_blocks, int E_loc, int64_t max_rows,
                                              int32_t* __restrict__ ws, SchedShared& sh) {
    const int tid = threadIdx.x, lane = moe_lane_id(), wave = tid / MOE_WAVE;
    int32_t* sorted_g = ws + WS_HEAD;
    int32_t* tiles = ws + WS_HEAD + max_blocks;
    // the block's expert, or -1 for a block the schedule skips
    auto blk_l = [&](int b) {
        if constexpr (kLds) {
            return sh.s_l[b];
        } else {
            const int4 v = reinterpret_cast<const int4*>(blocks)[b];
            return block_error(v.y, v.z, v.w, E_loc, max_rows) == 0 && v.w > 0 ? v.y : -1;
        }
    };
    auto blk_first = [&](int b) {
        if constexpr (kLds) return sh.s_first[b]; else return blocks[4 * b + 2];
    };
    auto blk_rows = [&](int b) {
        if constexpr (kLds) return sh.s_rows[b]; else return blocks[4 * b + 3];
    };
    auto sorted_at = [&](int i) {
        if constexpr (kLds) return sh.s_sorted[i]; else return sorted_g[i];
    };

    for (int b = tid; b < nb; b += 256) {
        const int l = blk_l(b);
        if (l >= 0) atomicAdd(&sh.cnt[l], 1);
    }
    __syncthreads();
    {
        int total;
        const int ex = block_exclusive_scan(tid < E_loc ? sh.cnt[tid] : 0, sh.scan_part, &total);
        if (tid < E_loc) sh.bstart[tid] = ex;
        if (tid == 0) sh.bstart[E_loc] = total;
    }
    __syncthreads();
    // stable counting sort of the blocks by expert, 256 blocks per round
    for (int b0 = 0; b0 < nb; b0 += 256) {
        for (int i = tid; i < 4 * 256; i += 256) sh.mask[i / 256][i % 256] = 0ull;
        __syncthreads();
        const int b = b0 + tid;
        const int l = b < nb ? blk_l(b) : -1;
        if (l >= 0) atomicOr(&sh.mask[wave][l], 1ull << lane);
        __syncthreads();
        if (l >= 0) {
            int pos = sh.running[l] + __popcll(sh.mask[wave][l] & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w) pos += __popcll(sh.mask[w][l]);
            if constexpr (kLds)
                sh.s_sorted[sh.bstart[l] + pos] = b;
            else
                sorted_g[sh.bstart[l] + pos] = b;
        }
        __syncthreads();
        for (int e = tid; e < E_loc; e += 256)
            sh.running[e] += __popcll(sh.mask[0][e]) + __popcll(sh.mask[1][e]) +
                             __popcll(sh.mask[2][e]) + __popcll(sh.mask[3][e]);
        __syncthreads();
    }
    if constexpr (!kLds) __threadfence_block();  // sorted_g written above, read below
    // pieces per expert: walk its blocks, joining row-contiguous ones into runs
    for (int l = tid; l < E_loc; l += 256) {
        int pieces = 0, run_first = 0, run_rows = 0;
        for (int i = sh.bstart[l]; i < sh.bstart[l + 1]; ++i) {
            const int b = sorted_at(i);
            const int first = blk_first(b), rows = blk_rows(b);
            if (run_rows > 0 && first == run_first + run_rows) {
                run_rows += rows;
            } else {
                pieces += (run_rows + HALF - 1) / HALF;
                run_first = first;
                run_rows = rows;
            }
        }
        pieces += (run_rows + HALF - 1) / HALF;
        sh.npieces[l] = pieces;
    }
    __syncthreads();
    {
        int total;
        const int ex = block_exclusive_scan(tid < E_loc ? (sh.npieces[tid] + 1) / 2 : 0,
                                            sh.scan_part, &total);
        if (tid < E_loc) sh.tstart[tid] = ex;
        if (tid == 0) {
            sh.tstart[E_loc] = total;
            ws[WS_NTILES] = total;
        }
    }
    __syncthreads();
    // emit the tiles: pieces of an expert in order, two per tile
    for (int l = tid; l < E_loc; l += 256) {
        const int t0 = sh.tstart[l], tcount = sh.tstart[l + 1] - t0;
        int piece = 0, run_first = 0, run_rows = 0;
        auto emit_run = [&]() {
            for (int off = 0; off < run_rows; off += HALF, ++piece) {
                int32_t* t = tiles + TILE_INTS * (t0 + piece / 2);
                const int rows = run_rows - off < HALF ? run_rows - off : HALF;
                if ((piece & 1) == 0) {
                    t[0] = l;
                    t[1] = run_first + off;
                    t[2] = rows;
                    t[3] = 0;
                    t[4] = 0;
                    t[5] = t0;
                    t[6] = tcount;
                } else {
                    t[3] = run_first + off;
                    t[4] = rows;
                }
            }
        };
        for (int i = sh.bstart[l]; i < sh.bstart[l + 1]; ++i) {
            const int b = sorted_at(i);
            const int first = blk_first(b), rows = blk_rows(b);
            if (run_rows > 0 && first == run_first + run_rows) {
                run_rows += rows;
            } else {
                emit_run();
                run_first = first;
                run_rows = rows;
            }
        }
        emit_run();
    }
}

// Common case: every expert's blocks cover one contiguous row range (a moe_plan table: an
// expert's shares are consecutive ranges of its segment).  Then its pieces are 128-row cuts
// of that range and each tile follows from the expert's first row and row count alone.
// Every block is checked here first (block_error); the error word of the call is written.
__device__ __forceinline__ bool schedule_contiguous(const int32_t* __restrict__ blocks, int nb,
                                                    int max_blocks, int E_loc, int64_t max_rows,
                                                    int32_t* __restrict__ ws, SchedShared& sh) {
    const int tid = threadIdx.x;
    for (int b = tid; b < nb; b += 256) {
        const int4 v = reinterpret_cast<const int4*>(blocks)[b];
        const int e = block_error(v.y, v.z, v.w, E_loc, max_rows);
        if (e != 0) {
            atomicOr(&sh.err, e);
            continue;
        }
        if (v.w == 0) continue;
        atomicAdd(&sh.sum_rows[v.y], v.w);
        atomicMin(&sh.min_first[v.y], v.z);
        atomicMax(&sh.max_end[v.y], v.z + v.w);
    }
    __syncthreads();
    if (tid == 0) ws[WS_ERR] = sh.err;
    // blocks never overlap, so the union is one range exactly when its span equals the sum
    const bool ok = tid >= E_loc || sh.sum_rows[tid] == 0 ||
                    sh.sum_rows[tid] == sh.max_end[tid] - sh.min_first[tid];
    if (!__syncthreads_and(ok)) return false;
    int total;
    const int pieces = tid < E_loc ? (sh.sum_rows[tid] + HALF - 1) / HALF : 0;
    const int ex = block_exclusive_scan((pieces + 1) / 2, sh.scan_part, &total);
    if (tid < E_loc) sh.tstart[tid] = ex;
    if (tid == 0) {
        sh.tstart[E_loc] = total;
        ws[WS_NTILES] = total;
    }
    __syncthreads();
    int32_t* tiles = ws + WS_HEAD + max_blocks;
    for (int t = tid; t < total; t += 256) {
        int lo = 0, hi = E_loc - 1;  // the expert l with tstart[l] <= t < tstart[l + 1]
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.tstart[mid] <= t) lo = mid; else hi = mid - 1;
        }
        const int l = lo, j = t - sh.tstart[l];
        const int n = sh.sum_rows[l], first = sh.min_first[l] + j * 2 * HALF;
        const int left = n - j * 2 * HALF;  // rows of the expert from this tile on
        int32_t* o = tiles + TILE_INTS * t;
        o[0] = l;
        o[1] = first;
        o[2] = left < HALF ? left : HALF;
        o[3] = left > HALF ? first + HALF : 0;
        o[4] = left > HALF ? (left - HALF < HALF ? left - HALF : HALF) : 0;
        o[5] = sh.tstart[l];
        o[6] = sh.tstart[l + 1] - sh.tstart[l];
    }
    return true;
}

__global__ void __launch_bounds__(256)
ffn_schedule_kernel(const int32_t* __restrict__ blocks, const int32_t* __restrict__ n_blocks_ptr,
                    int max_blocks, int E_loc, int64_t max_rows, int32_t* __restrict__ ws) {
    __shared__ SchedShared sh;
    const int tid = threadIdx.x;
    const int nb_in = *n_blocks_ptr;
    const int nb = nb_in < 0 ? 0 : (nb_in < max_blocks ? nb_in : max_blocks);
    if (tid >= WS_CTR_FC1 && tid < WS_HEAD) ws[tid] = 0;  // item and finished counters
    if (tid == 0) sh.err = nb_in < 0 || nb_in > max_blocks ? FFN_ERR_COUNT : 0;
    for (int l = tid; l < E_loc; l += 256) {
        sh.cnt[l] = 0;
        sh.running[l] = 0;
        sh.sum_rows[l] = 0;
        sh.min_first[l] = 0x7FFFFFFF;
        sh.max_end[l] = 0;
    }
    __syncthreads();
    if (schedule_contiguous(blocks, nb, max_blocks, E_loc, max_rows, ws, sh)) return;
    if (nb <= kSchedLds) {
        for (int b = tid; b < nb; b += 256) {
            const int4 v = reinterpret_cast<const int4*>(blocks)[b];
            const bool ok = block_error(v.y, v.z, v.w, E_loc, max_rows) == 0 && v.w > 0;
            sh.s_l[b] = ok ? v.y : -1;  // skipped
            sh.s_first[b] = v.z;
            sh.s_rows[b] = v.w;
        }
        __syncthreads();
        schedule_body<true>(blocks, nb, max_blocks, E_loc, max_rows, ws, sh);
    } else {
        __syncthreads();
        schedule_body<false>(blocks, nb, max_blocks, E_loc, max_rows, ws, sh);
    }
}

// ------------------------------------------------------------------ grouped GEMMs ---

// One item: C rows of tile (h_row0, h_rows) x column tile nt of expert B (see ffn_bf16_kernel).
// Wave (wm, wn) = (wave >> 2, wave & 3) computes kRowBlocks 32-row blocks starting at tile row
// wm * kRowsA / 2, against 64 B rows (FC1: 32 gate rows and the 32 matching up rows).
// Kernel-wide arguments of one grouped GEMM launch.
struct GemmArgs {
    const uint16_t* A;       // [a_rows, Kdim], or the token rows of x with `gather`
    int64_t a_rows;
    int Kdim;
    const uint16_t* B;       // [E_loc][b_rows, Kdim]
    int64_t b_expert_stride;
    int b_rows;
    uint16_t* C;             // [rows, ldc]
    int ldc, n_cols, I, NT;
    // the schedule's tile records, read with scalar loads: the schedule kernel wrote them
    // before this launch, and a scalar load is tracked by lgkmcnt, so waiting for it never
    // waits for the slice copies in flight (a vector load's wait would: the copies are
    // invisible to the compiler's vmcnt bookkeeping, which then waits for vmcnt(0))
    const __attribute__((address_space(4))) int32_t* tiles;
    int32_t* gidx;           // LDS: the gathered token rows of the item being decoded
    uint32_t gidx_lds;       // its LDS byte address
    int32_t* ctr;            // this GEMM's per-XCD item counters
    int total, per_xcd_items, xcd;
    const int32_t* gather;   // row_token (gather-on-load) or nullptr
    // FC2 with direct rows: dir[p] = the token whose only local entry is row p (else -1) and
    // dir[a_rows + p] its routing weight's bits; such a row goes to out[token], weighted
    const int32_t* dir;
    uint16_t* out;
    int T;
};

// One item (tile, column tile): its wave-uniform description and this lane's A copy offsets
// (byte offsets from the item's A base pointers: row * Kdim * 2 + chunk * 16, < 4 GiB; the B
// offsets follow from nt and are formed per copy).
struct Item {
    int rows_a;  // A rows staged per slice: 256, 128 or 64; 0 = no item (the queues are drained)
    int l, nt;
    int h_row0[2], h_rows[2];
    int it, ts, cnt;
    uint32_t offa[4];  // with gather (decode step 4 leaves the token rows here, step 5 the offsets)
};

// Thread 0's queue state: the queue being tried (own XCD first, then the others in turn).
struct Queue {
    int q;
};

// Two floats -> packed bf16x2 (low half = a), nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// v, in a form the compiler cannot see through: what is derived from it is computed where it
// is used, instead of being hoisted to the kernel's start and kept live (or spilled) across the
// item loop.  A spilled value's reload is a vector-memory read, and the compiler's wait for it
// would also wait for the slice copies in flight.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ int rows_mode(int h_rows1, int h_rows0) {
    return h_rows1 > 0 ? 256 : (h_rows0 > 64 ? 128 : 64);
}

// The item's wave-uniform fields as scalars.  They are uniform by construction (decoded from
// one LDS word), but the decode's joins with thread 0's queue branch hide that from the
// compiler, which would otherwise keep them (and the copy base pointers) in vector registers.
__device__ __forceinline__ Item uniform_item(const Item& it) {
    Item u = it;
    u.rows_a = __builtin_amdgcn_readfirstlane(it.rows_a);
    u.l = __builtin_amdgcn_readfirstlane(it.l);
    u.nt = __builtin_amdgcn_readfirstlane(it.nt);
    u.h_row0[0] = __builtin_amdgcn_readfirstlane(it.h_row0[0]);
    u.h_row0[1] = __builtin_amdgcn_readfirstlane(it.h_row0[1]);
    u.h_rows[0] = __builtin_amdgcn_readfirstlane(it.h_rows[0]);
    u.h_rows[1] = __builtin_amdgcn_readfirstlane(it.h_rows[1]);
    return u;
}

__device__ __forceinline__ const uint8_t* base_a(const GemmArgs& g, const Item& it, int h) {
    const int row0 = h ? it.h_row0[1] : it.h_row0[0];
    return reinterpret_cast<const uint8_t*>(g.gather ? g.A : g.A + (int64_t)row0 * g.Kdim);  // gather: rows of x
}

__device__ __forceinline__ const uint8_t* base_b(const GemmArgs& g, const Item& it) {
    return reinterpret_cast<const uint8_t*>(g.B + (int64_t)it.l * g.b_expert_stride);
}

// Decoding the next item takes six steps, each using what the step before loaded, so that
// the loads' latency hides behind the current item's last K slices (one step per slice
// boundary).  A copy q of wave w fills tile rows 64q + 8w + (0..7) (half q / 2).
//   0: thread 0 increments its queue's counter          3: load the tile record
//   1: thread 0 resolves the item (trying the other     4: with gather, load the token row
//      queues when its own is drained), publishes it       of each of this lane's A copies
//      in LDS                                            5: this lane's copy offsets
//   2: read the item; load its tile group's first tile and tile count
// Steps 1 and 2 must be separated by a barrier (the slice boundaries are).
template <bool kSwiGLU, bool kGather>
__device__ __forceinline__ void decode_step(int s, Item& n, const GemmArgs& g, Queue& qs,
                                            int* item_s, int tid, int wave, int seg_row,
                                            int seg_lchunk) {
    switch (s) {
        // The counter increment is the kernel's only vector-memory read the compiler sees (the
        // slice copies are inline asm, invisible to its bookkeeping, so its wait for the
        // increment is vmcnt(0)).  Its result goes to LDS at once, in wave 0: no register holds
        // it across slice boundaries, where a pending read would make the compiler drain all
        // copies in flight before later uses or writes of that register (e.g. every MFMA).
        case 0:
            if (wave == 0) {
                if (tid == 0 && qs.q < kXcds) item_s[1] = atomicAdd(&g.ctr[(g.xcd + qs.q) % kXcds], 1);
            }
            break;
        case 1:
            if (tid == 0) {
                int raw = item_s[1];
                int got = -1;
                while (qs.q < kXcds) {
                    const int x = (g.xcd + qs.q) % kXcds;
                    const int it = x * g.per_xcd_items + raw;
                    if (raw < g.per_xcd_items && it < g.total) {
                        got = it;
                        break;
                    }
                    if (++qs.q < kXcds) raw = atomicAdd(&g.ctr[(g.xcd + qs.q) % kXcds], 1);
                }
                asm volatile("" ::"v"(raw));  // the last increment is taken on every path
                item_s[0] = got;
            }
            break;
        case 2: {
            n.it = __builtin_amdgcn_readfirstlane(item_s[0]);
            n.rows_a = 0;
            if (n.it >= 0) {
                // wave-uniform operands (readfirstlane) keep the address in scalar registers,
                // so the record is read with scalar loads
                const int it = __builtin_amdgcn_readfirstlane(n.it);
                const auto tg = g.tiles + TILE_INTS * (it / g.NT);
                n.ts = __builtin_amdgcn_readfirstlane(tg[5]);
                n.cnt = __builtin_amdgcn_readfirstlane(tg[6]);
            }
            break;
        }
        case 3:
            if (n.it >= 0) {
                // item -> (tile, column tile): the expert's items [ts * NT, (ts + cnt) * NT) in
                // groups of kGroupTiles tiles, column-tile-major inside a group
                const int it = __builtin_amdgcn_readfirstlane(n.it);
                const int ts = __builtin_amdgcn_readfirstlane(n.ts);
                const int cnt = __builtin_amdgcn_readfirstlane(n.cnt);
                const int local = it - ts * g.NT;
                const int grp = local / (kGroupTiles * g.NT);
                const int r = local - grp * (kGroupTiles * g.NT);
                const int rest = cnt - grp * kGroupTiles;
                const int ct = rest < kGroupTiles ? rest : kGroupTiles;
                n.nt = r / ct;
                const int t = ts + grp * kGroupTiles + (r - n.nt * ct);
                const auto tl = g.tiles + TILE_INTS * t;
                n.l = __builtin_amdgcn_readfirstlane(tl[0]);
                n.h_row0[0] = __builtin_amdgcn_readfirstlane(tl[1]);
                n.h_rows[0] = __builtin_amdgcn_readfirstlane(tl[2]);
                n.h_row0[1] = __builtin_amdgcn_readfirstlane(tl[3]);
                n.h_rows[1] = __builtin_amdgcn_readfirstlane(tl[4]);
            }
            break;
        case 4:
            if (n.it >= 0) {
                n.rows_a = rows_mode(n.h_rows[1], n.h_rows[0]);
                if (kGather) {
                    // the token row of each of this lane's A copies, copied straight into LDS
                    // (lane l's word lands at gidx[(wave * 4 + q) * 64 + l]); the slice wait at
                    // the next boundary covers the copy, as it was issued before that
                    // boundary's newest slice copies
                    const int copies = n.rows_a / 64;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (q < copies) {
                            const int h = q >> 1;
                            int rr = ((q & 1) * 8 + wave) * SEG_ROWS + seg_row;
                            const int hr = h ? n.h_rows[1] : n.h_rows[0];
                            if (rr > hr - 1) rr = hr - 1;  // read, unused
                            const int row = (h ? n.h_row0[1] : n.h_row0[0]) + rr;
                            one_copy_dword(g.gidx_lds + (uint32_t)(wave * 4 + q) * (MOE_WAVE * 4), g.gather,
                                           (uint32_t)row * 4u);
                        }
                    }
                }
            }
            break;
        case 5:
            if (kGather && n.it >= 0) {
                const int copies = n.rows_a / 64;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // row_token -1 (padding) or out of range: read row 0, never stored
                    const int t = q < copies ? g.gidx[(wave * 4 + q) * MOE_WAVE + moe_lane_id()] : 0;
                    const int tok = q < copies && t >= 0 && t < g.a_rows ? t : 0;
                    n.offa[q] = (uint32_t)tok * (uint32_t)g.Kdim * 2u + seg_lchunk * 16u;
                }
            }
            break;
        default:
            break;
    }
}

// Copies of K slice kt of item `it` into ring slot kt % kStages (this wave's share).
// This lane's byte offset for B copy q of an item: B tile row (q * 8 + w) * 8 + seg_row is
// W1 row nt * 128 + r (gate, r < 128) or I + nt * 128 + r - 128 (up) for FC1, W2 row
// nt * 256 + r for FC2; rows past the end are clamped (read, not stored).
template <bool kSwiGLU>
__device__ __forceinline__ uint32_t b_offset(const GemmArgs& g, int nt, int q, int wave,
                                             int seg_row, uint32_t lane_chunk) {
    const int r0 = (q * 8 + wave) * SEG_ROWS;
    const int base = kSwiGLU ? (q < 2 ? nt * (BN / 2) + r0 : g.I + nt * (BN / 2) + r0 - BN / 2)
                             : nt * BN + r0;
    int br = base + seg_row;
    if (br > g.b_rows - 1) br = g.b_rows - 1;
    return (uint32_t)br * (uint32_t)g.Kdim * 2u + lane_chunk;
}

// This lane's byte offset for A copy q of an item without gather: row ((q & 1) * 8 + w) * 8 +
// seg_row of half q / 2, clamped to the last row of A (read, unused), from that half's base.
__device__ __forceinline__ uint32_t a_offset(const GemmArgs& g, const Item& it, int q, int wave,
                                             int seg_row, uint32_t lane_chunk) {
    const int h = q >> 1;
    const int row0 = h ? it.h_row0[1] : it.h_row0[0];
    int rr = ((q & 1) * 8 + wave) * SEG_ROWS + seg_row;
    if (row0 + rr > g.a_rows - 1) rr = (int)(g.a_rows - 1 - row0);
    return (uint32_t)rr * (uint32_t)g.Kdim * 2u + lane_chunk;
}

// 64-row items (at most 64 valid rows, decode-sized experts): wave w stages A rows
// 8w .. 8w + 7 only when some of them are valid.  Rows past the valid ones feed only MFMA
// rows that are never stored, so their LDS rows may hold anything; a tile of a few rows then
// stages 1 KB of A per slice instead of 8 KB, which a weight-streaming CU spends on weights.
template <int kRowsA>
__device__ __forceinline__ bool a_copy_needed(const Item& it, int wave) {
    return kRowsA != 64 || wave * SEG_ROWS < it.h_rows[0];
}

// issue_slice parts: the A rows' copies, and the B rows' first two and last two copies.
constexpr int kPartA = 1, kPartB01 = 2, kPartB23 = 4, kPartB = kPartB01 | kPartB23;
// Where the copies of the slice that a slice boundary makes room for go out: at the boundary
// itself (-1), with the wait, or before the MFMAs of K step k (0..3) of the next slice.  Issued
// all at the boundary, the 64 copies of the workgroup queue in the address unit (one 1 KB copy
// every ~18 cycles) while every wave waits there for its turn, before its first MFMA of the
// slice; spread into the K steps, a wave that waits on a copy leaves the MFMA pipe to the other
// wave of its SIMD.  Measured per GEMM (lab copies in one process, all bit-identical):
// FC1 B copies before step 1 (−1 to −3.5%), FC2 A copies before step 0 and B before step 1
// (−3 to −7%), against all at the boundary.
#ifndef FFN_DEFER_FC1
#define FFN_DEFER_FC1 -1, 1, 1
#endif
#ifndef FFN_DEFER_FC2
#define FFN_DEFER_FC2 0, 1, 1
#endif
struct Defer {
    int a, b01, b23;  // the K step of the A copies, B copies 0-1, B copies 2-3
};
template <bool kSwiGLU>
__device__ constexpr Defer defer_of() {
    return kSwiGLU ? Defer{FFN_DEFER_FC1} : Defer{FFN_DEFER_FC2};
}

template <bool kSwiGLU, bool kGather, int kRowsA>
__device__ __forceinline__ void issue_slice(const GemmArgs& g, const Item& it, int kt,
                                            uint32_t smem_base, int wave, int seg_row,
                                            uint32_t lane_chunk, int parts = kPartA | kPartB) {
    using M = Mode<kRowsA>;
    kt = __builtin_amdgcn_readfirstlane(kt);  // wave-uniform: M0 and the copy bases are scalars
    const uint32_t st = smem_base + (kt % M::kStages) * M::kStageBytes;
    const uint32_t koff = (uint32_t)kt * (BK * 2);
    const uint32_t ma = st + wave * (M::kACopies * 1024);
    const uint8_t* a0 = base_a(g, it, 0);
    const uint8_t* bx = base_b(g, it);
    if (parts & kPartA) {
        uint32_t oa[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            oa[q] = (kGather ? it.offa[q] : a_offset(g, it, q, wave, seg_row, lane_chunk)) + koff;
        if constexpr (kRowsA == 256) {
            const uint8_t* a1 = base_a(g, it, 1);
            four_copies(ma, a0, a0 - 1024, a1 - 2048, a1 - 3072, oa[0], oa[1], oa[2], oa[3], true);
        } else if constexpr (kRowsA == 128) {
            four_copies(ma, a0, a0 - 1024, a0, a0, oa[0], oa[1], 0, 0, false);
        } else if (a_copy_needed<kRowsA>(it, wave)) {
            one_copy(ma, a0, oa[0]);
        }
    }
    if ((parts & kPartB) == kPartB)
        four_copies(st + M::kARegion + wave * 4096, bx, bx - 1024, bx - 2048, bx - 3072,
                    b_offset<kSwiGLU>(g, it.nt, 0, wave, seg_row, lane_chunk) + koff,
                    b_offset<kSwiGLU>(g, it.nt, 1, wave, seg_row, lane_chunk) + koff,
                    b_offset<kSwiGLU>(g, it.nt, 2, wave, seg_row, lane_chunk) + koff,
                    b_offset<kSwiGLU>(g, it.nt, 3, wave, seg_row, lane_chunk) + koff, true);
    else if (parts & kPartB01)
        four_copies(st + M::kARegion + wave * 4096, bx, bx - 1024, bx, bx,
                    b_offset<kSwiGLU>(g, it.nt, 0, wave, seg_row, lane_chunk) + koff,
                    b_offset<kSwiGLU>(g, it.nt, 1, wave, seg_row, lane_chunk) + koff, 0, 0, false);
    else if (parts & kPartB23)
        four_copies(st + M::kARegion + wave * 4096 + 2048, bx, bx - 1024, bx, bx,
                    b_offset<kSwiGLU>(g, it.nt, 2, wave, seg_row, lane_chunk) + koff,
                    b_offset<kSwiGLU>(g, it.nt, 3, wave, seg_row, lane_chunk) + koff, 0, 0, false);
}

template <bool kSwiGLU, bool kGather, int kRowsA>
__device__ __forceinline__ void issue_prologue_m(const GemmArgs& g, const Item& it,
                                                 uint32_t smem_base, int wave, int seg_row,
                                                 uint32_t lane_chunk) {
    constexpr int kStages = Mode<kRowsA>::kStages;
    const int nk = g.Kdim / BK;
    const int pre = nk < kStages ? nk : kStages;
    for (int s = 0; s < pre; ++s)
        issue_slice<kSwiGLU, kGather, kRowsA>(g, it, s, smem_base, wave, seg_row, lane_chunk);
}

// Wait until this wave's copies of all but the last `pending` issued slices have landed, then
// meet the workgroup.  64-row items: a wave issues kCopies copies per slice, or one fewer
// when it stages no A rows (a_copy_needed).
template <int kRowsA>
__device__ __forceinline__ void wait_slices(int pending, bool a_copy) {
    using M = Mode<kRowsA>;
    if constexpr (kRowsA == 64) {
        if (a_copy)
            wait_pending_stages<M::kCopies, M::kStages - 1>(pending);
        else
            wait_pending_stages<M::kCopies - 1, M::kStages - 1>(pending);
    } else {
        wait_copies_and_barrier(pending * M::kCopies);
    }
}

// The first kStages slices of an item (the ring must be free).
template <bool kSwiGLU, bool kGather>
__device__ __forceinline__ void issue_prologue(const GemmArgs& g, const Item& item,
                                               uint32_t smem_base, int wave, int seg_row,
                                               uint32_t lane_chunk) {
    const Item it = uniform_item(item);
    if (it.rows_a == 256)
        issue_prologue_m<kSwiGLU, kGather, 256>(g, it, smem_base, wave, seg_row, lane_chunk);
    else if (it.rows_a == 128)
        issue_prologue_m<kSwiGLU, kGather, 128>(g, it, smem_base, wave, seg_row, lane_chunk);
    else if (it.rows_a == 64)
        issue_prologue_m<kSwiGLU, kGather, 64>(g, it, smem_base, wave, seg_row, lane_chunk);
}

// FC2 with direct rows: an item's 256 dir entries and their 256 weights, copied straight into
// buffer `buf` (512 words) of the gidx area of LDS (unused by FC2): lane l of wave w moves word
// e = 64 w + l, i.e. entry (e & 255) of side e >> 8, for tile row e & 255 (clamped to the
// item's first row where the row is past its half, read and unused).  Issued with the item's
// first slices, one item ahead, into the buffer the item before last used (every wave has
// passed a barrier since that item's epilogue read it); the waits that follow only become
// stricter, and the item's last wait covers it before its epilogue reads it.
__device__ __forceinline__ void issue_dir_copy(const GemmArgs& g, const Item& it, int wave,
                                               int buf) {
    const int e = wave * MOE_WAVE + moe_lane_id();
    const int side = e >> 8, r = e & 255, h = r >> 7, rl = r & (HALF - 1);
    const int hr = h ? it.h_rows[1] : it.h_rows[0];
    const int row = rl < hr ? (h ? it.h_row0[1] : it.h_row0[0]) + rl : it.h_row0[0];
    buf = __builtin_amdgcn_readfirstlane(buf);  // wave-uniform: the M0 base is a scalar
    one_copy_dword(g.gidx_lds + (uint32_t)(buf * 512 + wave * MOE_WAVE) * 4u, g.dir,
                   ((uint32_t)side * (uint32_t)g.a_rows + (uint32_t)row) * 4u);
}

// bf16 pair u reweighted as a one-entry combine does it: bf16(fmaf(w, y, 0)) per half, rounded
// to nearest even by the hardware conversion (the combine's software rounding gives the same
// bits for every finite value; one instruction per pair instead of about a dozen).
__device__ __forceinline__ uint32_t weight_bf16x2(uint32_t u, float w) {
    return pack_bf16x2(fmaf(w, __uint_as_float(u << 16), 0.f),
                       fmaf(w, __uint_as_float(u & 0xFFFF0000u), 0.f));
}

// One item whose first slices are already issued: the K loop; meanwhile the next item is
// decoded (decode_step, over the last slice boundaries); then the next item's first slices
// are issued, and this item's results are written from registers while they land.
template <bool kSwiGLU, bool kGather, int kRowsA, bool kDirect = false>
__device__ __forceinline__ void gemm_item(const GemmArgs& g, const Item& cur_in, Item& nxt,
                                          Queue& qs, int* item_s, uint8_t* smem,
                                          uint32_t smem_base, int tid, int wave, int lane,
                                          int seg_row, int seg_lchunk, int dbuf) {
    using M = Mode<kRowsA>;
    const Item cur = uniform_item(cur_in);
    constexpr int RB = M::kRowBlocks;
    constexpr int kDecodeSteps = 6;
    const int wm = wave >> 2;
    const int wn = wave & 3;
    const int wrow = wm * (kRowsA / 2);  // first tile row of this wave
    const bool active = kRowsA != 64 || wrow < cur.h_rows[0];  // 64-row items: idle past the rows
    const int nk = g.Kdim / BK;
    const int pre = nk < M::kStages ? nk : M::kStages;
    // the decode steps run at the boundaries after slices first_step .. first_step + 5
    const int first_step = nk - 1 - kDecodeSteps > 0 ? nk - 1 - kDecodeSteps : 0;

    f32x16_t acc[RB][2];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragments double-buffered one 16-wide K step ahead of the MFMAs
    bf16x8_t fa[2][RB], fb[2][2];
    auto load_frags = [&](int kt, int kk, int buf) {
        const uint8_t* st = smem + (kt % M::kStages) * M::kStageBytes;
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int br = kSwiGLU ? j * (BN / 2) + wn * 32 + (lane & 31)
                                   : wn * 64 + j * 32 + (lane & 31);
            fb[buf][j] = lds_frag<kRowsA>(st, br, true, ch);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
            fa[buf][i] = lds_frag<kRowsA>(st, wrow + i * 32 + (lane & 31), false, ch);
    };

    // slice 0 in LDS everywhere (stores of the previous item may still be counted: stricter)
    const bool a_copy = a_copy_needed<kRowsA>(cur, wave);
    wait_slices<kRowsA>(pre - 1, a_copy);
    if (active) load_frags(0, 0, 0);

    int step = 0;
    constexpr Defer kDefer = defer_of<kSwiGLU>();
    static_assert(kDefer.a < BK / 16 && kDefer.b01 < BK / 16 && kDefer.b23 < BK / 16,
                  "copies go out within the next slice");
    // the parts of a slice's copies that go out at step k of the next slice (k = -1: at the boundary)
    auto parts_at = [&](int k) {
        return (kDefer.a == k ? kPartA : 0) | (kDefer.b01 == k ? kPartB01 : 0) |
               (kDefer.b23 == k ? kPartB23 : 0);
    };
    int deferred = -1;  // the slice whose deferred copies go out in this slice's K steps
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur_buf = kk & 1;
            if (parts_at(kk) != 0 && deferred >= 0)
                issue_slice<kSwiGLU, kGather, kRowsA>(g, cur, deferred, smem_base, wave, seg_row,
                                                      seg_lchunk * 16u, parts_at(kk));
            if (active) {
                if (kk + 1 < BK / 16) load_frags(kt, kk + 1, cur_buf ^ 1);
                // FC1: the wave issuing MFMAs goes first while the other wave of its SIMD
                // issues copies or fragment reads (1-2% faster on FC1; FC2 measured 1-2%
                // slower with it)
                if constexpr (kSwiGLU) __builtin_amdgcn_s_setprio(1);
                // D = B-rows x A-rows: lane keeps one A row and 4 consecutive columns per
                // register group
#pragma unroll
                for (int i = 0; i < RB; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            fb[cur_buf][j], fa[cur_buf][i], acc[i][j], 0, 0, 0);
                if constexpr (kSwiGLU) __builtin_amdgcn_s_setprio(0);
            }
            if (kk + 1 == BK / 16 && kt + 1 < nk) {
                // behind slice kt's last MFMAs: wait for slice kt+1 everywhere (slices up to
                // kt+kStages-1 are issued); one decode step of the next item (its loads go
                // out before the next copies); slice kt's slot then takes slice kt+kStages;
                // first fragments of slice kt+1
                const int issued = kt + M::kStages - 1 < nk ? kt + M::kStages - 1 : nk - 1;
                wait_slices<kRowsA>(issued - (kt + 1), a_copy);
                if (kt >= first_step && step < kDecodeSteps)
                    decode_step<kSwiGLU, kGather>(step++, nxt, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
                deferred = -1;
                if (kt + M::kStages < nk) {
                    if (parts_at(-1) != 0)
                        issue_slice<kSwiGLU, kGather, kRowsA>(g, cur, kt + M::kStages, smem_base, wave,
                                                              seg_row, seg_lchunk * 16u, parts_at(-1));
                    if (parts_at(-1) != (kPartA | kPartB)) deferred = kt + M::kStages;
                }
                if (active) load_frags(kt + 1, 0, cur_buf ^ 1);
            }
        }
    }

    // every wave is done with the ring; finish decoding the next item and start its slices
    wait_copies_and_barrier(0);
    if (step < 2) {
        if (step == 0) decode_step<kSwiGLU, kGather>(0, nxt, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
        decode_step<kSwiGLU, kGather>(1, nxt, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
        __syncthreads();
        step = 2;
    }
    for (; step < kDecodeSteps; ++step) {
        // steps 4 and 5 back to back: the gathered rows must be in LDS first (only that copy
        // is in flight here)
        if (kGather && step == 5) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        decode_step<kSwiGLU, kGather>(step, nxt, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
    }
    issue_prologue<kSwiGLU, kGather>(g, nxt, smem_base, wave, opaque(seg_row), opaque(seg_lchunk) * 16u);
    if constexpr (kDirect) {
        const Item nu = uniform_item(nxt);
        if (nu.rows_a != 0) issue_dir_copy(g, nu, wave, dbuf ^ 1);
    }

    // epilogue: acc[i][j][4c + e] = C[tile row wrow + i*32 + lane%32][col + 8c + 4(lane/32) + e].
    // Lanes l and l + 32 hold one row.  One v_permlane32_swap per pair of packed registers
    // (groups c and c + 2) leaves lane l with columns 0..15 and lane l + 32 with columns
    // 16..31 of each 32-column block, each as two 16-byte pieces in column order.
    if (active) {
        const int le = opaque(lane);
        const int hi16 = le >= 32 ? 16 : 0;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int tr = wrow + i * 32 + (le & 31);
            const int rl = tr & (HALF - 1);
            // selects, not an indexed load: the item stays in registers
            const bool h1 = tr >= HALF;
            const bool row_ok = rl < (h1 ? cur.h_rows[1] : cur.h_rows[0]);
            uint16_t* crow = g.C + (int64_t)((h1 ? cur.h_row0[1] : cur.h_row0[0]) + rl) * g.ldc;
            // direct rows: out[token] instead of the expert-output row (tokens checked: a
            // table over rows the dir entries do not describe still stores inside out)
            int dtok = -1;
            float dw = 0.f;
            if constexpr (kDirect) {
                const int tk = g.gidx[dbuf * 512 + tr];
                if (tk >= 0 && tk < g.T) {
                    dtok = tk;
                    dw = __int_as_float(g.gidx[dbuf * 512 + 256 + tr]);
                    crow = g.out + (int64_t)tk * g.ldc;
                }
            }
            constexpr int NJ = kSwiGLU ? 1 : 2;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                uint32_t pk[4][2];  // [register group c][half]: columns 8c + 4(lane/32) + 0..3
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (kSwiGLU) {
                            const float gt = acc[i][0][4 * c + e];
                            const float up = acc[i][1][4 * c + e];
                            // SiLU(g) * u = g * u / (1 + 2^(-g log2 e))
                            const float den = 1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f);
                            v[e] = gt * __builtin_amdgcn_rcpf(den) * up;
                        } else {
                            v[e] = acc[i][j][4 * c + e];
                        }
                    }
                    pk[c][0] = pack_bf16x2(v[0], v[1]);
                    pk[c][1] = pack_bf16x2(v[2], v[3]);
                    if constexpr (kDirect) {
                        if (dtok >= 0) {
                            pk[c][0] = weight_bf16x2(pk[c][0], dw);
                            pk[c][1] = weight_bf16x2(pk[c][1], dw);
                        }
                    }
                }
                // swap(x, y) exchanges lanes 32..63 of x with lanes 0..31 of y: afterwards x
                // holds (lane l: own group c; lane l + 32: lane l's group c + 2) and y holds
                // (lane l: lane l + 32's group c; lane l + 32: own group c + 2)
                uint32_t xs[2][2], ys[2][2];
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const auto r = __builtin_amdgcn_permlane32_swap(pk[c][s], pk[c + 2][s], false, false);
                        xs[c][s] = r[0];
                        ys[c][s] = r[1];
                    }
                const int col0 = kSwiGLU ? cur.nt * (BN / 2) + wn * 32
                                         : cur.nt * BN + wn * 64 + j * 32;
                if (row_ok && col0 < g.n_cols) {  // n_cols is a multiple of 64: all or none
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        uint4 o;
                        o.x = xs[c][0];
                        o.y = xs[c][1];
                        o.z = ys[c][0];
                        o.w = ys[c][1];
                        *reinterpret_cast<uint4*>(crow + col0 + hi16 + 8 * c) = o;
                    }
                }
            }
        }
    }
}

// C[p][c] for the rows p of each tile (expert l):
//   FC1 (kSwiGLU): act[p][c] = SiLU(A[p].W1[l][c]) * (A[p].W1[l][I + c]), c < I
//   FC2:           yp[p][c]  = A[p].W2[l][c],                              c < H
// A is [a_rows, Kdim], B per expert [b_rows, Kdim]; both K-contiguous.  With `gather`
// (row_token of the dispatch permutation), A[p] above means A[gather[p]]: the rows are read
// straight from the token rows of x and no permuted copy is needed.
//
// Items (tile, column tile) are cut into 8 contiguous ranges, one per XCD (workgroup w runs
// on XCD w % 8), so the items in flight on an XCD share A rows and B rows in its L2.
// Workgroups take items from their XCD's range through an atomic counter (in order,
// self-balancing); a workgroup whose range is drained helps the others.  Items are
// pipelined: the next one is claimed and decoded during the current one's last K slices and
// its first slices are in flight while the current one's results are written.
template <bool kSwiGLU, bool kGather, bool kDirect = false>
__global__ void __launch_bounds__(kThreads, 1)
ffn_bf16_kernel(const uint16_t* __restrict__ A, int64_t a_rows, int Kdim,
                const uint16_t* __restrict__ B, int64_t b_expert_stride, int b_rows,
                uint16_t* __restrict__ C, int ldc, int n_cols, int I, int NT,
                int max_blocks, int32_t* __restrict__ ws, const int32_t* __restrict__ gather,
                const int32_t* __restrict__ dir = nullptr, uint16_t* __restrict__ out = nullptr,
                int T = 0) {
    static_assert(!kDirect || (!kSwiGLU && !kGather), "direct rows are an FC2 epilogue");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];
    __shared__ int item_s[2];  // [0] the next item, [1] thread 0's last counter increment
    __shared__ __attribute__((aligned(256))) int32_t gidx[kWaves * 4 * MOE_WAVE];

    GemmArgs g;
    g.A = A; g.a_rows = a_rows; g.Kdim = Kdim;
    g.B = B; g.b_expert_stride = b_expert_stride; g.b_rows = b_rows;
    g.C = C; g.ldc = ldc; g.n_cols = n_cols; g.I = I; g.NT = NT;
    g.tiles = (const __attribute__((address_space(4))) int32_t*)(ws + WS_HEAD + max_blocks);
    g.gidx = gidx;
    g.gidx_lds = (uint32_t)(uintptr_t)(lds_u8_t*)reinterpret_cast<uint8_t*>(gidx);
    g.ctr = ws + (kSwiGLU ? WS_CTR_FC1 : WS_CTR_FC2);
    g.total = ws[WS_NTILES] * g.NT;
    g.per_xcd_items = (g.total + kXcds - 1) / kXcds;
    g.xcd = blockIdx.x % kXcds;
    g.gather = gather;
    g.dir = dir;
    g.out = out;
    g.T = T;

    const int tid = threadIdx.x;
    const int lane = moe_lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);
    const uint32_t smem_base = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    // A copy fills one 8-row segment: lane j writes physical chunk j%8 of segment row j/8 and
    // so fetches the logical chunk stored there.  This wave's segments all have the parity of
    // w, which is the only part of the segment index that enters the swizzle.
    const int seg_row = lane >> 3;
    const int seg_lchunk = swz_chunk((wave & 1) * 8 + seg_row, lane & 7);

    Queue qs{0};
    Item cur;
    decode_step<kSwiGLU, kGather>(0, cur, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
    decode_step<kSwiGLU, kGather>(1, cur, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
    __syncthreads();
    for (int s = 2; s < 6; ++s) {
        if (kGather && s == 5) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        decode_step<kSwiGLU, kGather>(s, cur, g, qs, item_s, tid, wave, seg_row, seg_lchunk);
    }
    issue_prologue<kSwiGLU, kGather>(g, cur, smem_base, wave, seg_row, seg_lchunk * 16u);
    int dbuf = 0;  // direct rows: the gidx buffer of the current item's row table
    if constexpr (kDirect) {
        const Item u = uniform_item(cur);
        if (u.rows_a != 0) issue_dir_copy(g, u, wave, 0);
    }

    for (;;) {
        const int rows_a = __builtin_amdgcn_readfirstlane(cur.rows_a);
        if (rows_a == 0) break;
        Item nxt;
        if (rows_a == 256)
            gemm_item<kSwiGLU, kGather, 256, kDirect>(g, cur, nxt, qs, item_s, smem, smem_base, tid, wave, lane,
                                    seg_row, seg_lchunk, dbuf);
        else if (rows_a == 128)
            gemm_item<kSwiGLU, kGather, 128, kDirect>(g, cur, nxt, qs, item_s, smem, smem_base, tid, wave, lane,
                                    seg_row, seg_lchunk, dbuf);
        else
            gemm_item<kSwiGLU, kGather, 64, kDirect>(g, cur, nxt, qs, item_s, smem, smem_base, tid, wave, lane,
                                   seg_row, seg_lchunk, dbuf);
        dbuf ^= 1;
        cur = nxt;
    }
    // the last workgroup out clears this GEMM's counters so the kernel can run again
    if (tid == 0) {
        int32_t* done = ws + (kSwiGLU ? WS_DONE_FC1 : WS_DONE_FC2);
        if (atomicAdd(done, 1) == (int)gridDim.x - 1) {
            for (int x = 0; x < kXcds; ++x) atomicExch(&g.ctr[x], 0);
            atomicExch(done, 0);
        }
    }
}

// float32 path (small layers): C[p][c] = A[p] . B[l][c] over the block table (FC1: SiLU of
// the gate product times the up product, B rows c and I + c).  Blocks that fail block_error
// are skipped (the schedule pass of the same call reports them); gathered rows outside
// [0, a_rows) read as zeros.  One workgroup per (block, 64
// output columns), grid-stride over those items; K is staged 64 at a time through LDS: the
// block's A rows (64 rows per pass, gathered through `gather` when given) and the 64
// columns' B rows.  Thread (rg, c) accumulates rows rg, rg+4, ..., rg+60 of column c with
// fmaf in ascending K order.  Rows of 65 floats keep the B reads conflict-free (lane c reads
// row c); A reads are wave-uniform broadcasts.
template <bool kSwiGLU>
__global__ void __launch_bounds__(256)
ffn_f32_kernel(const float* __restrict__ A, const int32_t* __restrict__ gather, int64_t a_rows,
               int Kdim, const float* __restrict__ B, int64_t b_expert_stride, int I,
               float* __restrict__ C, int ldc, int n_cols, const int32_t* __restrict__ blocks,
               const int32_t* __restrict__ n_blocks_ptr, int max_blocks, int E_loc,
               int64_t max_rows, const int32_t* __restrict__ dir = nullptr,
               float* __restrict__ out = nullptr, int T = 0) {
    constexpr int TC = 64, TK = 64, TR = 64, RPT = TR / 4;
    __shared__ float a_s[TR][TK + 1];
    __shared__ float g_s[TC][TK + 1];
    __shared__ float u_s[kSwiGLU ? TC : 1][TK + 1];
    int nb = *n_blocks_ptr;
    nb = nb < max_blocks ? nb : max_blocks;
    const int nct = (n_cols + TC - 1) / TC;
    const int tid = threadIdx.x, c = tid & (TC - 1), rg = tid / TC;
    for (int item = blockIdx.x; item < nb * nct; item += gridDim.x) {
        const int b = item / nct, ct = item - b * nct;
        const int l = blocks[4 * b + 1], row0 = blocks[4 * b + 2], m = blocks[4 * b + 3];
        if (block_error(l, row0, m, E_loc, max_rows) != 0) continue;  // uniform: whole workgroup
        const float* Bl = B + (int64_t)l * b_expert_stride;
        const int col = ct * TC + c;
        for (int r0 = 0; r0 < m; r0 += TR) {
            float ag[RPT], au[RPT];
#pragma unroll
            for (int j = 0; j < RPT; ++j) ag[j] = au[j] = 0.f;
            for (int k0 = 0; k0 < Kdim; k0 += TK) {
                __syncthreads();  // the previous slice's LDS reads are done
                for (int e = tid; e < TR * TK; e += 256) {
                    const int rr = e / TK, kk = e - rr * TK, r = r0 + rr;
                    float v = 0.f;
                    if (r < m && k0 + kk < Kdim) {
                        const int64_t arow = gather ? gather[row0 + r] : row0 + r;
                        if (arow >= 0 && arow < a_rows) v = A[arow * Kdim + k0 + kk];
                    }
                    a_s[rr][kk] = v;
                }
                for (int e = tid; e < TC * TK; e += 256) {
                    const int cc = e / TK, kk = e - cc * TK, cl = ct * TC + cc;
                    const bool in = cl < n_cols && k0 + kk < Kdim;
                    g_s[cc][kk] = in ? Bl[(int64_t)cl * Kdim + k0 + kk] : 0.f;
                    if (kSwiGLU) u_s[cc][kk] = in ? Bl[(int64_t)(I + cl) * Kdim + k0 + kk] : 0.f;
                }
                __syncthreads();
                const int kn = Kdim - k0 < TK ? Kdim - k0 : TK;
                for (int kk = 0; kk < kn; ++kk) {
                    const float wg = g_s[c][kk];
                    const float wu = kSwiGLU ? u_s[c][kk] : 0.f;
#pragma unroll
                    for (int j = 0; j < RPT; ++j) {
                        const float av = a_s[rg + 4 * j][kk];
                        ag[j] = fmaf(av, wg, ag[j]);
                        if (kSwiGLU) au[j] = fmaf(av, wu, au[j]);
                    }
                }
            }
            if (col < n_cols) {
#pragma unroll
                for (int j = 0; j < RPT; ++j) {
                    const int r = r0 + rg + 4 * j;
                    if (r < m) {
                        const float g = ag[j];
                        float* dst = C + (int64_t)(row0 + r) * ldc + col;
                        float v = kSwiGLU ? g / (1.f + expf(-g)) * au[j] : g;
                        if (!kSwiGLU && dir) {
                            // direct row: out[token] = fmaf(w, y, 0), as a one-entry combine
                            const int tk = dir[row0 + r];
                            if (tk >= 0 && tk < T) {
                                dst = out + (int64_t)tk * ldc + col;
                                v = fmaf(__int_as_float(dir[max_rows + row0 + r]), g, 0.f);
                            }
                        }
                        *dst = v;
                    }
                }
            }
        }
    }
}

int persistent_grid() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    int g = cus / kXcds * kXcds;  // one workgroup per CU (144 KB of LDS each)
    return g < kXcds ? kXcds : g;
}

}  // namespace

int64_t moe_ffn_workspace_elems_impl(int max_blocks) {
    return WS_HEAD + (int64_t)max_blocks + (int64_t)TILE_INTS * 2 * max_blocks;
}

hipError_t moe_launch_ffn_schedule(const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                                   int E_loc, int64_t max_rows, int32_t* ws, hipStream_t stream) {
    ffn_schedule_kernel<<<1, 256, 0, stream>>>(blocks, n_blocks, max_blocks, E_loc, max_rows, ws);
    return hipGetLastError();
}

hipError_t moe_launch_ffn_fc1(const void* a, const void* w1, moe_dtype_t dt, int H, int I,
                              int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                              int max_blocks, int32_t* ws, void* act, int64_t max_rows,
                              int64_t a_rows, const int32_t* gather, hipStream_t stream) {
    if (dt == MOE_F32) {
        const int64_t items = (int64_t)max_blocks * ((I + 63) / 64);
        const int grid = items < 2048 ? (int)items : 2048;
        ffn_f32_kernel<true><<<grid, 256, 0, stream>>>(
            static_cast<const float*>(a), gather, a_rows, H, static_cast<const float*>(w1),
            (int64_t)2 * I * H, I, static_cast<float*>(act), I, I, blocks, n_blocks, max_blocks,
            E_loc, max_rows);
        return hipGetLastError();
    }
    if (gather)
        ffn_bf16_kernel<true, true><<<persistent_grid(), kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(a), a_rows, H, static_cast<const uint16_t*>(w1),
            (int64_t)2 * I * H, 2 * I, static_cast<uint16_t*>(act), I, I, I,
            (I + BN / 2 - 1) / (BN / 2), max_blocks, ws, gather);
    else
        ffn_bf16_kernel<true, false><<<persistent_grid(), kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(a), a_rows, H, static_cast<const uint16_t*>(w1),
            (int64_t)2 * I * H, 2 * I, static_cast<uint16_t*>(act), I, I, I,
            (I + BN / 2 - 1) / (BN / 2), max_blocks, ws, nullptr);
    return hipGetLastError();
}

hipError_t moe_launch_ffn_fc2(const void* act, const void* w2, moe_dtype_t dt, int H, int I,
                              int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                              int max_blocks, int32_t* ws, void* yp, int64_t max_rows,
                              hipStream_t stream, const int32_t* dir, void* out, int T) {
    if (dt == MOE_F32) {
        const int64_t items = (int64_t)max_blocks * ((H + 63) / 64);
        const int grid = items < 2048 ? (int)items : 2048;
        ffn_f32_kernel<false><<<grid, 256, 0, stream>>>(
            static_cast<const float*>(act), nullptr, max_rows, I, static_cast<const float*>(w2),
            (int64_t)H * I, I, static_cast<float*>(yp), H, H, blocks, n_blocks, max_blocks,
            E_loc, max_rows, dir, static_cast<float*>(out), T);
        return hipGetLastError();
    }
    if (dir)
        ffn_bf16_kernel<false, false, true><<<persistent_grid(), kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(act), max_rows, I, static_cast<const uint16_t*>(w2),
            (int64_t)H * I, H, static_cast<uint16_t*>(yp), H, H, I, (H + BN - 1) / BN,
            max_blocks, ws, nullptr, dir, static_cast<uint16_t*>(out), T);
    else
        ffn_bf16_kernel<false, false><<<persistent_grid(), kThreads, 0, stream>>>(
            static_cast<const uint16_t*>(act), max_rows, I, static_cast<const uint16_t*>(w2),
            (int64_t)H * I, H, static_cast<uint16_t*>(yp), H, H, I, (H + BN - 1) / BN,
            max_blocks, ws, nullptr);
    return hipGetLastError();
}
