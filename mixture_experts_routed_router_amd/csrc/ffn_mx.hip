// ffn_mx.hip -- SwiGLU expert FFN with MXFP4 weights and MXFP8 activations (moe_expert_ffn_mx).
//
// MegaFlux §4.1 (Platform and configurations): the forward pass runs the expert GEMMs with
// MXFP4 weights and MXFP8 activations, accumulating in float32; §2.1: FC1 (gate and up
// projections), the SwiGLU activation, FC2.  Element and scale encodings are those of the OCP
// Microscaling Formats (MX) v1.0: FP8 E4M3 / FP4 E2M1 elements, one E8M0 power-of-two scale per
// 32 consecutive values along K.  The activation between the GEMMs is itself stored in MXFP8:
// FC1's epilogue quantizes each row's 32-column blocks with the rule of moe_mx_quantize.
//
// Both GEMMs run on gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4): a 32 x 32
// x 64 product of FP4 weights (first operand) and FP8 token rows (second operand), each
// operand carrying one E8M0 scale per row per 32-value block, accumulated into float32.
// Measured operand layouts: an FP8 operand's lane l holds row l % 32, bytes 0..15 =
// K 16(l/32) .. +15 of the first 32-value block and bytes 16..31 the same of the second; an FP4
// operand's lane l holds row l % 32, K 32(l/32) .. +31 (low nibble first) in its first four
// registers; lane l's scale is that of (row l % 32, block l / 32); the result layout is that
// of the other 32 x 32 MFMAs (acc[r] = C[8(r/4) + 4(l/32) + r%4][l % 32], rows = weights).
//
// Structure: the bf16 path's tile schedule (each expert's rows cut into 128-row halves paired
// into 256-row tiles), items split statically over the XCDs; one item = one tile x 256 weight rows
// (FC1: 128 gate rows and the matching 128 up rows -> 128 activation columns; FC2: 256
// columns of H).  K advances 128 values per stage through a 3-deep LDS ring of 50 KB stages
// (256 token rows x 128 B of FP8 codes, 256 weight rows x 64 B of FP4 codes, and one 4-byte
// word of scales per row), filled by direct-to-LDS copies; each of the 8 waves computes 128
// weight rows x 64 token rows (8 accumulator tiles) with 16 MFMAs per stage.  Weight rows
// first means a lane ends with 16 output columns of one token row: the MXFP8 block maximum of
// FC1's activation is an in-lane max and one lane swap, and its codes leave as one 16-byte
// store per lane.  A K that is not a multiple of 128 ends with a half stage (the second MFMA
// step skipped; its copies re-read valid bytes of the same rows).
#include "moe_launch.h"
#include "moe_lds.h"
#include "moe_ffn_ws.h"
#include "moe_mx.h"

namespace {

using namespace moe_ffn_ws;

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * MOE_WAVE;
constexpr int BK = 128;                       // K values per stage
constexpr int kStages = 3;
constexpr int TOK_ROW = BK;                   // 128 B of FP8 codes per token row per stage
constexpr int W_ROW = BK / 2;                 // 64 B of FP4 codes per weight row per stage
constexpr int W_OFF = 256 * TOK_ROW;          // token rows: [0, 32 KB)
constexpr int TSC_OFF = W_OFF + 256 * W_ROW;  // weight rows: [32 KB, 48 KB)
constexpr int WSC_OFF = TSC_OFF + 256 * 4;    // token scale words, then weight scale words
constexpr int STAGE = WSC_OFF + 256 * 4;      // 50 KB
constexpr int SMEM_BYTES = kStages * STAGE;   // 150 KB
constexpr int kCopies = 7;                    // per wave per stage: 4 token, 2 weight, 1 scale

// Kernel-wide arguments.
struct MxArgs {
    const uint8_t* aq;      // token codes [a_rows, K] (FP8); the rows of x with `gather`
    const uint8_t* as;      // token scales [a_rows, sp]
    const int32_t* gather;  // row_token (row p's input is row gather[p]) or nullptr
    int64_t a_rows;         // rows of aq / as (gathered token rows outside [0, a_rows) read row 0)
    int K, sp;              // values per row, scale bytes per row
    const uint8_t* wq;      // weight codes [E_loc][wrows, K / 2] (FP4)
    const uint8_t* wsc;     // weight scales [E_loc][wrows, sp]
    int64_t wq_estride, ws_estride;
    int n_out;              // output columns: I (FC1) or H (FC2)
    int I;
    uint8_t* actq;          // FC1: [rows, I] FP8 codes
    uint8_t* acts;          // FC1: [rows, act_sp] scales
    int act_sp;
    uint16_t* yp;           // FC2: [rows, H] bf16
    // FC2 with direct rows: dir[p] = the token whose only local entry is row p (else -1),
    // dir[a_rows + p] its weight's bits; such a row goes to out[token], weighted
    const int32_t* dir;
    uint16_t* out;
    int T;
    const int32_t* tiles;
    const int32_t* ntiles;
    int NT;
};

// Per-launch values every workgroup derives once.
struct MxCtx {
    int total, per_xcd, xcd, rank, nwg_xcd;  // items; this workgroup's XCD, rank on it, count
    uint32_t gidx;                // LDS address of the staged row_token entries (gather)
    int tid, wave, lane;
    int tok_lc, w_lc;             // logical chunk this lane copies (token / weight rows)
    uint32_t tok_back, w_back;    // half-slice fallback distance for those chunks
    int nk;                       // K slices (the last one half when K % 128 == 64)
    bool k_half;
    uint32_t sbase;               // LDS address of the ring
};

// One item: (tile, column tile) and this lane's copy offsets (bytes from the copy bases at
// slice 0; token offsets below 4 GiB).  it < 0: no item, this workgroup is done.
struct MxItem {
    int it, j;  // item index; this workgroup's item count so far
    int ts, cnt;
    int l, nt;
    int h_row0[2], h_rows[2];
    uint32_t tok[4], w[2], sc;
};

// Row p (permuted position) of tile row r, clamped to a row of the tile (read, never stored).
__device__ __forceinline__ int tile_pos(const MxItem& it, int r) {
    const bool h1 = r >= HALF && it.h_rows[1] > 0;
    const int rr = h1 ? r - HALF : (r >= HALF ? 0 : r);
    const int hr = h1 ? it.h_rows[1] : it.h_rows[0];
    return (h1 ? it.h_row0[1] : it.h_row0[0]) + (rr < hr ? rr : hr - 1);
}

// Weight row of the expert for item row r (0..255).  FC1: rows 0-63 gate columns
// 128 nt + 0..63, 64-127 the matching up rows (I + column), 128-191 gate 128 nt + 64..127,
// 192-255 their up rows; FC2: column 256 nt + r of H.  Clamped to the last column (read,
// never stored).
template <bool kFC1>
__device__ __forceinline__ uint32_t w_row(const MxArgs& g, int nt, int r) {
    if (kFC1) {
        int c = nt * 128 + 64 * (r >> 7) + (r & 63);
        c = c < g.I ? c : g.I - 1;
        return (uint32_t)((r & 64) ? g.I + c : c);
    }
    const int c = nt * 256 + r;
    return (uint32_t)(c < g.n_out ? c : g.n_out - 1);
}

// Copy geometry.  Token copy j of wave w fills 8-row segment w + 8j (1 KB: tile rows
// 8(w + 8j) .. +7, lane i -> row + i/8, physical chunk i%8); weight copy j fills 16-row segment
// w + 8j (lane i -> row + i/4, physical chunk i%4); the scale copy of waves 0-3 fills token
// scale words 64w .. 64w + 63, of waves 4-7 weight scale words 64(w-4) .. +63.
// LDS swizzles (ds_read_b128 serves 16 lanes over 64 banks): token row r's logical 16-byte
// chunk c at physical chunk c ^ ((r >> 1) & 7) (128-byte rows), weight row r's chunk c at
// c ^ ((r >> 2) & 3) (64-byte rows); 16 consecutive rows reading one logical chunk then hit
// 16 distinct bank groups.  The logical chunk a lane fetches is the same for all its copies.

// Items are assigned statically: the item list is cut into 8 contiguous ranges, one per XCD
// (workgroup w runs on XCD w % 8), and the workgroups of an XCD take its range round-robin, so
// the items in flight on an XCD are neighbours (they share A rows and B rows in its L2).  Every
// item costs the same (256 token rows x 256 weight rows x K), so a static split is balanced and
// needs no counters.  Tile records are read with scalar loads and row_token entries are staged
// through LDS by a direct copy, so no decode step makes a wave wait for the slice copies in
// flight.  Decoding the next item takes four steps, one per slice boundary:
//   0: the item index; load its tile group's first tile and tile count
//   1: (tile, column tile); load the tile record
//   2: gather: copy the row_token entries of the tile's 256 rows into LDS (waves 0-3)
//   3: this lane's copy offsets (gather: from the staged entries; steps 2 and 3 must be
//      separated by a wait for the copies and a barrier, as slice boundaries are)
typedef const __attribute__((address_space(4))) int32_t* sgpr_ptr_t;

// row_token entries of the next item's 256 tile rows (gather), staged by decode step 2
__shared__ __attribute__((aligned(16))) int32_t mx_gidx[256];
// FC2 with direct rows: two buffers of an item's 256 dir entries and 256 weights
__shared__ __attribute__((aligned(16))) int32_t mx_dir[1024];

// Direct rows: item `it`'s dir entries and weights into buffer `buf` of mx_dir; lane l of wave w
// moves word e = 64 w + l, entry (e & 255) of side e >> 8, for tile row e & 255 (clamped to the
// item's first row where the row is past its half, read and unused).  Issued with the item's
// first slice, one item ahead, into the buffer the item before last used (every wave has passed
// a barrier since that item's epilogue read it); the item's last wait covers it.
__device__ __forceinline__ void issue_dir_copy(const MxArgs& g, const MxCtx& c, const MxItem& it,
                                               int buf) {
    const int e = c.wave * MOE_WAVE + c.lane;
    const int side = e >> 8, r = e & 255, h = r >> 7, rl = r & (HALF - 1);
    const int hr = h ? it.h_rows[1] : it.h_rows[0];
    const int row = rl < hr ? (h ? it.h_row0[1] : it.h_row0[0]) + rl : it.h_row0[0];
    buf = __builtin_amdgcn_readfirstlane(buf);
    const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int32_t*)mx_dir;
    one_copy_dword(base + (uint32_t)(buf * 512 + c.wave * MOE_WAVE) * 4u, g.dir,
                   ((uint32_t)side * (uint32_t)g.a_rows + (uint32_t)row) * 4u);
}

template <bool kFC1>
__device__ __forceinline__ void decode_step(int step, MxItem& n, const MxArgs& g, const MxCtx& c) {
    switch (step) {
        case 0: {
            const int k = c.rank + n.j * c.nwg_xcd;
            const int itn = c.xcd * c.per_xcd + k;
            n.it = (k < c.per_xcd && itn < c.total) ? itn : -1;
            n.j += 1;
            if (n.it >= 0) {
                sgpr_ptr_t tg = (sgpr_ptr_t)(g.tiles + TILE_INTS * (n.it / g.NT));
                n.ts = tg[5];
                n.cnt = tg[6];
            }
            break;
        }
        case 1:
            if (n.it >= 0) {
                // item -> (tile, column tile): the expert's items in groups of kGroupTiles
                // tiles, column-tile-major inside a group
                const int local = n.it - n.ts * g.NT;
                const int grp = local / (kGroupTiles * g.NT);
                const int r = local - grp * (kGroupTiles * g.NT);
                const int rest = n.cnt - grp * kGroupTiles;
                const int ct = rest < kGroupTiles ? rest : kGroupTiles;
                n.nt = r / ct;
                sgpr_ptr_t tl = (sgpr_ptr_t)(g.tiles + TILE_INTS * (n.ts + grp * kGroupTiles + (r - n.nt * ct)));
                n.l = tl[0];
                n.h_row0[0] = tl[1];
                n.h_rows[0] = tl[2];
                n.h_row0[1] = tl[3];
                n.h_rows[1] = tl[4];
            }
            break;
        case 2:
            if (n.it >= 0 && g.gather && c.wave < 4) {
                const int p = tile_pos(n, 64 * c.wave + c.lane);
                one_copy_dword(c.gidx + 256u * (uint32_t)c.wave, g.gather, 4u * (uint32_t)p);
            }
            break;
        case 3:
            if (n.it >= 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 8 * (c.wave + 8 * j) + (c.lane >> 3);
                    int t = g.gather ? mx_gidx[r] : tile_pos(n, r);
                    t = t >= 0 && t < g.a_rows ? t : 0;  // row_token -1 (no entry): read, unused
                    n.tok[j] = (uint32_t)t * (uint32_t)g.K + 16u * c.tok_lc;
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    n.w[j] = w_row<kFC1>(g, n.nt, 16 * (c.wave + 8 * j) + (c.lane >> 2)) *
                                 (uint32_t)(g.K / 2) + 16u * c.w_lc;
                if (c.wave < 4) {
                    const int r = 64 * c.wave + c.lane;
                    int t = g.gather ? mx_gidx[r] : tile_pos(n, r);
                    t = t >= 0 && t < g.a_rows ? t : 0;
                    n.sc = (uint32_t)t * (uint32_t)g.sp;
                } else {
                    n.sc = w_row<kFC1>(g, n.nt, 64 * (c.wave - 4) + c.lane) * (uint32_t)g.sp;
                }
            }
            break;
        default:
            break;
    }
}

// The wave-uniform item fields as scalars.
__device__ __forceinline__ MxItem uniform_item(const MxItem& it) {
    MxItem u = it;
    u.it = __builtin_amdgcn_readfirstlane(it.it);
    u.j = __builtin_amdgcn_readfirstlane(it.j);
    u.l = __builtin_amdgcn_readfirstlane(it.l);
    u.nt = __builtin_amdgcn_readfirstlane(it.nt);
    u.h_row0[0] = __builtin_amdgcn_readfirstlane(it.h_row0[0]);
    u.h_row0[1] = __builtin_amdgcn_readfirstlane(it.h_row0[1]);
    u.h_rows[0] = __builtin_amdgcn_readfirstlane(it.h_rows[0]);
    u.h_rows[1] = __builtin_amdgcn_readfirstlane(it.h_rows[1]);
    return u;
}

// Issue this wave's 7 copies of K slice s into ring stage s % 3.  In a half slice (the last,
// when K % 128 == 64) lanes whose chunk lies beyond K fetch the chunk 64 (tokens) / 32
// (weights) bytes before it instead: in bounds, and never read back.
__device__ __forceinline__ void issue_slice(const MxArgs& g, const MxCtx& c, const MxItem& it,
                                            int s) {
    const bool half = c.k_half && s == c.nk - 1;
    const uint32_t stage = c.sbase + (uint32_t)((s % kStages) * STAGE);
    const uint32_t kt = (uint32_t)s * TOK_ROW - (half ? c.tok_back : 0u);
    const uint32_t kw = (uint32_t)s * W_ROW - (half ? c.w_back : 0u);
    const uint8_t* wq_l = g.wq + (int64_t)it.l * g.wq_estride;
#pragma unroll
    for (int j = 0; j < 4; ++j) one_copy(stage + (uint32_t)((c.wave + 8 * j) * 1024), g.aq, it.tok[j] + kt);
#pragma unroll
    for (int j = 0; j < 2; ++j)
        one_copy(stage + (uint32_t)(W_OFF + (c.wave + 8 * j) * 1024), wq_l, it.w[j] + kw);
    if (c.wave < 4)
        one_copy_dword(stage + (uint32_t)(TSC_OFF + c.wave * 256), g.as, it.sc + 4u * (uint32_t)s);
    else
        one_copy_dword(stage + (uint32_t)(WSC_OFF + (c.wave - 4) * 256),
                       g.wsc + (int64_t)it.l * g.ws_estride, it.sc + 4u * (uint32_t)s);
}

// The first slices of an item (the ring must be free).
// Slices [s0, s1) of the first stages of an item (the ring must be free).
__device__ __forceinline__ void issue_prologue(const MxArgs& g, const MxCtx& c, const MxItem& item,
                                               int s0 = 0, int s1 = kStages) {
    const MxItem it = uniform_item(item);
    if (it.it < 0) return;
    const int pre = c.nk < s1 ? c.nk : s1;
    for (int s = s0; s < pre; ++s) issue_slice(g, c, it, s);
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Operands of one 64-value MFMA step m of a slice: wave (fh, tq) multiplies weight rows
// 128 fh + 32 fb (fb 0..3) by token rows 64 tq + 32 tb (tb 0..1).
struct Frags {
    uint4 wf[4];  // FP4: 16 bytes per lane (the MFMA's first four registers)
    v8i_t tf[2];
};

__device__ __forceinline__ void load_frags(Frags& f, const uint8_t* stage, int fh, int tq, int lane, int m) {
    const int r32 = lane & 31, hi = lane >> 5;
    const int wsw = (lane >> 2) & 3;  // weight row swizzle: ((32 fb + r32) >> 2) & 3
    const int tsw = (lane >> 1) & 7;  // token row swizzle: ((32 tb + r32) >> 1) & 7
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
        const int row = 128 * fh + 32 * fb + r32;
        f.wf[fb] = lds16(stage + W_OFF + row * W_ROW + (((2 * m + hi) ^ wsw) << 4));
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int row = 64 * tq + 32 * tb + r32;
        const uint4 a = lds16(stage + row * TOK_ROW + (((4 * m + hi) ^ tsw) << 4));
        const uint4 b = lds16(stage + row * TOK_ROW + (((4 * m + 2 + hi) ^ tsw) << 4));
        f.tf[tb] = v8i_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
}

// The slice's scales: lane l keeps the 4 scale bytes of its row shifted so that block
// 2m + l/32 of step m sits in bits 16m .. 16m + 7.
struct Scales {
    uint32_t w[4], t[2];
};

__device__ __forceinline__ void load_scales(Scales& sc, const uint8_t* stage, int fh, int tq, int lane) {
    const int r32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
        sc.w[fb] = *reinterpret_cast<const uint32_t*>(stage + WSC_OFF + 4 * (128 * fh + 32 * fb + r32)) >> (8 * hi);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
        sc.t[tb] = *reinterpret_cast<const uint32_t*>(stage + TSC_OFF + 4 * (64 * tq + 32 * tb + r32)) >> (8 * hi);
}

__device__ __forceinline__ void mfma_step(v16f_t (&acc)[4][2], const Frags& f, const Scales& sc, int m) {
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            acc[fb][tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                v8i_t{(int)f.wf[fb].x, (int)f.wf[fb].y, (int)f.wf[fb].z, (int)f.wf[fb].w, 0, 0, 0, 0},
                f.tf[tb], acc[fb][tb], 4 /* A: FP4 E2M1 */, 0 /* B: FP8 E4M3 */, 0,
                (int)((sc.w[fb] >> (16 * m)) & 0xFFu), 0, (int)((sc.t[tb] >> (16 * m)) & 0xFFu));
}

// FC1 epilogue: act = SiLU(gate) * up for this wave's 64 activation columns x 64 token rows,
// quantized per 32-column block to MXFP8 (the moe_mx_quantize rule) and stored.
__device__ __forceinline__ void epilogue_fc1(const MxArgs& g, const MxItem& it,
                                             const v16f_t (&acc)[4][2], int fh, int tq, int lane) {
    const int hi = lane >> 5;
#pragma unroll
    for (int ab = 0; ab < 2; ++ab) {
        const int col0 = it.nt * 128 + 64 * fh + 32 * ab;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            float a[16];
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float gt = acc[ab][tb][i], up = acc[ab + 2][tb][i];
                // SiLU(g) * u = g * u / (1 + 2^(-g log2 e))
                const float den = 1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f);
                a[i] = gt * __builtin_amdgcn_rcpf(den) * up;
                amax = fmaxf(amax, fabsf(a[i]));
            }
            // lanes l and l + 32 hold the two halves of one token row's 32-column block; after
            // the swap one of the two results is the lane's own maximum, the other its partner's
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax),
                                                             false, false);
            amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            const int se = mx_shared_exp(amax, 8);
            uint32_t w[4];  // columns 8q + 4 hi .. + 3
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = e4m3_word(ldexpf(a[4 * q], -se), ldexpf(a[4 * q + 1], -se),
                                 ldexpf(a[4 * q + 2], -se), ldexpf(a[4 * q + 3], -se));
            // swap groups q and q + 2: lane l keeps columns 0..15, lane l + 32 gets 16..31
            uint32_t xs[2], ys[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const auto r = __builtin_amdgcn_permlane32_swap(w[q], w[q + 2], false, false);
                xs[q] = r[0];
                ys[q] = r[1];
            }
            const int tr = 64 * tq + 32 * tb + (lane & 31);
            const bool h1 = tr >= HALF;
            const int rl = tr & (HALF - 1);
            if (col0 < g.I && rl < (h1 ? it.h_rows[1] : it.h_rows[0])) {
                const int64_t p = (h1 ? it.h_row0[1] : it.h_row0[0]) + rl;
                uint4 o;
                o.x = xs[0];
                o.y = ys[0];
                o.z = xs[1];
                o.w = ys[1];
                *reinterpret_cast<uint4*>(g.actq + p * g.I + col0 + 16 * hi) = o;
                if (!hi) g.acts[p * g.act_sp + col0 / 32] = (uint8_t)(se + 127);
            }
        }
    }
}

// Two floats -> packed bf16x2 (low half = a), nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// bf16 pair u reweighted as a one-entry combine does it: bf16(fmaf(w, y, 0)) per half, rounded
// to nearest even by the hardware conversion (the combine's software rounding gives the same
// bits for finite values).
__device__ __forceinline__ uint32_t weight_bf16x2(uint32_t u, float w) {
    return pack_bf16x2(fmaf(w, __uint_as_float(u << 16), 0.f),
                       fmaf(w, __uint_as_float(u & 0xFFFF0000u), 0.f));
}

// FC2 epilogue: this wave's 128 columns of H x 64 token rows, bf16.  kDirect: rows whose dir
// entry (buffer dbuf) names a token in [0, T) go to that token's out row, weighted.
template <bool kDirect>
__device__ __forceinline__ void epilogue_fc2(const MxArgs& g, const MxItem& it,
                                             const v16f_t (&acc)[4][2], int fh, int tq, int lane,
                                             int dbuf) {
    const int hi = lane >> 5;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int tr = 64 * tq + 32 * tb + (lane & 31);
        const bool h1 = tr >= HALF;
        const int rl = tr & (HALF - 1);
        const bool row_ok = rl < (h1 ? it.h_rows[1] : it.h_rows[0]);
        const int64_t p = (h1 ? it.h_row0[1] : it.h_row0[0]) + rl;
        int dtok = -1;
        float dw = 0.f;
        if constexpr (kDirect) {
            const int tk = mx_dir[dbuf * 512 + tr];
            if (tk >= 0 && tk < g.T) {
                dtok = tk;
                dw = __int_as_float(mx_dir[dbuf * 512 + 256 + tr]);
            }
        }
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) {
            const int col0 = it.nt * 256 + 128 * fh + 32 * fb;
            uint32_t pk[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    pk[q][s] = pack_bf16x2(acc[fb][tb][4 * q + 2 * s], acc[fb][tb][4 * q + 2 * s + 1]);
            if constexpr (kDirect) {
                if (dtok >= 0) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int s = 0; s < 2; ++s) pk[q][s] = weight_bf16x2(pk[q][s], dw);
                }
            }
            uint32_t xs[2][2], ys[2][2];
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const auto r = __builtin_amdgcn_permlane32_swap(pk[q][s], pk[q + 2][s], false, false);
                    xs[q][s] = r[0];
                    ys[q][s] = r[1];
                }
            if (row_ok && col0 < g.n_out) {
                uint16_t* dst = (kDirect && dtok >= 0 ? g.out + (int64_t)dtok * g.n_out
                                                      : g.yp + p * g.n_out) + col0 + 16 * hi;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    uint4 o;
                    o.x = xs[q][0];
                    o.y = xs[q][1];
                    o.z = ys[q][0];
                    o.w = ys[q][1];
                    *reinterpret_cast<uint4*>(dst + 8 * q) = o;
                }
            }
        }
    }
}

// One item whose first slices are in flight: the K loop (slice s's MFMAs, then a wait for
// slice s + 1, one decode step of the next item, the copies of slice s + 3 into slice s's
// stage, and slice s + 1's first fragments); then the next item's first slices are issued
// and this item's results leave from registers while they land.
// The copies of the slice that a slice boundary makes room for go out after the next slice's
// first MFMA step instead of at the boundary, where every wave would wait in the address unit's
// queue before its first MFMA of the slice (FC1 2-4% and FC2 0-3% faster over the workloads'
// shapes, bit-identical).  All of them still go out before the next boundary's wait.
#ifndef FFN_MX_DEFER
#define FFN_MX_DEFER 1
#endif
constexpr bool kMxDeferCopies = FFN_MX_DEFER != 0;

template <bool kFC1, bool kDirect = false>
__device__ __forceinline__ void mx_item(const MxArgs& g, const MxCtx& c, const MxItem& cur_in,
                                        MxItem& nxt, uint8_t* smem, int dbuf) {
    const MxItem cur = uniform_item(cur_in);
    constexpr int kDecodeSteps = 4;
    nxt.j = cur.j;
    const int fh = c.wave >> 2, tq = c.wave & 3;
    const int nk = c.nk;
    const int pre = nk < kStages ? nk : kStages;
    const int first_step = nk - 1 - kDecodeSteps > 0 ? nk - 1 - kDecodeSteps : 0;

    v16f_t acc[4][2];
#pragma unroll
    for (int fb = 0; fb < 4; ++fb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[fb][tb][e] = 0.f;

    // slice 0 in LDS everywhere (stores of the previous item may still be counted: stricter)
    wait_pending_stages<kCopies, kStages - 1>(pre - 1);
    Frags f[2];  // operands of MFMA steps 0 and 1
    Scales sc;
    load_scales(sc, smem, fh, tq, c.lane);
    load_frags(f[0], smem, fh, tq, c.lane, 0);

    int step = 0;
    int deferred = -1;  // the slice whose copies go out after this slice's first MFMA step
    for (int s = 0; s < nk; ++s) {
        const uint8_t* stage = smem + (s % kStages) * STAGE;
        const bool half = c.k_half && s == nk - 1;
        mfma_step(acc, f[0], sc, 0);
        if (kMxDeferCopies && deferred >= 0) issue_slice(g, c, cur, deferred);
        if (!half) {
            load_frags(f[1], stage, fh, tq, c.lane, 1);
            mfma_step(acc, f[1], sc, 1);
        }
        if (s + 1 < nk) {
            // behind slice s's MFMAs: slice s + 1 everywhere (slices up to s + 2 are issued);
            // one decode step; slice s's stage takes slice s + 3; slice s + 1's first operands
            const int issued = s + kStages - 1 < nk ? s + kStages - 1 : nk - 1;
            wait_pending_stages<kCopies, kStages - 2>(issued - (s + 1));
            if (s >= first_step && step < kDecodeSteps) decode_step<kFC1>(step++, nxt, g, c);
            deferred = -1;
            if (s + kStages < nk) {
                if (kMxDeferCopies)
                    deferred = s + kStages;
                else
                    issue_slice(g, c, cur, s + kStages);
            }
            const uint8_t* nst = smem + ((s + 1) % kStages) * STAGE;
            load_scales(sc, nst, fh, tq, c.lane);
            load_frags(f[0], nst, fh, tq, c.lane, 0);
        }
    }

    // every wave is done with the ring; finish decoding the next item and start its slices
    wait_copies_n_and_barrier<0>();
    for (; step < kDecodeSteps; ++step) {
        if (step == 3) wait_copies_n_and_barrier<0>();  // staged row_token entries
        decode_step<kFC1>(step, nxt, g, c);
    }
    // the next item's slice 0 goes out before this item's stores, its other first slices after
    // them: the next item's first wait (for all but the last (stages - 1) slices' copies) then
    // covers slice 0 and the stores, not the slices behind them
    issue_prologue(g, c, nxt, 0, 1);
    if constexpr (kDirect) {
        const MxItem nu = uniform_item(nxt);
        if (nu.it >= 0) issue_dir_copy(g, c, nu, dbuf ^ 1);
    }

    if (kFC1)
        epilogue_fc1(g, cur, acc, fh, tq, c.lane);
    else
        epilogue_fc2<kDirect>(g, cur, acc, fh, tq, c.lane, dbuf);
    issue_prologue(g, c, nxt, 1, kStages);
}

// Persistent grouped GEMM, one workgroup per CU (150 KB of LDS).
template <bool kFC1, bool kDirect = false>
__global__ void __launch_bounds__(kThreads, 1)
ffn_mx_kernel(MxArgs g) {
    static_assert(!kDirect || !kFC1, "direct rows are an FC2 epilogue");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];
    MxCtx c;
    c.tid = threadIdx.x;
    c.lane = moe_lane_id();
    c.wave = __builtin_amdgcn_readfirstlane(c.tid / MOE_WAVE);
    c.sbase = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
    c.gidx = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int32_t*)mx_gidx;
    c.total = *g.ntiles * g.NT;
    c.per_xcd = (c.total + kXcds - 1) / kXcds;
    c.xcd = blockIdx.x % kXcds;
    c.rank = blockIdx.x / kXcds;
    c.nwg_xcd = (int)(gridDim.x / kXcds);
    c.tok_lc = (c.lane & 7) ^ ((4 * (c.wave & 1) + (c.lane >> 4)) & 7);
    c.w_lc = (c.lane & 3) ^ ((c.lane >> 4) & 3);
    c.tok_back = c.tok_lc >= 4 ? 64u : 0u;
    c.w_back = c.w_lc >= 2 ? 32u : 0u;
    c.nk = (g.K + BK - 1) / BK;
    c.k_half = (g.K % BK) != 0;

    MxItem cur;
    cur.j = 0;
    for (int s = 0; s < 4; ++s) {
        if (s == 3) wait_copies_n_and_barrier<0>();
        decode_step<kFC1>(s, cur, g, c);
    }
    issue_prologue(g, c, cur);
    int dbuf = 0;  // direct rows: the mx_dir buffer of the current item
    if constexpr (kDirect) {
        const MxItem u = uniform_item(cur);
        if (u.it >= 0) issue_dir_copy(g, c, u, 0);
    }
    for (;;) {
        if (__builtin_amdgcn_readfirstlane(cur.it) < 0) break;
        MxItem nxt;
        mx_item<kFC1, kDirect>(g, c, cur, nxt, smem, dbuf);
        dbuf ^= 1;
        cur = nxt;
    }
}

int mx_grid() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int g = cus / kXcds * kXcds;
    return g < kXcds ? kXcds : g;
}

}  // namespace

hipError_t moe_launch_ffn_mx_fc1(const uint8_t* xq, const uint8_t* xs, const int32_t* gather,
                                 int64_t x_rows, const uint8_t* w1q, const uint8_t* w1s, int H,
                                 int I,
                                 int max_blocks, int32_t* ws, uint8_t* actq, uint8_t* acts,
                                 hipStream_t stream) {
    MxArgs g{};
    g.aq = xq;
    g.as = xs;
    g.gather = gather;
    g.a_rows = x_rows;
    g.K = H;
    g.sp = (int)moe_mx_scale_pitch_impl(H);
    g.wq = w1q;
    g.wsc = w1s;
    g.wq_estride = (int64_t)2 * I * (H / 2);
    g.ws_estride = (int64_t)2 * I * g.sp;
    g.n_out = I;
    g.I = I;
    g.actq = actq;
    g.acts = acts;
    g.act_sp = (int)moe_mx_scale_pitch_impl(I);
    g.tiles = ws + WS_HEAD + max_blocks;
    g.NT = (I + 127) / 128;
    g.ntiles = ws + WS_NTILES;
    ffn_mx_kernel<true><<<mx_grid(), kThreads, 0, stream>>>(g);
    return hipGetLastError();
}

hipError_t moe_launch_ffn_mx_fc2(const uint8_t* actq, const uint8_t* acts, const uint8_t* w2q,
                                 const uint8_t* w2s, int H, int I, int max_blocks, int32_t* ws,
                                 uint16_t* yp, int64_t max_rows, hipStream_t stream,
                                 const int32_t* dir, void* out, int T) {
    MxArgs g{};
    g.aq = actq;
    g.as = acts;
    g.gather = nullptr;
    g.a_rows = max_rows;
    g.K = I;
    g.sp = (int)moe_mx_scale_pitch_impl(I);
    g.wq = w2q;
    g.wsc = w2s;
    g.wq_estride = (int64_t)H * (I / 2);
    g.ws_estride = (int64_t)H * g.sp;
    g.n_out = H;
    g.I = I;
    g.yp = yp;
    g.tiles = ws + WS_HEAD + max_blocks;
    g.NT = (H + 255) / 256;
    g.ntiles = ws + WS_NTILES;
    g.dir = dir;
    g.out = static_cast<uint16_t*>(out);
    g.T = T;
    if (dir)
        ffn_mx_kernel<false, true><<<mx_grid(), kThreads, 0, stream>>>(g);
    else
        ffn_mx_kernel<false><<<mx_grid(), kThreads, 0, stream>>>(g);
    return hipGetLastError();
}
