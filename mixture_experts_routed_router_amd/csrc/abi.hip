// abi.hip -- the C ABI of libmoe (declared in include/moe.h): host-side argument checks,
// static bounds, and the launches.  No allocation, no synchronisation, no global state.
#include "moe_launch.h"

namespace {

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t local_entries_bound(int T, int K, int E_loc) {
    int64_t a = (int64_t)T * K, b = (int64_t)T * E_loc;
    return a < b ? a : b;
}

bool valid_local_set(int E, int begin, int stride, int E_loc) {
    return E >= 1 && E_loc >= 1 && stride >= 1 && begin >= 0 &&
           (int64_t)begin + (int64_t)(E_loc - 1) * stride < E;
}

moe_status_t launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case MOE_ERR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

int64_t moe_max_rows(int T, int K, int E_loc, int block_m) {
    if (T < 1 || K < 1 || E_loc < 1 || !valid_block_m(block_m)) return -1;
    return local_entries_bound(T, K, E_loc) + (int64_t)E_loc * (block_m - 1);
}

int32_t moe_max_blocks(int T, int K, int E_loc, int P, int block_m) {
    if (T < 1 || K < 1 || E_loc < 1 || P < 1 || !valid_block_m(block_m)) return -1;
    int64_t n = (local_entries_bound(T, K, E_loc) + block_m - 1) / block_m + (int64_t)E_loc * P;
    return n > 0x7FFFFFFF ? -1 : (int32_t)n;
}

int32_t moe_max_moves(int E_loc, int P) {
    if (E_loc < 1 || P < 1) return -1;
    return E_loc + P;
}

int64_t moe_permute_workspace_elems(int T, int E_loc) {
    if (T < 1 || E_loc < 1) return -1;
    return (int64_t)((T + MOE_PERMUTE_CHUNK - 1) / MOE_PERMUTE_CHUNK) * E_loc;
}

moe_status_t moe_route(const float* logits, int T, int E, int K, int renormalize,
                       int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                       hipStream_t stream) {
    if (!logits || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_INVALID;
    if (T < 1 || E < 1 || K < 1 || K > E || (int64_t)T * E > 0x7FFFFFFFLL) return MOE_ERR_INVALID;
    if (E > 256 || K > MOE_MAX_K) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_route(logits, T, E, K, renormalize ? K : E, topk_ids, topk_w,
                                     expert_counts, stream));
}

moe_status_t moe_route_ref(const float* logits, int T, int E, int K, int k_ref,
                           int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                           hipStream_t stream) {
    if (!logits || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_INVALID;
    if (T < 1 || E < 1 || K < 1 || K > E || (int64_t)T * E > 0x7FFFFFFFLL) return MOE_ERR_INVALID;
    if (k_ref < K || k_ref > E) return MOE_ERR_INVALID;
    if (E > 256 || K > MOE_MAX_K || (k_ref > MOE_MAX_K && k_ref < E)) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_route(logits, T, E, K, k_ref, topk_ids, topk_w, expert_counts,
                                     stream));
}

moe_status_t moe_router_topk(const void* x, moe_dtype_t dt, const void* w_router, int T, int H,
                             int E, int K, int k_ref, float* logits, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_counts, hipStream_t stream) {
    if (!x || !w_router || !topk_ids || !topk_w || !expert_counts) return MOE_ERR_INVALID;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (T < 1 || H < 1 || E < 1 || K < 1 || K > E || k_ref < K || k_ref > E) return MOE_ERR_INVALID;
    if ((int64_t)T * E > 0x7FFFFFFFLL) return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID;
    if (E > 256 || K > MOE_MAX_K || (k_ref > MOE_MAX_K && k_ref < E)) return MOE_ERR_UNSUPPORTED;
    if (dt == MOE_BF16 && (H % 64 != 0 || (int64_t)T * H * 2 > 0xFFFFFFFFLL - 16))
        return MOE_ERR_UNSUPPORTED;
    if (dt == MOE_F32 && H % 4 != 0) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_router_topk(x, dt, w_router, T, H, E, K, k_ref, logits, topk_ids,
                                           topk_w, expert_counts, stream));
}

moe_status_t moe_permute(const void* x, moe_dtype_t dt, int T, int H, int K, int E,
                         const int32_t* topk_ids, const int32_t* expert_counts,
                         int expert_begin, int expert_stride, int E_loc, int block_m,
                         int32_t* expert_offsets, int32_t* entry_pos, int32_t* row_token,
                         void* xp, int64_t max_rows, int32_t* workspace,
                         int64_t workspace_elems, hipStream_t stream) {
    if (!x || !topk_ids || !expert_counts || !expert_offsets || !entry_pos || !row_token ||
        !workspace)
        return MOE_ERR_INVALID;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (T < 1 || H < 1 || K < 1 || K > E || !valid_block_m(block_m)) return MOE_ERR_INVALID;
    if (!valid_local_set(E, expert_begin, expert_stride, E_loc)) return MOE_ERR_INVALID;
    if ((int64_t)T * K > 0x7FFFFFFFLL) return MOE_ERR_INVALID;
    const int64_t row_bytes = (int64_t)H * (dt == MOE_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || !aligned16(x) || (xp && !aligned16(xp))) return MOE_ERR_INVALID;
    if (max_rows < moe_max_rows(T, K, E_loc, block_m)) return MOE_ERR_INVALID;
    if (max_rows > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
    if (workspace_elems < moe_permute_workspace_elems(T, E_loc)) return MOE_ERR_INVALID;
    if (K > MOE_MAX_K || E_loc > 256) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_permute(x, row_bytes, T, K, topk_ids, expert_counts, expert_begin,
                                       expert_stride, E_loc, block_m, expert_offsets, entry_pos,
                                       row_token, xp, workspace, stream));
}

moe_status_t moe_plan(const int32_t* expert_counts, int E, int expert_begin, int expert_stride,
                      int E_loc, int P, int block_m, int32_t* q, int32_t* moves,
                      int32_t* n_moves, int max_moves, int32_t* blocks, int32_t* n_blocks,
                      int max_blocks, int32_t* err_word, hipStream_t stream) {
    if (!expert_counts || !q || !moves || !n_moves || !blocks || !n_blocks)
        return MOE_ERR_INVALID;
    if (!aligned16(moves) || !aligned16(blocks)) return MOE_ERR_INVALID;  // 16-byte records
    if (!valid_local_set(E, expert_begin, expert_stride, E_loc) || P < 1 || E_loc % P != 0 ||
        !valid_block_m(block_m) || max_moves < 0 || max_blocks < 1)
        return MOE_ERR_INVALID;
    if (P > 64 || E_loc > 256 || E_loc * P > 4096) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_plan(expert_counts, expert_begin, expert_stride, E_loc, P,
                                    block_m, q, moves, n_moves, max_moves, blocks, n_blocks,
                                    max_blocks, err_word, stream));
}

namespace {

moe_status_t check_ffn_shape(moe_dtype_t dt, int H, int I, int E_loc, int max_blocks,
                             int64_t max_rows) {
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (H < 1 || I < 1 || E_loc < 1 || max_blocks < 1 || max_rows < 1) return MOE_ERR_INVALID;
    if (dt == MOE_BF16 && (H % 64 != 0 || I % 64 != 0)) return MOE_ERR_UNSUPPORTED;
    if (dt == MOE_F32 && (H % 4 != 0 || I % 4 != 0)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

int64_t moe_ffn_workspace_elems(int max_blocks) {
    if (max_blocks < 1) return -1;
    return moe_ffn_workspace_elems_impl(max_blocks);
}

moe_status_t moe_plan_blocks(const int32_t* expert_counts, int E, int expert_begin,
                             int expert_stride, int E_loc, int P, int block_m, int replica_budget,
                             int32_t* q, int32_t* moves, int32_t* n_moves, int max_moves,
                             int32_t* blocks, int32_t* n_blocks, int max_blocks,
                             int32_t* err_word, hipStream_t stream) {
    if (!expert_counts || !q || !moves || !n_moves || !blocks || !n_blocks)
        return MOE_ERR_INVALID;
    if (!valid_local_set(E, expert_begin, expert_stride, E_loc) || P < 1 || E_loc % P != 0 ||
        !valid_block_m(block_m) || max_moves < 0 || max_blocks < 1 || replica_budget < 0)
        return MOE_ERR_INVALID;
    if (P > 64 || E_loc / P > 64 || E_loc > 256 || E_loc * P > 4096 || replica_budget > 65536)
        return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_plan_blocks(expert_counts, expert_begin, expert_stride, E_loc, P,
                                           block_m, replica_budget, q, moves, n_moves, max_moves,
                                           blocks, n_blocks, max_blocks, err_word, stream));
}

moe_status_t moe_expert_ffn_tile_schedule(const int32_t* blocks, const int32_t* n_blocks,
                                          int max_blocks, int E_loc, int64_t max_rows,
                                          int32_t* workspace, int64_t workspace_elems,
                                          hipStream_t stream) {
    if (!blocks || !n_blocks || !workspace || max_blocks < 1 || E_loc < 1 || max_rows < 1)
        return MOE_ERR_INVALID;
    if (!aligned16(blocks)) return MOE_ERR_INVALID;  // 16-byte records
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256 || max_rows > 0x7FFFFFFFLL) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_ffn_schedule(blocks, n_blocks, max_blocks, E_loc, max_rows,
                                            workspace, stream));
}

moe_status_t moe_expert_ffn_fc1(const void* xp, const void* w1, moe_dtype_t dt, int H, int I,
                                int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                                int max_blocks, void* act, int64_t max_rows,
                                int32_t* workspace, int64_t workspace_elems,
                                hipStream_t stream) {
    if (!xp || !w1 || !blocks || !n_blocks || !act || !workspace) return MOE_ERR_INVALID;
    if (!aligned16(xp) || !aligned16(w1) || !aligned16(act) || !aligned16(blocks))
        return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_shape(dt, H, I, E_loc, max_blocks, max_rows);
    if (st != MOE_OK) return st;
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
    // the schedule checks every block (and writes the error word) for both dtypes
    st = launched(moe_launch_ffn_schedule(blocks, n_blocks, max_blocks, E_loc, max_rows,
                                          workspace, stream));
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_fc1(xp, w1, dt, H, I, E_loc, blocks, n_blocks, max_blocks,
                                       workspace, act, max_rows, max_rows, nullptr, stream));
}

moe_status_t moe_expert_ffn_fc1_gather(const void* x, const int32_t* row_token, int T,
                                       const void* w1, moe_dtype_t dt, int H, int I, int E_loc,
                                       const int32_t* blocks, const int32_t* n_blocks,
                                       int max_blocks, void* act, int64_t max_rows,
                                       int32_t* workspace, int64_t workspace_elems,
                                       hipStream_t stream) {
    if (!x || !row_token || !w1 || !blocks || !n_blocks || !act || !workspace)
        return MOE_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(act) || !aligned16(blocks) || T < 1)
        return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_shape(dt, H, I, E_loc, max_blocks, max_rows);
    if (st != MOE_OK) return st;
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
    // the bf16 GEMM addresses x rows with 32-bit byte offsets
    if (dt == MOE_BF16 && (int64_t)T * H * 2 > 0xFFFFFFFFLL - 16) return MOE_ERR_UNSUPPORTED;
    st = launched(moe_launch_ffn_schedule(blocks, n_blocks, max_blocks, E_loc, max_rows,
                                          workspace, stream));
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_fc1(x, w1, dt, H, I, E_loc, blocks, n_blocks, max_blocks,
                                       workspace, act, max_rows, T, row_token, stream));
}

moe_status_t moe_expert_ffn_fc2(const void* act, const void* w2, moe_dtype_t dt, int H, int I,
                                int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                                int max_blocks, void* yp, int64_t max_rows,
                                int32_t* workspace, int64_t workspace_elems,
                                hipStream_t stream) {
    if (!act || !w2 || !blocks || !n_blocks || !yp || !workspace) return MOE_ERR_INVALID;
    if (!aligned16(act) || !aligned16(w2) || !aligned16(yp)) return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_shape(dt, H, I, E_loc, max_blocks, max_rows);
    if (st != MOE_OK) return st;
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_ffn_fc2(act, w2, dt, H, I, E_loc, blocks, n_blocks, max_blocks,
                                       workspace, yp, max_rows, stream));
}

moe_status_t moe_expert_ffn_fc2_direct(const void* act, const void* w2, moe_dtype_t dt, int H,
                                       int I, int E_loc, const int32_t* blocks,
                                       const int32_t* n_blocks, int max_blocks, void* yp,
                                       int64_t max_rows, const int32_t* row_token,
                                       const int32_t* entry_pos, const float* topk_w, int T,
                                       int K, void* out, int32_t* row_direct,
                                       int32_t* workspace, int64_t workspace_elems,
                                       hipStream_t stream) {
    if (!act || !w2 || !blocks || !n_blocks || !yp || !workspace || !row_token || !entry_pos ||
        !topk_w || !out || !row_direct)
        return MOE_ERR_INVALID;
    if (!aligned16(act) || !aligned16(w2) || !aligned16(yp) || !aligned16(out))
        return MOE_ERR_INVALID;
    if (T < 1 || K < 1) return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_shape(dt, H, I, E_loc, max_blocks, max_rows);
    if (st != MOE_OK) return st;
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256 || K > MOE_MAX_K) return MOE_ERR_UNSUPPORTED;
    // the bf16 GEMM addresses the row table with 32-bit byte offsets
    if (max_rows > 0x7FFFFFFLL) return MOE_ERR_UNSUPPORTED;
    st = launched(moe_launch_direct_rows(row_token, entry_pos, topk_w, T, K, max_rows, row_direct,
                                         stream));
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_fc2(act, w2, dt, H, I, E_loc, blocks, n_blocks, max_blocks,
                                       workspace, yp, max_rows, stream, row_direct, out, T));
}

moe_status_t moe_expert_ffn(const void* xp, const void* w1, const void* w2, moe_dtype_t dt,
                            int H, int I, int E_loc, const int32_t* blocks,
                            const int32_t* n_blocks, int max_blocks, void* act, void* yp,
                            int64_t max_rows, int32_t* workspace, int64_t workspace_elems,
                            hipStream_t stream) {
    if (!w2 || !yp || !aligned16(w2) || !aligned16(yp)) return MOE_ERR_INVALID;
    moe_status_t st = moe_expert_ffn_fc1(xp, w1, dt, H, I, E_loc, blocks, n_blocks, max_blocks,
                                         act, max_rows, workspace, workspace_elems, stream);
    if (st != MOE_OK) return st;
    return moe_expert_ffn_fc2(act, w2, dt, H, I, E_loc, blocks, n_blocks, max_blocks, yp,
                              max_rows, workspace, workspace_elems, stream);
}

moe_status_t moe_expert_ffn_gather(const void* x, const int32_t* row_token, int T,
                                   const void* w1, const void* w2, moe_dtype_t dt, int H, int I,
                                   int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                                   int max_blocks, void* act, void* yp, int64_t max_rows,
                                   int32_t* workspace, int64_t workspace_elems,
                                   hipStream_t stream) {
    if (!w2 || !yp || !aligned16(w2) || !aligned16(yp)) return MOE_ERR_INVALID;
    moe_status_t st = moe_expert_ffn_fc1_gather(x, row_token, T, w1, dt, H, I, E_loc, blocks,
                                                n_blocks, max_blocks, act, max_rows, workspace,
                                                workspace_elems, stream);
    if (st != MOE_OK) return st;
    return moe_expert_ffn_fc2(act, w2, dt, H, I, E_loc, blocks, n_blocks, max_blocks, yp,
                              max_rows, workspace, workspace_elems, stream);
}

int64_t moe_mx_scale_pitch(int64_t cols) { return cols < 0 ? 0 : moe_mx_scale_pitch_impl(cols); }

moe_status_t moe_mx_quantize(const void* src, moe_dtype_t dt, int64_t rows, int64_t cols,
                             moe_mx_format_t fmt, uint8_t* codes, uint8_t* scales,
                             hipStream_t stream) {
    if (!src || !codes || !scales) return MOE_ERR_INVALID;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (fmt != MOE_MX_FP8 && fmt != MOE_MX_FP4) return MOE_ERR_INVALID;
    if (rows < 0 || cols < 32 || cols % 32 != 0) return MOE_ERR_INVALID;
    if (!aligned16(src) || !aligned16(codes)) return MOE_ERR_INVALID;
    if (rows > ((int64_t)1 << 40) / cols) return MOE_ERR_UNSUPPORTED;
    return launched(moe_launch_mx_quantize(src, dt, rows, cols, fmt, codes, scales, stream));
}

namespace {

bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

moe_status_t check_ffn_mx_shape(int H, int I, int E_loc, int max_blocks, int64_t max_rows,
                                const int32_t* blocks, const int32_t* n_blocks,
                                const int32_t* workspace, int64_t workspace_elems) {
    if (!blocks || !n_blocks || !workspace) return MOE_ERR_INVALID;
    if (H < 64 || I < 64 || E_loc < 1 || max_blocks < 1 || max_rows < 1) return MOE_ERR_INVALID;
    if (H % 64 != 0 || I % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (workspace_elems < moe_ffn_workspace_elems(max_blocks)) return MOE_ERR_INVALID;
    if (E_loc > 256) return MOE_ERR_UNSUPPORTED;
    // the GEMMs address rows with 32-bit byte offsets: token rows (x or act) and one expert's
    // weight rows
    const int64_t lim = 0xFFFFFFFFLL - 256;
    if (max_rows * I > lim || (int64_t)I * H > lim) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

moe_status_t moe_expert_ffn_mx_fc1(const uint8_t* xq, const uint8_t* xs, const int32_t* row_token,
                                   int64_t x_rows, const uint8_t* w1q, const uint8_t* w1s, int H,
                                   int I, int E_loc, const int32_t* blocks,
                                   const int32_t* n_blocks, int max_blocks, uint8_t* actq,
                                   uint8_t* acts, int64_t max_rows, int32_t* workspace,
                                   int64_t workspace_elems, hipStream_t stream) {
    if (!xq || !xs || !w1q || !w1s || !actq || !acts) return MOE_ERR_INVALID;
    if (!aligned16(xq) || !aligned16(w1q) || !aligned16(actq)) return MOE_ERR_INVALID;
    if (!aligned4(xs) || !aligned4(w1s)) return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_mx_shape(H, I, E_loc, max_blocks, max_rows, blocks, n_blocks,
                                         workspace, workspace_elems);
    if (st != MOE_OK) return st;
    if (x_rows < 1 || (!row_token && x_rows < max_rows)) return MOE_ERR_INVALID;
    if (x_rows * H > 0xFFFFFFFFLL - 256) return MOE_ERR_UNSUPPORTED;
    st = launched(moe_launch_ffn_schedule(blocks, n_blocks, max_blocks, E_loc, max_rows, workspace,
                                          stream));
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_mx_fc1(xq, xs, row_token, x_rows, w1q, w1s, H, I, max_blocks,
                                          workspace, actq, acts, stream));
}

moe_status_t moe_expert_ffn_mx_fc2(const uint8_t* actq, const uint8_t* acts, const uint8_t* w2q,
                                   const uint8_t* w2s, int H, int I, int E_loc,
                                   const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                                   void* yp, int64_t max_rows, int32_t* workspace,
                                   int64_t workspace_elems, hipStream_t stream) {
    if (!actq || !acts || !w2q || !w2s || !yp) return MOE_ERR_INVALID;
    if (!aligned16(actq) || !aligned16(w2q) || !aligned16(yp)) return MOE_ERR_INVALID;
    if (!aligned4(acts) || !aligned4(w2s)) return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_mx_shape(H, I, E_loc, max_blocks, max_rows, blocks, n_blocks,
                                         workspace, workspace_elems);
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_mx_fc2(actq, acts, w2q, w2s, H, I, max_blocks, workspace,
                                          static_cast<uint16_t*>(yp), max_rows, stream));
}

moe_status_t moe_expert_ffn_mx_fc2_direct(const uint8_t* actq, const uint8_t* acts,
                                          const uint8_t* w2q, const uint8_t* w2s, int H, int I,
                                          int E_loc, const int32_t* blocks,
                                          const int32_t* n_blocks, int max_blocks, void* yp,
                                          int64_t max_rows, const int32_t* row_token,
                                          const int32_t* entry_pos, const float* topk_w, int T,
                                          int K, void* out, int32_t* row_direct,
                                          int32_t* workspace, int64_t workspace_elems,
                                          hipStream_t stream) {
    if (!actq || !acts || !w2q || !w2s || !yp || !row_token || !entry_pos || !topk_w || !out ||
        !row_direct)
        return MOE_ERR_INVALID;
    if (!aligned16(actq) || !aligned16(w2q) || !aligned16(yp) || !aligned16(out))
        return MOE_ERR_INVALID;
    if (!aligned4(acts) || !aligned4(w2s)) return MOE_ERR_INVALID;
    if (T < 1 || K < 1) return MOE_ERR_INVALID;
    moe_status_t st = check_ffn_mx_shape(H, I, E_loc, max_blocks, max_rows, blocks, n_blocks,
                                         workspace, workspace_elems);
    if (st != MOE_OK) return st;
    if (K > MOE_MAX_K || max_rows > 0x7FFFFFFLL) return MOE_ERR_UNSUPPORTED;
    st = launched(moe_launch_direct_rows(row_token, entry_pos, topk_w, T, K, max_rows, row_direct,
                                         stream));
    if (st != MOE_OK) return st;
    return launched(moe_launch_ffn_mx_fc2(actq, acts, w2q, w2s, H, I, max_blocks, workspace,
                                          static_cast<uint16_t*>(yp), max_rows, stream, row_direct,
                                          out, T));
}

moe_status_t moe_expert_ffn_mx(const uint8_t* xq, const uint8_t* xs, const int32_t* row_token,
                               int64_t x_rows, const uint8_t* w1q, const uint8_t* w1s,
                               const uint8_t* w2q, const uint8_t* w2s, int H, int I, int E_loc,
                               const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                               uint8_t* actq, uint8_t* acts, void* yp, int64_t max_rows,
                               int32_t* workspace, int64_t workspace_elems, hipStream_t stream) {
    if (!w2q || !w2s || !yp || !aligned16(w2q) || !aligned16(yp) || !aligned4(w2s))
        return MOE_ERR_INVALID;
    moe_status_t st = moe_expert_ffn_mx_fc1(xq, xs, row_token, x_rows, w1q, w1s, H, I, E_loc,
                                            blocks, n_blocks, max_blocks, actq, acts, max_rows,
                                            workspace, workspace_elems, stream);
    if (st != MOE_OK) return st;
    return moe_expert_ffn_mx_fc2(actq, acts, w2q, w2s, H, I, E_loc, blocks, n_blocks, max_blocks,
                                 yp, max_rows, workspace, workspace_elems, stream);
}

moe_status_t moe_combine(const void* yp, moe_dtype_t dt, const float* topk_w,
                         const int32_t* entry_pos, int T, int H, int K, void* out,
                         hipStream_t stream) {
    if (!yp || !topk_w || !entry_pos || !out) return MOE_ERR_INVALID;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (T < 1 || H < 1 || K < 1) return MOE_ERR_INVALID;
    if (K > MOE_MAX_K) return MOE_ERR_UNSUPPORTED;
    const int64_t row_bytes = (int64_t)H * (dt == MOE_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || !aligned16(yp) || !aligned16(out)) return MOE_ERR_INVALID;
    return launched(moe_launch_combine(yp, dt, topk_w, entry_pos, T, H, K, out, stream));
}

moe_status_t moe_combine_multi(const void* yp, moe_dtype_t dt, const float* topk_w,
                               const int32_t* entry_pos, int T, int H, int K, void* out,
                               hipStream_t stream) {
    if (!yp || !topk_w || !entry_pos || !out) return MOE_ERR_INVALID;
    if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID;
    if (T < 1 || H < 1 || K < 1) return MOE_ERR_INVALID;
    if (K > MOE_MAX_K) return MOE_ERR_UNSUPPORTED;
    const int64_t row_bytes = (int64_t)H * (dt == MOE_BF16 ? 2 : 4);
    if (row_bytes % 16 != 0 || !aligned16(yp) || !aligned16(out)) return MOE_ERR_INVALID;
    return launched(moe_launch_combine(yp, dt, topk_w, entry_pos, T, H, K, out, stream, true));
}

}  // extern "C"
