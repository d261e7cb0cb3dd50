// moe_launch.h -- internal launchers of libmoe (one per step), called by the C ABI in abi.hip
// after the host-side argument checks.  Not part of the public interface.
#pragma once

#include "moe_device.h"

#define MOE_PERMUTE_CHUNK 16  // tokens per permutation chunk
#define MOE_MAX_K 16          // largest top-k

// k_ref: weights over the mass of the top k_ref experts (k_ref >= E: plain softmax)
hipError_t moe_launch_route(const float* logits, int T, int E, int K, int k_ref,
                            int32_t* topk_ids, float* topk_w, int32_t* counts,
                            hipStream_t stream);
hipError_t moe_launch_zero_counts(int32_t* counts, int E, hipStream_t stream);
hipError_t moe_launch_router_topk(const void* x, moe_dtype_t dt, const void* w_router, int T,
                                  int H, int E, int K, int k_ref, float* logits,
                                  int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  hipStream_t stream);

hipError_t moe_launch_permute(const void* x, int64_t row_bytes, int T, int K,
                              const int32_t* ids, const int32_t* counts, int begin, int stride,
                              int E_loc, int beta, int32_t* offsets, int32_t* entry_pos,
                              int32_t* row_token, void* xp, int32_t* ws, hipStream_t stream);

hipError_t moe_launch_plan(const int32_t* counts, int begin, int stride, int E_loc, int P,
                           int beta, int32_t* q, int32_t* moves, int32_t* n_moves,
                           int max_moves, int32_t* blocks, int32_t* n_blocks, int max_blocks,
                           int32_t* err_word, hipStream_t stream);

int64_t moe_ffn_workspace_elems_impl(int max_blocks);

hipError_t moe_launch_plan_blocks(const int32_t* counts, int begin, int stride, int E_loc, int P,
                                  int beta, int s, int32_t* q, int32_t* moves, int32_t* n_moves,
                                  int max_moves, int32_t* blocks, int32_t* n_blocks,
                                  int max_blocks, int32_t* err_word, hipStream_t stream);
hipError_t moe_launch_ffn_schedule(const int32_t* blocks, const int32_t* n_blocks, int max_blocks,
                                   int E_loc, int64_t max_rows, int32_t* ws, hipStream_t stream);

hipError_t moe_launch_ffn_fc1(const void* a, const void* w1, moe_dtype_t dt, int H, int I,
                              int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                              int max_blocks, int32_t* ws, void* act, int64_t max_rows,
                              int64_t a_rows, const int32_t* gather, hipStream_t stream);

hipError_t moe_launch_ffn_fc2(const void* act, const void* w2, moe_dtype_t dt, int H, int I,
                              int E_loc, const int32_t* blocks, const int32_t* n_blocks,
                              int max_blocks, int32_t* ws, void* yp, int64_t max_rows,
                              hipStream_t stream, const int32_t* dir = nullptr,
                              void* out = nullptr, int T = 0);

hipError_t moe_launch_ffn_mx_fc1(const uint8_t* xq, const uint8_t* xs, const int32_t* gather,
                                 int64_t x_rows, const uint8_t* w1q, const uint8_t* w1s, int H,
                                 int I,
                                 int max_blocks, int32_t* ws, uint8_t* actq, uint8_t* acts,
                                 hipStream_t stream);
hipError_t moe_launch_ffn_mx_fc2(const uint8_t* actq, const uint8_t* acts, const uint8_t* w2q,
                                 const uint8_t* w2s, int H, int I, int max_blocks, int32_t* ws,
                                 uint16_t* yp, int64_t max_rows, hipStream_t stream,
                                 const int32_t* dir = nullptr, void* out = nullptr, int T = 0);
inline int64_t moe_mx_scale_pitch_impl(int64_t cols) { return (cols / 32 + 3) / 4 * 4; }
hipError_t moe_launch_mx_quantize(const void* src, moe_dtype_t dt, int64_t rows, int64_t cols,
                                  int fmt, uint8_t* codes, uint8_t* scales, hipStream_t stream);
// skip_one: leave out the tokens with exactly one local entry (moe_combine_multi)
hipError_t moe_launch_combine(const void* yp, moe_dtype_t dt, const float* w,
                              const int32_t* entry_pos, int T, int H, int K, void* out,
                              hipStream_t stream, bool skip_one = false);
// dir[p] / dir[max_rows + p] for p < max_rows (moe_expert_ffn_fc2_direct)
hipError_t moe_launch_direct_rows(const int32_t* row_token, const int32_t* entry_pos,
                                  const float* w, int T, int K, int64_t max_rows, int32_t* dir,
                                  hipStream_t stream);
