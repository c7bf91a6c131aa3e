// Internal launchers behind the C ABI (moe_api.hip validates arguments, then calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Token block used by the permutation's per-block histograms (a function of T only).
int permute_token_block(int T);
int64_t permute_num_blocks(int T);

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t st);

hipError_t launch_route(const moe_shape_t& s, const uint16_t* x, const float* wg,
                        const float* logit_bias, const float* sel_bias, float* logits,
                        float* probs, int32_t* topk_idx, float* topk_w, int32_t* counts,
                        hipStream_t st);

hipError_t launch_permute(const moe_shape_t& s, int64_t mcap, const int32_t* topk_idx,
                          const uint16_t* x, int32_t* seg_offsets, int32_t* tile_group,
                          int32_t* total_rows, int32_t* row_token, int32_t* pos, uint16_t* x_perm,
                          int32_t* ws, hipStream_t st);

// x_perm[r] = x[row_token[r]] (zero where row_token[r] < 0) for r < min(mcap, total_rows[0]).
hipError_t launch_gather_rows(const moe_shape_t& s, int64_t mcap, const int32_t* total_rows,
                              const int32_t* row_token, const uint16_t* x, uint16_t* x_perm,
                              hipStream_t st);

// x_perm: the permuted rows [Mcap,H], or (row_token != NULL) the token rows x[T,H], which the
// gate/up product then reads through row_token (T*H*2 must not exceed 2^31 bytes); in that case
// x_perm_out (may be NULL) receives the permuted rows too.
hipError_t launch_ggemm_fwd(const moe_shape_t& s, uint32_t which, int64_t mcap, const uint16_t* x_perm,
                            const int32_t* row_token, const int32_t* seg_offsets,
                            const int32_t* tile_group, const int32_t* total_rows,
                            const uint16_t* w1, const uint16_t* w2, uint16_t* h_save, uint16_t* a,
                            uint16_t* y_perm, uint16_t* x_perm_out, hipStream_t st);

hipError_t launch_ggemm_dgrad(const moe_shape_t& s, uint32_t which, int64_t mcap, const uint16_t* dy_perm,
                              const uint16_t* h_save, const int32_t* seg_offsets,
                              const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* dh, uint16_t* dx_perm, hipStream_t st);

// dW1/dW2 are bf16 (f32 == false) or fp32 (f32 == true) arrays of the same shapes.
hipError_t launch_ggemm_wgrad(const moe_shape_t& s, uint32_t which, const uint16_t* x_perm, const uint16_t* a,
                              const uint16_t* dy_perm, const uint16_t* dh,
                              const int32_t* seg_offsets, void* dw1, void* dw2, bool f32,
                              hipStream_t st);

hipError_t launch_combine(const moe_shape_t& s, const uint16_t* y_perm, const int32_t* pos,
                          const float* topk_w, const int32_t* seg_offsets, uint16_t* y,
                          hipStream_t st);

hipError_t launch_combine_bwd(const moe_shape_t& s, int64_t mcap, const uint16_t* dy,
                              const uint16_t* y_perm, const int32_t* pos, const float* topk_w,
                              const int32_t* seg_offsets, const int32_t* row_token,
                              const int32_t* total_rows, uint16_t* dy_perm, float* dtopk_w,
                              hipStream_t st);

hipError_t launch_unpermute_bwd(const moe_shape_t& s, const uint16_t* dx_perm, const int32_t* pos,
                                const int32_t* seg_offsets, uint16_t* dx, hipStream_t st);

hipError_t launch_route_bwd(const moe_shape_t& s, const float* dtopk_w, const int32_t* topk_idx,
                            const float* probs, const uint16_t* x, const float* wg, float* dlogits,
                            float* dw_gate, float* dx_router, hipStream_t st);

hipError_t launch_router_grads(const moe_shape_t& s, const float* dlogits, const uint16_t* x,
                               const float* wg, float* dw_gate, float* dx_router, hipStream_t st);

// 4-byte words of scratch moe_balance_loss needs (per 256-token chunk of each sequence: a partial
// loss and E selection counts)
int64_t balance_workspace_floats(int T, int seq_len, int E);

hipError_t launch_balance_loss(const moe_shape_t& s, int seq_len, float alpha, const float* probs,
                               const int32_t* topk_idx, float* seq_loss, float* dlogits, float* ws,
                               hipStream_t st);

hipError_t launch_bias_update(const moe_shape_t& s, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st);

}  // namespace moe
