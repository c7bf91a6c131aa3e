/*
 * moe.h — C ABI of the MI355X (gfx950) MoE feed-forward hot path of dots.llm1.
 *
 * What the calls compute comes from the dots.llm1 Technical Report notes page (papercache.org),
 * cited below as TR:
 *   - TR section A2 "Architecture", mixture-of-experts paragraph: routed experts chosen top-k per
 *     token plus shared experts active for every token; each expert a two-layer FFN with SwiGLU;
 *     the gating layer computed in FP32.
 *   - TR section A2, load-balancing paragraph: a per-expert bias added to the affinity scores
 *     decides the top-k routing only; no token is dropped.
 *   - TR section 3.2 "Efficient grouped GEMM": every expert's token segment is padded to a fixed
 *     block size that is a multiple of the matrix instruction's M, so a workgroup's rows always
 *     belong to one expert and the grouped GEMM schedules like an ordinary GEMM.
 *   - TR section 6 "MoE analysis": the per-expert token count behind the expert load.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE memory owned by the caller; the library never allocates, frees
 *     or keeps state between calls, so calls are reentrant. Everything is row-major, contiguous.
 *   - bf16 tensors are passed as uint16_t bit patterns. fp32 tensors as float.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream) and never
 *     synchronises the host. Data-dependent sizes (total_rows, tile_group) stay on the device.
 *   - Arguments are checked on the host before any launch: MOE_ERR_INVALID_ARG for a NULL
 *     required pointer, a bf16 activation or weight tensor that is not 16-byte aligned (every
 *     kernel moves them in 16-byte chunks), or an impossible shape, MOE_ERR_UNSUPPORTED for
 *     shapes the kernels are not built for, MOE_ERR_WORKSPACE if ws_bytes is too small.
 *   - T == 0 (an empty batch) reads nothing: moe_route writes expert_counts = 0 (if given),
 *     moe_permute writes seg_offsets = 0 and total_rows = 0, grouped_gemm_bwd with a WGRAD bit
 *     writes zero weight gradients, every other call is a no-op returning MOE_OK; pointers to
 *     T- or Mcap-sized arrays may then be NULL.
 *     A failed launch returns MOE_ERR_HIP; moe_last_error() then describes it.
 *   - Notation: T tokens, H hidden, E routed experts, K experts per token, I expert intermediate
 *     size, S shared experts, G = E + S groups (shared groups last), B = block_m, R = T*K and
 *     Mcap = moe_row_capacity(shape) rows for every permuted buffer.
 *   - Supported: 1 <= K <= E, E <= 256, K <= 8, S <= 4, H % 128 == 0, I % 64 == 0,
 *     block_m in {16, 32, 64, 128, 256}.
 *   - 32-bit spans: the GEMM kernels address each operand block with 32-bit byte offsets, so the
 *     grouped_gemm_* calls return MOE_ERR_UNSUPPORTED (before any launch) unless
 *       4*I*H < 2^32                       (one expert's W1, 2I x H bf16),
 *       768*max(H, 2I) < 2^32              (a 384-row tile of the widest bf16 operand),
 *     and, for the weight gradients (grouped_gemm_bwd with a WGRAD bit, grouped_gemm_wgrad_f32),
 *       ceil(T/B)*B * 2*max(H, 2I) < 2^32  (the longest segment of the widest operand),
 *       2I*H*e <= 2^31                     (one expert's dW1, e = 2 bytes bf16, 4 fp32).
 *     grouped_gemm_fwd_gather also needs T*H*2 <= 2^31 (the rows of x it gathers from).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,
  MOE_ERR_UNSUPPORTED = -2,
  MOE_ERR_WORKSPACE = -3,
  MOE_ERR_HIP = -4
} moe_status_t;

/* Problem shape. flags: MOE_NORM_TOPK renormalises the K selected affinities so the routed
 * weights sum to 1 (otherwise w = p); MOE_PROBS_IN makes moe_route take probs as its input. */
typedef struct {
  int32_t T, H, E, K, I, S, block_m;
  uint32_t flags;
} moe_shape_t;

#define MOE_NORM_TOPK 0x1u
#define MOE_PROBS_IN 0x2u

/* grouped_gemm_fwd `which` bits: each selects one kernel launch */
#define MOE_FWD_GATEUP 0x1u /* h = x_perm W1^T with the SwiGLU epilogue -> a (, h_save) */
#define MOE_FWD_DOWN 0x2u   /* y_perm = a W2^T */
#define MOE_FWD (MOE_FWD_GATEUP | MOE_FWD_DOWN)

/* grouped_gemm_bwd `which` bits: each selects one kernel launch */
#define MOE_DGRAD_DOWN 0x1u   /* da = dy_perm W2, SwiGLU backward epilogue -> dh */
#define MOE_DGRAD_GATEUP 0x2u /* dx_perm = dh W1 */
#define MOE_WGRAD_DOWN 0x4u   /* dW2 = dy_perm^T a per segment */
#define MOE_WGRAD_GATEUP 0x8u /* dW1 = dh^T x_perm per segment */
#define MOE_DGRAD (MOE_DGRAD_DOWN | MOE_DGRAD_GATEUP)
#define MOE_WGRAD (MOE_WGRAD_DOWN | MOE_WGRAD_GATEUP)

/* Version of this ABI (monotonic integer). */
int32_t moe_abi_version(void);

/* Static text for a status code. */
const char* moe_status_string(int32_t status);

/* Text of the last MOE_ERR_HIP / validation failure on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Mcap: rows reserved for x_perm, a, h_save, y_perm, dy_perm, dh, dx_perm and row_token.
 * B * (min(R, floor((R + E*(B-1))/B)) + S*ceil(T/B)); covers every routing (no token dropped,
 * TR section A2 load balancing). Returns -1 for an invalid shape. */
int64_t moe_row_capacity(const moe_shape_t* shape);

/* Bytes of scratch `ws` that moe_permute needs (per-block expert histograms). */
size_t moe_workspace_size(const moe_shape_t* shape);

/*
 * moe_route — FP32 gating and biased top-k (TR section A2, MoE and load-balancing paragraphs).
 *   logits[T,E] = fp32(x[T,H]) . w_gate[E,H]^T (+ logit_bias[E])      fp32 accumulation
 *   probs[T,E]  = softmax over the E routed experts (reading of "affinity scores")
 *   key         = probs + sel_bias (one fp32 add); topk_idx[T,K] = K largest keys, ties to the
 *                 lower expert index, NaN below every number; slots in rank order
 *   topk_w[T,K] = p_e / sum of the selected p (MOE_NORM_TOPK) or p_e: the bias never enters it
 *   expert_counts[E] = tokens routed to each expert (TR section 6)
 * Modes: x != NULL computes logits into `logits` (one kernel), then routes from them (a second;
 * a third counts the routed slots per expert when expert_counts is given);
 * x == NULL reads `logits` as the input; flag MOE_PROBS_IN reads `probs` as the input (x, w_gate,
 * logits unused).
 * Optional (may be NULL): logit_bias, sel_bias (= 0), probs (unless MOE_PROBS_IN), expert_counts.
 * Required: topk_idx, topk_w; logits unless MOE_PROBS_IN; with x != NULL, x and w_gate non-NULL
 * and 16-byte aligned (else MOE_ERR_INVALID_ARG).
 */
moe_status_t moe_route(const moe_shape_t* shape, const uint16_t* x, const float* w_gate,
                       const float* logit_bias, const float* sel_bias, float* logits, float* probs,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* stream);

/*
 * moe_permute — block-aligned expert segments and the token permutation (TR section 3.2).
 *   seg_offsets[G+1]: group g owns rows [seg_offsets[g], seg_offsets[g+1]), its count rounded up
 *                     to a multiple of B (routed experts 0..E-1 in index order, then the S shared
 *                     experts with T rows each). total_rows[1] = seg_offsets[G].
 *   tile_group[Mcap/B]: group of rows [i*B, i*B+B), -1 past total_rows.
 *   row_token[Mcap]:  token of each row, -1 on padding rows (rows >= total_rows are not written).
 *                     Inside a segment tokens ascend (deterministic, stable).
 *   pos[T,K]:         row of token t's slot j in its expert's segment.
 *   x_perm[Mcap,H]:   x[row_token[r]] or 0 on padding rows, r < total_rows (skipped if x == NULL;
 *                     with x given, x and x_perm must be 16-byte aligned).
 * topk_idx entries must lie in [0, E) and be distinct per token (moe_route guarantees it). Other
 * indices give unspecified outputs but no access out of bounds: an entry outside [0, E) gets
 * pos = -1, which moe_combine, moe_combine_bwd and moe_unpermute_bwd skip, and a segment row that
 * no slot claims (a repeated expert) has row_token = -1 and reads as padding.
 * ws: device scratch of at least moe_workspace_size(shape) bytes (unused when T == 0).
 */
moe_status_t moe_permute(const moe_shape_t* shape, const int32_t* topk_idx, const uint16_t* x,
                         int32_t* seg_offsets, int32_t* tile_group, int32_t* total_rows,
                         int32_t* row_token, int32_t* pos, uint16_t* x_perm, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc — moe_permute without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid it).
 * The per-token-block histograms go to a fixed 128 KiB array in the library's device memory
 * (one per GPU, held until the process ends), which covers every supported shape; a shape
 * needing more would get MOE_ERR_WORKSPACE. It calls no allocating routine. Outputs, arguments
 * and errors are moe_permute's, bit for bit. The stream must belong to the current device (else
 * MOE_ERR_INVALID_ARG); the first call on a device looks up that device's array. Every call on a
 * GPU shares its array: calls that overlap on one GPU (concurrent streams, or host threads)
 * race and must be serialised by the caller. No state carries over between calls (each fully
 * rewrites the histograms before reading them).
 */
moe_status_t moe_permute_noalloc(const moe_shape_t* shape, const int32_t* topk_idx,
                                 const uint16_t* x, int32_t* seg_offsets, int32_t* tile_group,
                                 int32_t* total_rows, int32_t* row_token, int32_t* pos,
                                 uint16_t* x_perm, void* stream);

/*
 * grouped_gemm_fwd — every group's SwiGLU FFN on its segment (TR section A2 MoE paragraph; TR
 * section 3.2 grouped GEMM). Rows r < total_rows of group g = tile_group[r/B]:
 *   MOE_FWD_GATEUP: h = x_perm[r] . w1[g]^T  (w1: [G, 2I, H]; rows 0..I-1 gate, I..2I-1 up),
 *                   fp32 accumulate; a[r] = bf16(silu(h_gate) * h_up) in the fused epilogue;
 *                   h_save[r] = bf16(h) if h_save != NULL (the backward needs it)
 *   MOE_FWD_DOWN:   y_perm[r] = bf16(a[r] . w2[g]^T)  (w2: [G, H, I])
 * `which` is a non-empty combination (MOE_FWD = both, gate/up first). Padding rows (zero inputs)
 * give zero outputs. Rows >= total_rows are neither read nor written. Pointers a stage does not
 * use may be NULL (x_perm and w1 for DOWN alone; w2 and y_perm for GATEUP alone).
 */
moe_status_t grouped_gemm_fwd(const moe_shape_t* shape, uint32_t which, const uint16_t* x_perm,
                              const int32_t* seg_offsets, const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* h_save, uint16_t* a, uint16_t* y_perm, void* stream);

/*
 * grouped_gemm_fwd_gather — grouped_gemm_fwd with the permutation's row copy left out (TR section
 * 3.2: the segments stay block-aligned; only where the rows come from changes). The gate/up
 * product reads row r of its A operand straight from the token rows: x[row_token[r]] for
 * row_token[r] >= 0 and zero on padding rows (row_token[r] == -1), so moe_permute can be called
 * with x == NULL and no x_perm buffer exists. row_token [Mcap] and the segments come from that
 * moe_permute call. Every output equals grouped_gemm_fwd's on the x_perm moe_permute would have
 * written, bit for bit (same operands, same arithmetic).
 * x_perm [Mcap,H] bf16 (optional, may be NULL; 16-byte aligned, must not overlap x): the weight
 * gradient of the gate/up projection (grouped_gemm_bwd) reads the permuted rows, so a training
 * step passes x_perm here and gets for rows r < total_rows exactly what moe_permute would have
 * written (x[row_token[r]], zero on padding rows; rows >= total_rows untouched). On tall tiles
 * (block_m a multiple of 128) the gate/up product writes it from the rows it has staged for its
 * own use, so x is read once; otherwise a separate row copy runs on the same stream.
 * x [T,H] bf16, 16-byte aligned; needs T*H*2 <= 2^31 bytes (else MOE_ERR_UNSUPPORTED).
 * Other arguments, layouts and errors as grouped_gemm_fwd; x, row_token and x_perm are unused
 * (may be NULL) for MOE_FWD_DOWN alone.
 */
moe_status_t grouped_gemm_fwd_gather(const moe_shape_t* shape, uint32_t which, const uint16_t* x,
                                     const int32_t* row_token, const int32_t* seg_offsets,
                                     const int32_t* tile_group, const int32_t* total_rows,
                                     const uint16_t* w1, const uint16_t* w2, uint16_t* h_save,
                                     uint16_t* a, uint16_t* y_perm, uint16_t* x_perm,
                                     void* stream);

/*
 * grouped_gemm_bwd — gradients of the grouped expert FFN with the routing held fixed.
 *   MOE_DGRAD_DOWN (dy_perm, h_save, w2 -> dh):
 *     da = dy_perm[r] . w2[g]  (fp32);  g_ = h_save gate, u_ = h_save up, s = sigmoid(g_)
 *     dh[r] = bf16([da*u_*s*(1 + g_*(1-s)) | da*g_*s])     (fused SwiGLU backward epilogue)
 *   MOE_DGRAD_GATEUP (dh, w1 -> dx_perm):   dx_perm[r] = bf16(dh[r] . w1[g])
 *   MOE_WGRAD_DOWN (dy_perm, a -> dw2):      dw2[g] = bf16(sum over the segment's rows of
 *                                            dy_perm[r]^T a[r])               [G, H, I]
 *   MOE_WGRAD_GATEUP (dh, x_perm -> dw1):    dw1[g] = bf16(sum over the segment's rows of
 *                                            dh[r]^T x_perm[r])               [G, 2I, H]
 * Groups with an empty segment get zero weight gradients (so T == 0 still writes dw1/dw2 = 0).
 * `which` is a non-empty combination; launches run in the order listed. Pointers a selected stage
 * does not use may be NULL. Padding rows of dy_perm must be zero (moe_combine_bwd writes them).
 */
moe_status_t grouped_gemm_bwd(const moe_shape_t* shape, uint32_t which, const uint16_t* x_perm,
                              const uint16_t* h_save, const uint16_t* a, const uint16_t* dy_perm,
                              const int32_t* seg_offsets, const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* dh, uint16_t* dx_perm, uint16_t* dw1, uint16_t* dw2,
                              void* stream);

/*
 * grouped_gemm_wgrad_f32 — the weight gradients of grouped_gemm_bwd (MOE_WGRAD_DOWN and/or
 * MOE_WGRAD_GATEUP in `which`, no other bits) with fp32 dW outputs instead of bf16: the same fp32
 * accumulation over each group's segment, stored without rounding to bf16 (for optimizers that
 * keep fp32 gradients). dw1 [G,2I,H] and dw2 [G,H,I] are fp32, 16-byte aligned; the inputs and
 * their layouts are grouped_gemm_bwd's. Empty segments give zero gradients. Errors as there.
 */
moe_status_t grouped_gemm_wgrad_f32(const moe_shape_t* shape, uint32_t which, const uint16_t* x_perm,
                                    const uint16_t* a, const uint16_t* dy_perm, const uint16_t* dh,
                                    const int32_t* seg_offsets, float* dw1, float* dw2,
                                    void* stream);

/*
 * moe_combine — weighted unpermute: y[t] = bf16( sum_j topk_w[t,j] * y_perm[pos[t,j]]
 *               + sum_s y_perm[seg_offsets[E+s] + t] ), fp32 sum in slot order, shared last
 * (shared experts weigh 1: TR section A2, always active).
 */
moe_status_t moe_combine(const moe_shape_t* shape, const uint16_t* y_perm, const int32_t* pos,
                         const float* topk_w, const int32_t* seg_offsets, uint16_t* y,
                         void* stream);

/*
 * moe_combine_bwd — backward of moe_combine for dy[T,H]:
 *   dy_perm[pos[t,j]] = bf16(topk_w[t,j] * dy[t]);  dy_perm[seg_offsets[E+s] + t] = dy[t];
 *   dy_perm = 0 on padding rows (row_token < 0, rows < total_rows);
 *   dtopk_w[t,j] = sum_h dy[t,h] * y_perm[pos[t,j],h]  (fp32)
 */
moe_status_t moe_combine_bwd(const moe_shape_t* shape, const uint16_t* dy, const uint16_t* y_perm,
                             const int32_t* pos, const float* topk_w, const int32_t* seg_offsets,
                             const int32_t* row_token, const int32_t* total_rows,
                             uint16_t* dy_perm, float* dtopk_w, void* stream);

/*
 * moe_unpermute_bwd — dx[t] = bf16( sum_j dx_perm[pos[t,j]] + sum_s dx_perm[seg_offsets[E+s]+t] )
 * (the expert path's part of the input gradient; moe_route_bwd gives the router's part).
 */
moe_status_t moe_unpermute_bwd(const moe_shape_t* shape, const uint16_t* dx_perm,
                               const int32_t* pos, const int32_t* seg_offsets, uint16_t* dx,
                               void* stream);

/*
 * moe_route_bwd — the router's backward (TR section A2, load-balancing paragraph: the bias only
 * selects; the routing weights come from the affinity scores). Given dtopk_w[T,K] = dL/dtopk_w
 * (moe_combine_bwd's output) and the forward's topk_idx and probs:
 *   MOE_NORM_TOPK: w_j = p_{e_j} / S (S summed in slot order, as moe_route does),
 *                  c = sum_j w_j dtopk_w[t,j], dlogits[t,e_j] = w_j (dtopk_w[t,j] - c), and 0 on
 *                  every unselected expert;
 *   otherwise:     c = sum_j p_{e_j} dtopk_w[t,j], dlogits[t,e] = p_e (g_e - c) with
 *                  g_{e_j} = dtopk_w[t,j] and g = 0 elsewhere.
 * The selection (piecewise constant) passes no gradient and sel_bias gets none.
 *   dw_gate[E,H]   = dlogits^T x          (fp32; optional, needs x)
 *   dx_router[T,H] = dlogits w_gate       (fp32; the router's share of the input gradient,
 *                                          to be added to moe_unpermute_bwd's; optional, needs w_gate)
 * Layouts: dtopk_w, topk_idx [T,K]; probs, dlogits [T,E] fp32; x [T,H] bf16; w_gate [E,H] fp32.
 * Required when T > 0: dtopk_w, topk_idx, probs, dlogits; x 16-byte aligned when dw_gate is
 * given (else MOE_ERR_INVALID_ARG). With T == 0 nothing is read and dw_gate
 * (if given) is filled with zeros. Logit_bias, if the forward used one, gets sum_t dlogits[t,e]; it
 * is not computed here.
 */
moe_status_t moe_route_bwd(const moe_shape_t* shape, const float* dtopk_w, const int32_t* topk_idx,
                           const float* probs, const uint16_t* x, const float* w_gate,
                           float* dlogits, float* dw_gate, float* dx_router, void* stream);

/*
 * moe_router_grads — the router's contractions from a given dlogits [T,E] fp32 (for instance
 * moe_route_bwd's plus moe_balance_loss's): dw_gate[E,H] = dlogits^T x and dx_router[T,H] =
 * dlogits w_gate, both fp32 and each optional (dw_gate needs x, 16-byte aligned; dx_router needs
 * w_gate). With T == 0 dw_gate (if given) is filled with zeros. Layouts as moe_route_bwd.
 */
moe_status_t moe_router_grads(const moe_shape_t* shape, const float* dlogits, const uint16_t* x,
                              const float* w_gate, float* dw_gate, float* dx_router, void* stream);

/*
 * moe_balance_loss — the sequence-wise balance loss (TR section A2, load-balancing paragraph names
 * it to keep any one sequence from routing very unevenly; the formula is a reading). The batch is
 * T / seq_len sequences of seq_len consecutive tokens (seq_len must divide T). In sequence q:
 *   f_e = E / (K seq_len) * #{(t, j) in q : topk_idx[t, j] = e}      (1 for every e when balanced)
 *   P_e = (1 / seq_len) * sum_{t in q} probs[t, e]
 *   seq_loss[q] = alpha * sum_e f_e P_e                               (fp32, device, [T/seq_len])
 * The batch loss is the mean of seq_loss. Its gradient with respect to the logits (through P and
 * the softmax; the counts f are piecewise constant) is ADDED to dlogits [T,E] fp32:
 *   dlogits[t, e] += p_e (g_e - sum_i p_i g_i),  g = alpha f / (seq_len * T / seq_len).
 * Either output may be NULL, not both. probs [T,E] fp32 and topk_idx [T,K] int32 are moe_route's
 * outputs; experts outside 0..E-1 in topk_idx are not counted. alpha must be finite and >= 0.
 * ws (device, caller-owned, ws_bytes >= moe_balance_workspace_size) holds per-chunk counts and
 * partial sums; the loss
 * is summed in a fixed order, so it is deterministic.
 * Errors: MOE_ERR_INVALID_ARG for a bad seq_len, alpha or pointer; MOE_ERR_WORKSPACE for a small
 * ws. T == 0 is a no-op.
 */
moe_status_t moe_balance_loss(const moe_shape_t* shape, int32_t seq_len, float alpha,
                              const float* probs, const int32_t* topk_idx, float* seq_loss,
                              float* dlogits, void* ws, size_t ws_bytes, void* stream);

/* Bytes of scratch `ws` that moe_balance_loss needs (per 256-token chunk of each sequence: a
 * partial sum of the loss and E selection counts); 0 for an invalid shape or seq_len. */
size_t moe_balance_workspace_size(const moe_shape_t* shape, int32_t seq_len);

/*
 * moe_bias_update — one step of the aux-loss-free load balancing (TR section A2, load-balancing
 * paragraph: the per-expert bias is adjusted during training to keep the loads balanced; the
 * rule is a reading): with the mean load T*K/E,
 *   sel_bias[e] += gamma  if expert_counts[e] < T*K/E,
 *   sel_bias[e] -= gamma  if expert_counts[e] > T*K/E, unchanged if equal
 * (the comparison is exact in integers; the update one fp32 add). sel_bias [E] fp32 is updated in
 * place; expert_counts [E] int32 is moe_route's output. gamma (the update speed) must be a
 * finite number >= 0, else MOE_ERR_INVALID_ARG.
 */
moe_status_t moe_bias_update(const moe_shape_t* shape, const int32_t* expert_counts, float gamma,
                             float* sel_bias, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
