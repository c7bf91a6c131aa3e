// C ABI of the MoE feed-forward path (declared in include/moe.h): host-side argument checks,
// then launches on the caller's stream. No allocation, no synchronisation, no global state.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "moe_common.h"
#include "moe_internal.h"

namespace {

thread_local char g_err[256] = "";

void set_err(const char* what) {
  snprintf(g_err, sizeof(g_err), "%s", what);
}

moe_status_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  snprintf(g_err, sizeof(g_err), "%s: %s", where, hipGetErrorString(e));
  return MOE_ERR_HIP;
}

constexpr int kMaxT = 262144;

// Shape checks shared by every entry point. Returns MOE_OK or the failure code.
moe_status_t check_shape(const moe_shape_t* s) {
  if (!s) { set_err("shape is NULL"); return MOE_ERR_INVALID_ARG; }
  if (s->T < 0 || s->H <= 0 || s->E <= 0 || s->K < 1 || s->K > s->E || s->I <= 0 || s->S < 0 ||
      s->block_m <= 0) {
    set_err("invalid shape (need T>=0, H,E,I>0, 1<=K<=E, S>=0, block_m>0)");
    return MOE_ERR_INVALID_ARG;
  }
  const int b = s->block_m;
  if (!(b == 16 || b == 32 || b == 64 || b == 128 || b == 256)) {
    set_err("block_m must be one of 16, 32, 64, 128, 256");
    return MOE_ERR_UNSUPPORTED;
  }
  if (s->H % 128 != 0 || s->I % 64 != 0) {
    set_err("need H % 128 == 0 and I % 64 == 0");
    return MOE_ERR_UNSUPPORTED;
  }
  if (s->E > 256 || s->K > 8 || s->S > 4 || s->T > kMaxT) {
    set_err("need E <= 256, K <= 8, S <= 4, T <= 262144");
    return MOE_ERR_UNSUPPORTED;
  }
  if (s->flags & ~(uint32_t)(MOE_NORM_TOPK | MOE_PROBS_IN)) {
    set_err("unknown flag bits");
    return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

// The GEMM engines address their operands through buffer resources with 32-bit byte offsets,
// and the weight-gradient stores and the gathering DMA mark masked lanes with an offset of 2^31
// past the buffer's start. These checks reject every shape whose spans would not fit:
//   - one group's expert weights, W1[g] = 2I x H bf16 (the larger of W1[g] and W2[g]);
//   - one row tile of a row-grouped product, at most 384 rows of an operand up to max(H, 2I)
//     wide;
//   - (weight gradients) one segment's rows of an operand up to max(H, 2I) wide: a segment holds
//     at most ceil(T/B)*B rows (each token picks distinct experts; shared segments hold T);
//   - (weight gradients) one group's dW, which the 2^31 marker must lie past.
constexpr int64_t kSpan32 = (int64_t)1 << 32;
constexpr int64_t kMarker = (int64_t)1 << 31;
constexpr int64_t kMaxTileRows = 384;

moe_status_t check_gemm_spans(const moe_shape_t* s) {
  const int64_t H = s->H, I = s->I, wide = H > 2 * I ? H : 2 * I;
  if (4 * I * H >= kSpan32) {
    set_err("an expert's W1 (2I x H bf16) must be smaller than 4 GiB: need I*H < 2^30");
    return MOE_ERR_UNSUPPORTED;
  }
  if (kMaxTileRows * wide * 2 >= kSpan32) {
    set_err("a 384-row tile of a max(H, 2I)-wide bf16 operand must be smaller than 4 GiB");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

moe_status_t check_wgrad_spans(const moe_shape_t* s, int64_t dw_elem_bytes) {
  const moe_status_t r = check_gemm_spans(s);
  if (r != MOE_OK) return r;
  const int64_t H = s->H, I = s->I, wide = H > 2 * I ? H : 2 * I, B = s->block_m;
  const int64_t seg_rows = ((int64_t)s->T + B - 1) / B * B;
  if (seg_rows * wide * 2 >= kSpan32) {
    set_err("weight gradients: a segment of ceil(T/B)*B rows of a max(H, 2I)-wide bf16 operand "
            "must be smaller than 4 GiB");
    return MOE_ERR_UNSUPPORTED;
  }
  if (2 * I * H * dw_elem_bytes > kMarker) {
    set_err("weight gradients: one expert's dW1 (2I x H) must fit in 2^31 bytes");
    return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int64_t capacity(const moe_shape_t* s) {
  const int64_t T = s->T, B = s->block_m;
  const int64_t R = T * s->K;
  int64_t routed = (R + (int64_t)s->E * (B - 1)) / B;
  if (routed > R) routed = R;
  return B * (routed + (int64_t)s->S * ((T + B - 1) / B));
}

#define REQUIRE(p)                                                \
  do {                                                            \
    if (!(p)) {                                                   \
      set_err("required pointer is NULL: " #p);                   \
      return MOE_ERR_INVALID_ARG;                                 \
    }                                                             \
  } while (0)

// A bf16 activation or weight tensor: non-NULL and 16-byte aligned (every kernel that reads or
// writes one moves 16-byte chunks).
#define REQUIRE_T(p)                                                   \
  do {                                                                 \
    REQUIRE(p);                                                        \
    if ((uintptr_t)(p) % 16 != 0) {                                    \
      set_err("tensor pointer is not 16-byte aligned: " #p);           \
      return MOE_ERR_INVALID_ARG;                                      \
    }                                                                  \
  } while (0)

#define CHECK_SHAPE(s)                       \
  do {                                       \
    moe_status_t st_ = check_shape(s);       \
    if (st_ != MOE_OK) return st_;           \
    g_err[0] = 0;                            \
  } while (0)

// moe_permute with T == 0: still define the (empty) segments, so later calls see G+1 zero offsets
// and no rows.
moe_status_t permute_empty(const moe_shape_t* s, int32_t* seg_offsets, int32_t* total_rows,
                           void* stream) {
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = moe::launch_fill_i32(seg_offsets, 0, s->E + s->S + 1, st);
  if (e == hipSuccess) e = moe::launch_fill_i32(total_rows, 0, 1, st);
  return hip_status(e, "moe_permute");
}

// moe_permute's pointer checks for T > 0 (the workspace aside).
moe_status_t check_permute_args(const moe_shape_t* s, const int32_t* topk_idx, const uint16_t* x,
                                int32_t* tile_group, int32_t* row_token, int32_t* pos,
                                uint16_t* x_perm) {
  (void)s;
  REQUIRE(topk_idx);
  REQUIRE(tile_group);
  REQUIRE(row_token);
  REQUIRE(pos);
  if (x) {
    REQUIRE_T(x);
    REQUIRE_T(x_perm);
  }
  return MOE_OK;
}

// Fixed device scratch of moe_permute_noalloc: the permutation's per-token-block expert
// histograms, at most 128 token blocks x 256 experts int32 (128 KiB) for every shape that
// check_shape accepts. Each GPU the library runs on holds its own copy until the process ends.
// Host code never uses the array's name as an address (on the host it is only a stand-in for the
// symbol): the device address comes from hipGetSymbolAddress, once per device, with that device
// current.
constexpr size_t kScratchBytes = (size_t)128 * 256 * sizeof(int32_t);
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (which must be the current one).
moe_status_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc(hipGetDevice)");
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc(hipStreamGetDevice)");
    if (sdev != dev) {
      snprintf(g_err, sizeof(g_err),
               "moe_permute_noalloc: the stream belongs to device %d but device %d is current",
               (int)sdev, dev);
      return MOE_ERR_INVALID_ARG;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_err("moe_permute_noalloc: device index beyond the library's table of 64");
    return MOE_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "moe_permute_noalloc(hipGetSymbolAddress)");
    if (!ptr) {
      set_err("moe_permute_noalloc: hipGetSymbolAddress returned NULL");
      return MOE_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 4; }

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_row_capacity(const moe_shape_t* s) {
  if (check_shape(s) != MOE_OK) return -1;
  return capacity(s);
}

size_t moe_workspace_size(const moe_shape_t* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return sizeof(int32_t) * (size_t)moe::permute_num_blocks(s->T) * (size_t)s->E;
}

moe_status_t moe_route(const moe_shape_t* s, const uint16_t* x, const float* w_gate,
                       const float* logit_bias, const float* sel_bias, float* logits, float* probs,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* stream) {
  CHECK_SHAPE(s);
  if (s->T == 0) {
    // no token routed: every expert's count is zero
    if (!expert_counts) return MOE_OK;
    return hip_status(moe::launch_fill_i32(expert_counts, 0, s->E, (hipStream_t)stream),
                      "moe_route");
  }
  REQUIRE(topk_idx);
  REQUIRE(topk_w);
  if (s->flags & MOE_PROBS_IN) {
    REQUIRE(probs);
  } else if (x) {
    REQUIRE_T(x);
    REQUIRE_T(w_gate);
    REQUIRE(logits);
  } else {
    REQUIRE(logits);
  }
  return hip_status(moe::launch_route(*s, x, w_gate, logit_bias, sel_bias, logits, probs, topk_idx,
                                      topk_w, expert_counts, (hipStream_t)stream),
                    "moe_route");
}

moe_status_t moe_permute(const moe_shape_t* s, const int32_t* topk_idx, const uint16_t* x,
                         int32_t* seg_offsets, int32_t* tile_group, int32_t* total_rows,
                         int32_t* row_token, int32_t* pos, uint16_t* x_perm, void* ws,
                         size_t ws_bytes, void* stream) {
  CHECK_SHAPE(s);
  REQUIRE(seg_offsets);
  REQUIRE(total_rows);
  if (s->T == 0) return permute_empty(s, seg_offsets, total_rows, stream);
  {
    const moe_status_t r = check_permute_args(s, topk_idx, x, tile_group, row_token, pos, x_perm);
    if (r != MOE_OK) return r;
  }
  REQUIRE(ws);
  if (ws_bytes < moe_workspace_size(s)) {
    set_err("workspace smaller than moe_workspace_size()");
    return MOE_ERR_WORKSPACE;
  }
  return hip_status(moe::launch_permute(*s, capacity(s), topk_idx, x, seg_offsets, tile_group,
                                        total_rows, row_token, pos, x_perm, (int32_t*)ws,
                                        (hipStream_t)stream),
                    "moe_permute");
}

moe_status_t moe_permute_noalloc(const moe_shape_t* s, const int32_t* topk_idx, const uint16_t* x,
                                 int32_t* seg_offsets, int32_t* tile_group, int32_t* total_rows,
                                 int32_t* row_token, int32_t* pos, uint16_t* x_perm, void* stream) {
  CHECK_SHAPE(s);
  REQUIRE(seg_offsets);
  REQUIRE(total_rows);
  if (s->T == 0) return permute_empty(s, seg_offsets, total_rows, stream);
  {
    const moe_status_t r = check_permute_args(s, topk_idx, x, tile_group, row_token, pos, x_perm);
    if (r != MOE_OK) return r;
  }
  if (moe_workspace_size(s) > kScratchBytes) {
    set_err("moe_permute_noalloc: the shape needs more than the 128 KiB of fixed scratch");
    return MOE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  {
    const moe_status_t r = device_scratch((hipStream_t)stream, &ws);
    if (r != MOE_OK) return r;
  }
  return hip_status(moe::launch_permute(*s, capacity(s), topk_idx, x, seg_offsets, tile_group,
                                        total_rows, row_token, pos, x_perm, (int32_t*)ws,
                                        (hipStream_t)stream),
                    "moe_permute_noalloc");
}

moe_status_t grouped_gemm_fwd(const moe_shape_t* s, uint32_t which, const uint16_t* x_perm,
                              const int32_t* seg_offsets, const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* h_save, uint16_t* a, uint16_t* y_perm, void* stream) {
  CHECK_SHAPE(s);
  if (which == 0 || (which & ~(uint32_t)MOE_FWD)) {
    set_err("which must be a non-empty combination of MOE_FWD_GATEUP and MOE_FWD_DOWN");
    return MOE_ERR_INVALID_ARG;
  }
  {
    const moe_status_t r = check_gemm_spans(s);
    if (r != MOE_OK) return r;
  }
  if (s->T == 0) return MOE_OK;
  REQUIRE(seg_offsets);
  REQUIRE(tile_group);
  REQUIRE(total_rows);
  REQUIRE_T(a);
  if (h_save) REQUIRE_T(h_save);
  if (which & MOE_FWD_GATEUP) {
    REQUIRE_T(x_perm);
    REQUIRE_T(w1);
  }
  if (which & MOE_FWD_DOWN) {
    REQUIRE_T(w2);
    REQUIRE_T(y_perm);
  }
  return hip_status(moe::launch_ggemm_fwd(*s, which, capacity(s), x_perm, nullptr, seg_offsets,
                                          tile_group, total_rows, w1, w2, h_save, a, y_perm,
                                          nullptr, (hipStream_t)stream),
                    "grouped_gemm_fwd");
}

moe_status_t grouped_gemm_fwd_gather(const moe_shape_t* s, uint32_t which, const uint16_t* x,
                                     const int32_t* row_token, const int32_t* seg_offsets,
                                     const int32_t* tile_group, const int32_t* total_rows,
                                     const uint16_t* w1, const uint16_t* w2, uint16_t* h_save,
                                     uint16_t* a, uint16_t* y_perm, uint16_t* x_perm,
                                     void* stream) {
  CHECK_SHAPE(s);
  if (which == 0 || (which & ~(uint32_t)MOE_FWD)) {
    set_err("which must be a non-empty combination of MOE_FWD_GATEUP and MOE_FWD_DOWN");
    return MOE_ERR_INVALID_ARG;
  }
  // the gathering DMA addresses x with 32-bit byte offsets and a past-the-end marker at 2^31
  if ((int64_t)s->T * s->H * 2 > kMarker) {
    set_err("grouped_gemm_fwd_gather needs T*H*2 <= 2^31 bytes; use moe_permute + grouped_gemm_fwd");
    return MOE_ERR_UNSUPPORTED;
  }
  {
    const moe_status_t r = check_gemm_spans(s);
    if (r != MOE_OK) return r;
  }
  if (s->T == 0) return MOE_OK;
  REQUIRE(seg_offsets);
  REQUIRE(tile_group);
  REQUIRE(total_rows);
  REQUIRE_T(a);
  if (h_save) REQUIRE_T(h_save);
  if (which & MOE_FWD_GATEUP) {
    REQUIRE_T(x);
    REQUIRE(row_token);
    REQUIRE_T(w1);
    if (x_perm) {
      REQUIRE_T(x_perm);
      const uintptr_t x0 = (uintptr_t)x, x1 = x0 + (uintptr_t)s->T * s->H * 2;
      const uintptr_t p0 = (uintptr_t)x_perm, p1 = p0 + (uintptr_t)capacity(s) * s->H * 2;
      if (p0 < x1 && x0 < p1) {
        set_err("x_perm overlaps x");
        return MOE_ERR_INVALID_ARG;
      }
    }
  }
  if (which & MOE_FWD_DOWN) {
    REQUIRE_T(w2);
    REQUIRE_T(y_perm);
  }
  return hip_status(moe::launch_ggemm_fwd(*s, which, capacity(s), x,
                                          (which & MOE_FWD_GATEUP) ? row_token : nullptr,
                                          seg_offsets, tile_group, total_rows, w1, w2, h_save, a,
                                          y_perm, (which & MOE_FWD_GATEUP) ? x_perm : nullptr,
                                          (hipStream_t)stream),
                    "grouped_gemm_fwd_gather");
}

moe_status_t grouped_gemm_bwd(const moe_shape_t* s, uint32_t which, const uint16_t* x_perm,
                              const uint16_t* h_save, const uint16_t* a, const uint16_t* dy_perm,
                              const int32_t* seg_offsets, const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* dh, uint16_t* dx_perm, uint16_t* dw1, uint16_t* dw2,
                              void* stream) {
  CHECK_SHAPE(s);
  if (which == 0 || (which & ~(uint32_t)(MOE_DGRAD | MOE_WGRAD))) {
    set_err("which must be a non-empty combination of the MOE_DGRAD_* and MOE_WGRAD_* bits");
    return MOE_ERR_INVALID_ARG;
  }
  {
    const moe_status_t r = (which & MOE_WGRAD) ? check_wgrad_spans(s, 2) : check_gemm_spans(s);
    if (r != MOE_OK) return r;
  }
  const bool rows = s->T > 0;  // with T == 0 no activation row is read and dgrad is a no-op
  if (rows && (which & MOE_DGRAD)) {
    REQUIRE(seg_offsets);
    REQUIRE(tile_group);
    REQUIRE(total_rows);
    REQUIRE_T(dh);
  }
  if (rows && (which & MOE_DGRAD_DOWN)) {
    REQUIRE_T(dy_perm);
    REQUIRE_T(h_save);
    REQUIRE_T(w2);
  }
  if (rows && (which & MOE_DGRAD_GATEUP)) {
    REQUIRE_T(w1);
    REQUIRE_T(dx_perm);
  }
  if (which & MOE_WGRAD) REQUIRE(seg_offsets);
  if (which & MOE_WGRAD_DOWN) {
    REQUIRE_T(dw2);
    if (rows) {
      REQUIRE_T(dy_perm);
      REQUIRE_T(a);
    }
  }
  if (which & MOE_WGRAD_GATEUP) {
    REQUIRE_T(dw1);
    if (rows) {
      REQUIRE_T(dh);
      REQUIRE_T(x_perm);
    }
  }
  hipStream_t st = (hipStream_t)stream;
  if (rows && (which & MOE_DGRAD)) {
    moe_status_t r = hip_status(moe::launch_ggemm_dgrad(*s, which, capacity(s), dy_perm, h_save,
                                                        seg_offsets, tile_group, total_rows, w1, w2, dh,
                                                        dx_perm, st),
                                "grouped_gemm_bwd(dgrad)");
    if (r != MOE_OK) return r;
  }
  if (which & MOE_WGRAD) {
    return hip_status(moe::launch_ggemm_wgrad(*s, which, x_perm, a, dy_perm, dh, seg_offsets, dw1,
                                              dw2, false, st),
                      "grouped_gemm_bwd(wgrad)");
  }
  return MOE_OK;
}

moe_status_t grouped_gemm_wgrad_f32(const moe_shape_t* s, uint32_t which, const uint16_t* x_perm,
                                    const uint16_t* a, const uint16_t* dy_perm, const uint16_t* dh,
                                    const int32_t* seg_offsets, float* dw1, float* dw2,
                                    void* stream) {
  CHECK_SHAPE(s);
  if (which == 0 || (which & ~(uint32_t)MOE_WGRAD)) {
    set_err("which must be a non-empty combination of the MOE_WGRAD_* bits");
    return MOE_ERR_INVALID_ARG;
  }
  {
    const moe_status_t r = check_wgrad_spans(s, 4);
    if (r != MOE_OK) return r;
  }
  const bool rows = s->T > 0;
  REQUIRE(seg_offsets);
  if (which & MOE_WGRAD_DOWN) {
    REQUIRE_T(dw2);
    if (rows) {
      REQUIRE_T(dy_perm);
      REQUIRE_T(a);
    }
  }
  if (which & MOE_WGRAD_GATEUP) {
    REQUIRE_T(dw1);
    if (rows) {
      REQUIRE_T(dh);
      REQUIRE_T(x_perm);
    }
  }
  return hip_status(moe::launch_ggemm_wgrad(*s, which, x_perm, a, dy_perm, dh, seg_offsets, dw1, dw2,
                                            true, (hipStream_t)stream),
                    "grouped_gemm_wgrad_f32");
}

moe_status_t moe_combine(const moe_shape_t* s, const uint16_t* y_perm, const int32_t* pos,
                         const float* topk_w, const int32_t* seg_offsets, uint16_t* y,
                         void* stream) {
  CHECK_SHAPE(s);
  if (s->T == 0) return MOE_OK;
  REQUIRE_T(y_perm);
  REQUIRE(pos);
  REQUIRE(topk_w);
  REQUIRE(seg_offsets);
  REQUIRE_T(y);
  return hip_status(moe::launch_combine(*s, y_perm, pos, topk_w, seg_offsets, y,
                                        (hipStream_t)stream),
                    "moe_combine");
}

moe_status_t moe_combine_bwd(const moe_shape_t* s, const uint16_t* dy, const uint16_t* y_perm,
                             const int32_t* pos, const float* topk_w, const int32_t* seg_offsets,
                             const int32_t* row_token, const int32_t* total_rows,
                             uint16_t* dy_perm, float* dtopk_w, void* stream) {
  CHECK_SHAPE(s);
  if (s->T == 0) return MOE_OK;
  REQUIRE_T(dy);
  REQUIRE_T(y_perm);
  REQUIRE(pos);
  REQUIRE(topk_w);
  REQUIRE(seg_offsets);
  REQUIRE(row_token);
  REQUIRE(total_rows);
  REQUIRE_T(dy_perm);
  REQUIRE(dtopk_w);
  return hip_status(moe::launch_combine_bwd(*s, capacity(s), dy, y_perm, pos, topk_w, seg_offsets,
                                            row_token, total_rows, dy_perm, dtopk_w,
                                            (hipStream_t)stream),
                    "moe_combine_bwd");
}

moe_status_t moe_unpermute_bwd(const moe_shape_t* s, const uint16_t* dx_perm, const int32_t* pos,
                               const int32_t* seg_offsets, uint16_t* dx, void* stream) {
  CHECK_SHAPE(s);
  if (s->T == 0) return MOE_OK;
  REQUIRE_T(dx_perm);
  REQUIRE(pos);
  REQUIRE(seg_offsets);
  REQUIRE_T(dx);
  return hip_status(moe::launch_unpermute_bwd(*s, dx_perm, pos, seg_offsets, dx,
                                              (hipStream_t)stream),
                    "moe_unpermute_bwd");
}

moe_status_t moe_route_bwd(const moe_shape_t* s, const float* dtopk_w, const int32_t* topk_idx,
                           const float* probs, const uint16_t* x, const float* w_gate,
                           float* dlogits, float* dw_gate, float* dx_router, void* stream) {
  CHECK_SHAPE(s);
  if (s->T > 0) {
    REQUIRE(dtopk_w);
    REQUIRE(topk_idx);
    REQUIRE(probs);
    REQUIRE(dlogits);
    if (dw_gate) REQUIRE_T(x);
    if (dx_router) REQUIRE(w_gate);
  }
  if (s->T == 0 && !dw_gate) return MOE_OK;
  return hip_status(moe::launch_route_bwd(*s, dtopk_w, topk_idx, probs, x, w_gate, dlogits, dw_gate,
                                          dx_router, (hipStream_t)stream),
                    "moe_route_bwd");
}

moe_status_t moe_router_grads(const moe_shape_t* s, const float* dlogits, const uint16_t* x,
                              const float* w_gate, float* dw_gate, float* dx_router, void* stream) {
  CHECK_SHAPE(s);
  if (s->T > 0) {
    REQUIRE(dlogits);
    if (dw_gate) REQUIRE_T(x);
    if (dx_router) REQUIRE(w_gate);
  }
  return hip_status(moe::launch_router_grads(*s, dlogits, x, w_gate, dw_gate, dx_router,
                                             (hipStream_t)stream),
                    "moe_router_grads");
}

size_t moe_balance_workspace_size(const moe_shape_t* s, int32_t seq_len) {
  if (check_shape(s) != MOE_OK || seq_len < 1 || s->T % seq_len != 0) return 0;
  return sizeof(float) * (size_t)moe::balance_workspace_floats(s->T, seq_len, s->E);
}

moe_status_t moe_balance_loss(const moe_shape_t* s, int32_t seq_len, float alpha, const float* probs,
                              const int32_t* topk_idx, float* seq_loss, float* dlogits, void* ws,
                              size_t ws_bytes, void* stream) {
  CHECK_SHAPE(s);
  if (seq_len < 1 || s->T % seq_len != 0) {
    set_err("seq_len must be >= 1 and divide T");
    return MOE_ERR_INVALID_ARG;
  }
  if (!(alpha >= 0.0f) || alpha > 3.0e38f) {
    set_err("alpha must be a finite number >= 0");
    return MOE_ERR_INVALID_ARG;
  }
  if (!seq_loss && !dlogits) {
    set_err("nothing to compute: seq_loss and dlogits are both NULL");
    return MOE_ERR_INVALID_ARG;
  }
  if (s->T == 0) return MOE_OK;
  REQUIRE(probs);
  REQUIRE(topk_idx);
  REQUIRE(ws);
  if (ws_bytes < sizeof(float) * (size_t)moe::balance_workspace_floats(s->T, seq_len, s->E)) {
    set_err("workspace smaller than moe_balance_workspace_size()");
    return MOE_ERR_WORKSPACE;
  }
  return hip_status(moe::launch_balance_loss(*s, seq_len, alpha, probs, topk_idx, seq_loss, dlogits,
                                             static_cast<float*>(ws), (hipStream_t)stream),
                    "moe_balance_loss");
}

moe_status_t moe_bias_update(const moe_shape_t* s, const int32_t* expert_counts, float gamma,
                             float* sel_bias, void* stream) {
  CHECK_SHAPE(s);
  REQUIRE(expert_counts);
  REQUIRE(sel_bias);
  if (!(gamma >= 0.0f) || gamma > 3.0e38f) {
    set_err("gamma must be a finite number >= 0");
    return MOE_ERR_INVALID_ARG;
  }
  return hip_status(moe::launch_bias_update(*s, expert_counts, gamma, sel_bias,
                                            (hipStream_t)stream),
                    "moe_bias_update");
}

}  // extern "C"
