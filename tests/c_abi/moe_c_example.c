/*
 * A plain C caller of libmoe (include/moe.h): no Python, no torch, only the HIP runtime's C API
 * for device memory. It runs one forward + backward step of a MoE layer through the C entry points
 * and writes the results to a file, which the GPU tests compare with the CPU oracle.
 *
 *   moe_c_example <in.bin> <out.bin>
 *
 * in.bin (little endian): int32 T, H, E, K, I, S, block_m, flags; then bf16 x[T,H]; fp32 w_gate[E,H];
 * fp32 sel_bias[E]; bf16 w1[G,2I,H]; bf16 w2[G,H,I]; bf16 dy[T,H]   (G = E + S).
 * out.bin: int32 topk_idx[T,K]; fp32 topk_w[T,K]; bf16 y[T,H]; fp32 dtopk_w[T,K]; bf16 dx[T,H];
 * bf16 dw1[G,2I,H]; bf16 dw2[G,H,I].
 * Exit status 0 on success; on any failure the failing call and its message go to stderr.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));            \
      exit(1);                                                                     \
    }                                                                              \
  } while (0)

#define MOE_OK_(call)                                                              \
  do {                                                                             \
    moe_status_t s_ = (call);                                                      \
    if (s_ != MOE_OK) {                                                            \
      fprintf(stderr, "%s failed: %s (%s)\n", #call, moe_status_string(s_),        \
              moe_last_error());                                                   \
      exit(1);                                                                     \
    }                                                                              \
  } while (0)

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes > 0 ? bytes : 16));
  return p;
}

/* Read n bytes from f into a new device buffer. */
static void* dev_from_file(FILE* f, size_t bytes) {
  void* h = malloc(bytes > 0 ? bytes : 1);
  if (!h || fread(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(1);
  }
  void* d = dev_alloc(bytes);
  HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return d;
}

static void dev_to_file(FILE* f, const void* d, size_t bytes) {
  void* h = malloc(bytes > 0 ? bytes : 1);
  if (!h) exit(1);
  HIP_OK(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost));
  if (fwrite(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "write failed\n");
    exit(1);
  }
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[8];
  if (fread(hdr, sizeof(int32_t), 8, in) != 8) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  moe_shape_t s;
  s.T = hdr[0]; s.H = hdr[1]; s.E = hdr[2]; s.K = hdr[3]; s.I = hdr[4]; s.S = hdr[5];
  s.block_m = hdr[6]; s.flags = (uint32_t)hdr[7];
  const int64_t mcap = moe_row_capacity(&s);
  if (mcap < 0) {
    fprintf(stderr, "invalid shape: %s\n", moe_last_error());
    return 1;
  }
  const size_t T = (size_t)s.T, H = (size_t)s.H, E = (size_t)s.E, K = (size_t)s.K;
  const size_t I = (size_t)s.I, G = (size_t)(s.E + s.S), B = (size_t)s.block_m, R = (size_t)mcap;
  const size_t bf = 2, f4 = 4;

  uint16_t* x = dev_from_file(in, T * H * bf);
  float* w_gate = dev_from_file(in, E * H * f4);
  float* sel_bias = dev_from_file(in, E * f4);
  uint16_t* w1 = dev_from_file(in, G * 2 * I * H * bf);
  uint16_t* w2 = dev_from_file(in, G * H * I * bf);
  uint16_t* dy = dev_from_file(in, T * H * bf);
  fclose(in);

  float* logits = dev_alloc(T * E * f4);
  float* probs = dev_alloc(T * E * f4);
  int32_t* topk_idx = dev_alloc(T * K * f4);
  float* topk_w = dev_alloc(T * K * f4);
  int32_t* counts = dev_alloc(E * f4);
  int32_t* seg = dev_alloc((G + 1) * f4);
  int32_t* tile_group = dev_alloc((R / B) * f4);
  int32_t* total_rows = dev_alloc(f4);
  int32_t* row_token = dev_alloc(R * f4);
  int32_t* pos = dev_alloc(T * K * f4);
  const size_t ws_bytes = moe_workspace_size(&s);
  void* ws = dev_alloc(ws_bytes);
  uint16_t* x_perm = dev_alloc(R * H * bf);
  uint16_t* h_save = dev_alloc(R * 2 * I * bf);
  uint16_t* a = dev_alloc(R * I * bf);
  uint16_t* y_perm = dev_alloc(R * H * bf);
  uint16_t* y = dev_alloc(T * H * bf);
  uint16_t* dy_perm = dev_alloc(R * H * bf);
  float* dtopk_w = dev_alloc(T * K * f4);
  uint16_t* dh = dev_alloc(R * 2 * I * bf);
  uint16_t* dx_perm = dev_alloc(R * H * bf);
  uint16_t* dx = dev_alloc(T * H * bf);
  uint16_t* dw1 = dev_alloc(G * 2 * I * H * bf);
  uint16_t* dw2 = dev_alloc(G * H * I * bf);

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  MOE_OK_(moe_route(&s, x, w_gate, NULL, sel_bias, logits, probs, topk_idx, topk_w, counts, st));
  MOE_OK_(moe_permute(&s, topk_idx, x, seg, tile_group, total_rows, row_token, pos, x_perm, ws,
                      ws_bytes, st));
  MOE_OK_(grouped_gemm_fwd(&s, MOE_FWD_GATEUP | MOE_FWD_DOWN, x_perm, seg, tile_group, total_rows,
                           w1, w2, h_save, a, y_perm, st));
  MOE_OK_(moe_combine(&s, y_perm, pos, topk_w, seg, y, st));
  MOE_OK_(moe_combine_bwd(&s, dy, y_perm, pos, topk_w, seg, row_token, total_rows, dy_perm,
                          dtopk_w, st));
  MOE_OK_(grouped_gemm_bwd(&s, MOE_DGRAD_DOWN | MOE_DGRAD_GATEUP | MOE_WGRAD_DOWN | MOE_WGRAD_GATEUP,
                           x_perm, h_save, a, dy_perm, seg, tile_group, total_rows, w1, w2, dh,
                           dx_perm, dw1, dw2, st));
  MOE_OK_(moe_unpermute_bwd(&s, dx_perm, pos, seg, dx, st));
  HIP_OK(hipStreamSynchronize(st));

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  dev_to_file(out, topk_idx, T * K * f4);
  dev_to_file(out, topk_w, T * K * f4);
  dev_to_file(out, y, T * H * bf);
  dev_to_file(out, dtopk_w, T * K * f4);
  dev_to_file(out, dx, T * H * bf);
  dev_to_file(out, dw1, G * 2 * I * H * bf);
  dev_to_file(out, dw2, G * H * I * bf);
  fclose(out);
  HIP_OK(hipStreamDestroy(st));
  printf("moe_c_example: T=%d H=%d E=%d K=%d I=%d S=%d block_m=%d, %lld permuted rows: ok\n", s.T,
         s.H, s.E, s.K, s.I, s.S, s.block_m, (long long)mcap);
  return 0;
}
