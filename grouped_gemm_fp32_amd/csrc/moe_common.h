// Device helpers shared by the gfx950 kernels of the MoE feed-forward path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kNumXcd = 8;         // MI355X: 8 XCDs, workgroups dispatched round-robin over them

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// Two fp32 -> packed pair of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// Exact split of 8 fp32 values into three bf16 vectors with hi + mid + lo == w (each part is the
// remainder rounded to bf16, so every subtraction is exact in fp32).
__device__ __forceinline__ void split3(const float4& w0, const float4& w1, bf16x8_t& hi,
                                       bf16x8_t& mid, bf16x8_t& lo) {
  float r[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)r[i];
    hi[i] = h;
    r[i] -= (float)h;
    const __bf16 m = (__bf16)r[i];
    mid[i] = m;
    r[i] -= (float)m;
    lo[i] = (__bf16)r[i];
  }
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Wave-wide reductions over 64 lanes (butterfly: every lane ends with the result, and the order
// of operations is fixed, so results are deterministic run to run).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Workgroup id -> logical tile id so that consecutive logical tiles run on the same XCD (and so
// share its L2). Hardware places workgroup b on XCD b % 8; XCD x takes logical tiles
// [x*per, (x+1)*per). Returns -1 for workgroups with no tile (the grid may be an upper bound).
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t n_tiles) {
  const int64_t per = (n_tiles + kNumXcd - 1) / kNumXcd;
  if (bid >= per * kNumXcd) return -1;
  const int64_t l = (bid % kNumXcd) * per + bid / kNumXcd;
  return l < n_tiles ? l : -1;
}

}  // namespace moe
