// Weighted combine (unpermute) of the expert outputs and its backward, on gfx950.
//
// dots.llm1 Technical Report, section A2 "Architecture", MoE paragraph: a token's output is the
// gate-weighted sum of its top-k routed experts plus its always-active shared experts (weight 1).
// These kernels are HBM-bound gathers: one workgroup per token, 16-byte vector loads of the
// token's K + S expert rows, fp32 accumulation in slot order, shared experts last. No atomics.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 8;
constexpr int kMaxS = 4;

__device__ __forceinline__ void acc8(float* a, uint4 v, float w) {
  a[0] += w * lo_bf(v.x); a[1] += w * hi_bf(v.x);
  a[2] += w * lo_bf(v.y); a[3] += w * hi_bf(v.y);
  a[4] += w * lo_bf(v.z); a[5] += w * hi_bf(v.z);
  a[6] += w * lo_bf(v.w); a[7] += w * hi_bf(v.w);
}

__device__ __forceinline__ void add8(float* a, uint4 v) {
  a[0] += lo_bf(v.x); a[1] += hi_bf(v.x);
  a[2] += lo_bf(v.y); a[3] += hi_bf(v.y);
  a[4] += lo_bf(v.z); a[5] += hi_bf(v.z);
  a[6] += lo_bf(v.w); a[7] += hi_bf(v.w);
}

__device__ __forceinline__ uint4 pack8(const float* a) {
  return make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(a[4], a[5]),
                    pack_bf2(a[6], a[7]));
}

// y[t] = bf16( sum_j w[t,j] y_perm[pos[t,j]] + sum_s y_perm[seg[E+s] + t] ).
// WEIGHTED = false gives the unpermute backward: dx[t] = sum_j dx_perm[pos] + sum_s dx_perm[...].
template <bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void gather_sum_kernel(int H, int E, int K, int S,
                                                              const uint16_t* __restrict__ src,
                                                              const int32_t* __restrict__ pos,
                                                              const float* __restrict__ w,
                                                              const int32_t* __restrict__ seg,
                                                              uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  int64_t rows[kMaxK + kMaxS];
  float wt[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = j < K ? pos[(int64_t)t * K + j] : 0;
    wt[j] = (WEIGHTED && j < K) ? w[(int64_t)t * K + j] : 1.0f;
  }
#pragma unroll
  for (int s = 0; s < kMaxS; ++s) rows[kMaxK + s] = s < S ? (int64_t)seg[E + s] + t : 0;
  const int nv = H / 8;
  for (int c = threadIdx.x; c < nv; c += kThreads) {
    float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < K && rows[j] >= 0) {   // pos < 0: a slot that got no row (invalid expert index)
        const uint4 v = reinterpret_cast<const uint4*>(src + rows[j] * H)[c];
        if (WEIGHTED) acc8(a, v, wt[j]); else add8(a, v);
      }
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      if (s < S) add8(a, reinterpret_cast<const uint4*>(src + rows[kMaxK + s] * H)[c]);
    reinterpret_cast<uint4*>(out + (int64_t)t * H)[c] = pack8(a);
  }
}

// Backward of the combine for token t:
//   dy_perm[pos[t,j]] = bf16(w[t,j] dy[t]); dy_perm[seg[E+s] + t] = dy[t];
//   dtopk_w[t,j] = <dy[t], y_perm[pos[t,j]]> (fp32, fixed reduction order).
__global__ __launch_bounds__(kThreads) void combine_bwd_kernel(int H, int E, int K, int S,
                                                               const uint16_t* __restrict__ dy,
                                                               const uint16_t* __restrict__ y_perm,
                                                               const int32_t* __restrict__ pos,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ seg,
                                                               uint16_t* __restrict__ dy_perm,
                                                               float* __restrict__ dtopk_w) {
  __shared__ float red[kThreads / 64][kMaxK];
  const int t = blockIdx.x;
  int64_t rows[kMaxK];
  float wt[kMaxK], dot[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = j < K ? pos[(int64_t)t * K + j] : 0;
    wt[j] = j < K ? w[(int64_t)t * K + j] : 0.0f;
    dot[j] = 0.0f;
  }
  const int nv = H / 8;
  const uint4* dyr = reinterpret_cast<const uint4*>(dy + (int64_t)t * H);
  for (int c = threadIdx.x; c < nv; c += kThreads) {
    const uint4 g = dyr[c];
    const float gv[8] = {lo_bf(g.x), hi_bf(g.x), lo_bf(g.y), hi_bf(g.y),
                         lo_bf(g.z), hi_bf(g.z), lo_bf(g.w), hi_bf(g.w)};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < K && rows[j] >= 0) {   // pos < 0: no row (invalid expert index); dtopk_w = 0
        const uint4 v = reinterpret_cast<const uint4*>(y_perm + rows[j] * H)[c];
        float d = 0.0f;
        d += gv[0] * lo_bf(v.x); d += gv[1] * hi_bf(v.x);
        d += gv[2] * lo_bf(v.y); d += gv[3] * hi_bf(v.y);
        d += gv[4] * lo_bf(v.z); d += gv[5] * hi_bf(v.z);
        d += gv[6] * lo_bf(v.w); d += gv[7] * hi_bf(v.w);
        dot[j] += d;
        float o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = wt[j] * gv[q];
        reinterpret_cast<uint4*>(dy_perm + rows[j] * H)[c] = pack8(o);
      }
    for (int s = 0; s < S; ++s)
      reinterpret_cast<uint4*>(dy_perm + ((int64_t)seg[E + s] + t) * H)[c] = g;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const float v = wave_sum(dot[j]);
    if (lane == 0) red[wave][j] = v;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    float v = 0.0f;
    for (int q = 0; q < kThreads / 64; ++q) v += red[q][threadIdx.x];
    dtopk_w[(int64_t)t * K + threadIdx.x] = v;
  }
}

// Zero the padding rows (row_token < 0) of a permuted buffer, rows < total_rows.
__global__ __launch_bounds__(kThreads) void zero_pad_rows_kernel(int H, int64_t mcap,
                                                                 const int32_t* __restrict__ total,
                                                                 const int32_t* __restrict__ row_token,
                                                                 uint16_t* __restrict__ buf) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= mcap || r >= total[0] || row_token[r] >= 0) return;
  uint4* dst = reinterpret_cast<uint4*>(buf + r * H);
  for (int c = lane; c < H / 8; c += 64) dst[c] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_combine(const moe_shape_t& s, const uint16_t* y_perm, const int32_t* pos,
                          const float* topk_w, const int32_t* seg_offsets, uint16_t* y,
                          hipStream_t st) {
  hipLaunchKernelGGL(gather_sum_kernel<true>, dim3(s.T), dim3(kThreads), 0, st, s.H, s.E, s.K,
                     s.S, y_perm, pos, topk_w, seg_offsets, y);
  return hipGetLastError();
}

hipError_t launch_unpermute_bwd(const moe_shape_t& s, const uint16_t* dx_perm, const int32_t* pos,
                                const int32_t* seg_offsets, uint16_t* dx, hipStream_t st) {
  hipLaunchKernelGGL(gather_sum_kernel<false>, dim3(s.T), dim3(kThreads), 0, st, s.H, s.E, s.K,
                     s.S, dx_perm, pos, (const float*)nullptr, seg_offsets, dx);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const moe_shape_t& s, int64_t mcap, const uint16_t* dy,
                              const uint16_t* y_perm, const int32_t* pos, const float* topk_w,
                              const int32_t* seg_offsets, const int32_t* row_token,
                              const int32_t* total_rows, uint16_t* dy_perm, float* dtopk_w,
                              hipStream_t st) {
  const int64_t rpw = kThreads / 64;
  hipLaunchKernelGGL(zero_pad_rows_kernel, dim3((unsigned)((mcap + rpw - 1) / rpw)),
                     dim3(kThreads), 0, st, s.H, mcap, total_rows, row_token, dy_perm);
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(s.T), dim3(kThreads), 0, st, s.H, s.E, s.K, s.S, dy,
                     y_perm, pos, topk_w, seg_offsets, dy_perm, dtopk_w);
  return hipGetLastError();
}

}  // namespace moe
