// Router backward and the load-balancing bias update on gfx950.
//
// dots.llm1 Technical Report, section A2 "Architecture", load-balancing paragraph: the router's
// per-expert bias decides the top-k only and is adjusted during training to keep the expert loads
// balanced. The routing weights reach the loss only through the softmax probabilities of the
// selected experts, so the logits' gradient follows from the weights' gradient (dtopk_w, from the
// combine backward) by the chain rule; the selection and the bias pass none.
//
// Kernels:
//   route_bwd_kernel    one wavefront per token (a few consecutive tokens each):
//                       renormalised weights w_k = p_k / S (S summed in slot order, as the forward
//                       does), c = sum_k w_k dw_k, dlogits = w_k (dw_k - c) on the selected experts
//                       and 0 elsewhere; unnormalised weights: c = sum_k p_k dw_k and
//                       dlogits_e = p_e (g_e - c) with g_e = dw_k on the selected experts.
//   router_dwg_kernel   dWg[E,H] = dlogits^T x, an fp32 contraction over the tokens on the fp32
//                       matrix unit (v_mfma_f32_32x32x2_f32): one workgroup per 32 x 32 tile of dWg,
//                       its four wavefronts take a quarter of the tokens each and their partial
//                       sums are added in wavefront order (deterministic).
//   router_dx_kernel    dx_router[T,H] = dlogits Wg, the same instruction with the contraction
//                       over the experts: a 32-token tile of dlogits in LDS, Wg read from L2.
//   bias_update_kernel  b_e += gamma * sign(T K - E c_e), one fp32 add per expert.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 2048;   // target wavefront count of the per-token kernel
constexpr int kMaxE = 256;     // most routed experts a shape may have

// ---- dlogits ------------------------------------------------------------------------------------
template <bool NORM>
__global__ __launch_bounds__(kThreads) void route_bwd_kernel(int T, int E, int K, int tpw,
                                                             const float* __restrict__ dtopk_w,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ probs,
                                                             float* __restrict__ dlogits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tb = (blockIdx.x * (kThreads / 64) + wave) * tpw;
  const int tn = min(T, tb + tpw);
  for (int t = tb; t < tn; ++t) {
    // Slot data, the same on every lane: expert, its probability and its weight gradient.
    int ek[8];
    float pk[8], dk[8];
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ek[j] = -1;
      pk[j] = 0.0f;
      dk[j] = 0.0f;
      if (j < K) {
        ek[j] = topk_idx[(int64_t)t * K + j];
        pk[j] = probs[(int64_t)t * E + ek[j]];
        dk[j] = dtopk_w[(int64_t)t * K + j];
        S += pk[j];   // slot order, as the forward's weight sum
      }
    }
    float c = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) c += (NORM ? pk[j] / S : pk[j]) * dk[j];
    for (int e = lane; e < E; e += 64) {
      float g = 0.0f;
      bool sel = false;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < K && ek[j] == e) { g = dk[j]; sel = true; }
      float dz;
      if (NORM) {
        // p_e / S is bit-identical to the forward's weight of this expert
        dz = sel ? (probs[(int64_t)t * E + e] / S) * (g - c) : 0.0f;
      } else {
        dz = probs[(int64_t)t * E + e] * (g - c);
      }
      dlogits[(int64_t)t * E + e] = dz;
    }
  }
}

// ---- dWg = dlogits^T x ----------------------------------------------------------------------------
// MFMA 32x32x2 f32: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; the result D[i][j]
// sits in lane j (+32 for rows 4..7 of each group of 8), register q -> row 8 (q / 4) + 4 (l / 32)
// + q % 4.
constexpr int kDwgUnroll = 8;

__global__ __launch_bounds__(kThreads) void router_dwg_kernel(int T, int H, int E,
                                                              const float* __restrict__ dz,
                                                              const uint16_t* __restrict__ x,
                                                              float* __restrict__ dwg) {
  __shared__ float red[4][32][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * 32, h0 = blockIdx.y * 32;
  const int r = lane & 31, kh = lane >> 5;
  const int e = e0 + r, h = h0 + r;
  const bool e_ok = e < E;
  // this wave's quarter of the tokens, in pairs (one MFMA each)
  const int per = (((T + 3) / 4) + 1) & ~1;
  const int ta = min(T, wave * per), tz = min(T, ta + per);
  f32x16_t acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  for (int t0 = ta; t0 < tz; t0 += 2 * kDwgUnroll) {
    float a[kDwgUnroll], b[kDwgUnroll];
#pragma unroll
    for (int u = 0; u < kDwgUnroll; ++u) {
      const int t = t0 + 2 * u + kh;
      const bool ok = t < tz;
      a[u] = (ok && e_ok) ? dz[(int64_t)t * E + e] : 0.0f;
      b[u] = ok ? __uint_as_float((uint32_t)x[(int64_t)t * H + h] << 16) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kDwgUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], b[u], acc, 0, 0, 0);
  }
  // D[e][h]: lane -> h = h0 + r, register q -> e = e0 + 8 (q / 4) + 4 kh + q % 4
#pragma unroll
  for (int q = 0; q < 16; ++q) red[wave][8 * (q >> 2) + 4 * kh + (q & 3)][r] = acc[q];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 32; idx += kThreads) {
    const int el = idx / 32, hl = idx % 32;
    if (e0 + el < E) {
      const float v = red[0][el][hl] + red[1][el][hl] + red[2][el][hl] + red[3][el][hl];
      dwg[(int64_t)(e0 + el) * H + h0 + hl] = v;
    }
  }
}

// ---- dx_router = dlogits Wg ---------------------------------------------------------------------
constexpr int kDxTok = 32;

__global__ __launch_bounds__(kThreads) void router_dx_kernel(int T, int H, int E,
                                                             const float* __restrict__ dz,
                                                             const float* __restrict__ wg,
                                                             float* __restrict__ dx) {
  __shared__ float tile[kDxTok * (kMaxE + 1)];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kDxTok, h0 = blockIdx.y * 128 + wave * 32;
  const int nt = min(kDxTok, T - t0);
  const int ld = E + 1;
  for (int i = threadIdx.x; i < kDxTok * E; i += kThreads) {
    const int tl = i / E, e = i % E;
    tile[tl * ld + e] = tl < nt ? dz[(int64_t)(t0 + tl) * E + e] : 0.0f;
  }
  __syncthreads();
  const int r = lane & 31, kh = lane >> 5;
  f32x16_t acc;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.0f;
  // D[t][h] = sum_e A[t][e] B[e][h]: A from the LDS tile, B = Wg rows (128 contiguous bytes)
  for (int e0 = 0; e0 < E; e0 += 2) {
    const int e = e0 + kh;
    const float a = e < E ? tile[r * ld + e] : 0.0f;
    const float b = e < E ? wg[(int64_t)e * H + h0 + r] : 0.0f;
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
  // lane -> h = h0 + r, register q -> t = t0 + 8 (q / 4) + 4 kh + q % 4
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int tl = 8 * (q >> 2) + 4 * kh + (q & 3);
    if (tl < nt) dx[(int64_t)(t0 + tl) * H + h0 + r] = acc[q];
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ---- bias update --------------------------------------------------------------------------------
__global__ void bias_update_kernel(int E, int64_t TK, float gamma, const int32_t* __restrict__ counts,
                                   float* __restrict__ bias) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int64_t d = TK - (int64_t)E * counts[e];   // sign of (mean load - load), exactly
  if (d > 0) bias[e] = bias[e] + gamma;
  else if (d < 0) bias[e] = bias[e] - gamma;
}

}  // namespace

hipError_t launch_route_bwd(const moe_shape_t& s, const float* dtopk_w, const int32_t* topk_idx,
                            const float* probs, const uint16_t* x, const float* wg, float* dlogits,
                            float* dw_gate, float* dx_router, hipStream_t st) {
  const bool norm = (s.flags & MOE_NORM_TOPK) != 0;
  if (s.T == 0) {   // an empty batch: the weight gradient is a sum over no tokens
    if (dw_gate) {
      const int64_t n = (int64_t)s.E * s.H;
      hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         dw_gate, n);
    }
    return hipGetLastError();
  }
  const int tpw = (s.T + kWaves - 1) / kWaves;
  const int per_wg = tpw * (kThreads / 64);
  const dim3 grid((unsigned)((s.T + per_wg - 1) / per_wg));
  if (norm)
    hipLaunchKernelGGL(route_bwd_kernel<true>, grid, dim3(kThreads), 0, st, s.T, s.E, s.K, tpw,
                       dtopk_w, topk_idx, probs, dlogits);
  else
    hipLaunchKernelGGL(route_bwd_kernel<false>, grid, dim3(kThreads), 0, st, s.T, s.E, s.K, tpw,
                       dtopk_w, topk_idx, probs, dlogits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dw_gate) {
    hipLaunchKernelGGL(router_dwg_kernel, dim3((unsigned)((s.E + 31) / 32), (unsigned)(s.H / 32)),
                       dim3(kThreads), 0, st, s.T, s.H, s.E, dlogits, x, dw_gate);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dx_router) {
    hipLaunchKernelGGL(router_dx_kernel, dim3((unsigned)((s.T + kDxTok - 1) / kDxTok), (unsigned)(s.H / 128)),
                       dim3(kThreads), 0, st, s.T, s.H, s.E, dlogits, wg, dx_router);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_bias_update(const moe_shape_t& s, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((unsigned)((s.E + 255) / 256)), dim3(256), 0, st, s.E,
                     (int64_t)s.T * s.K, gamma, counts, bias);
  return hipGetLastError();
}

}  // namespace moe
