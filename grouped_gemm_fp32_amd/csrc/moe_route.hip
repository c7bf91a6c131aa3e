// Router of the MoE layer on gfx950: FP32 gating and biased top-k selection.
//
// dots.llm1 Technical Report, section A2 "Architecture" (MoE paragraph): the gating layer is
// computed in FP32 and picks the top-6 routed experts per token. Section A2, load-balancing
// paragraph: a per-expert bias is added to the affinity scores to decide the top-k, and only there.
//
// One kernel does the whole router for a block of 32 tokens:
//   1. logits[32, E] = fp32(x) . Wg^T with v_mfma_f32_32x32x2_f32 (fp32 inputs, fp32 accumulate),
//      x and Wg staged through LDS in k-chunks of 64;
//   2. one wavefront per token: softmax over E (wave reductions), key = p + b, K rounds of a
//      wave-wide arg-max on a 64-bit (key, index) code, weights, per-expert counts.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokPerWg = 32;   // tokens per workgroup (the MFMA's 32 rows)
constexpr int kRouteThreads = 256;
constexpr int kKc = 64;          // k-chunk staged in LDS
constexpr int kMaxE = 256;

enum RouteMode { kFromX = 0, kFromLogits = 1, kFromProbs = 2 };

// Order-preserving map of a float key to uint32 (larger key -> larger code). -0 and +0 map to the
// same code; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t key_code(float k) {
  if (k != k) return 0u;
  uint32_t u = __float_as_uint(k);
  if (k == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int MODE>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int T, int H, int E, int K, uint32_t flags, const uint16_t* __restrict__ x,
    const float* __restrict__ wg, const float* __restrict__ logit_bias,
    const float* __restrict__ sel_bias, float* __restrict__ logits, float* __restrict__ probs,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ counts) {
  // LDS: staging for the GEMM (x chunk 32 x 64, Wg chunk E x 64, padded rows), then reused for
  // the [32][E] score tile.
  __shared__ float sx[kTokPerWg][kKc + 4];
  __shared__ float sw[kMaxE][kKc + 4];
  __shared__ int hist[kMaxE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kTokPerWg;
  const int ntok = min(kTokPerWg, T - t0);

  for (int e = tid; e < E; e += kRouteThreads) hist[e] = 0;

  // score[tok][e] lives in sw's storage after the GEMM: [32][E] floats.
  float* score = &sw[0][0];
  const int sstride = kMaxE + 1;  // 32 * 257 floats fits in sw (256 * 68)

  if (MODE == kFromX) {
    // ---- 1. logits = x . Wg^T on fp32 MFMA -------------------------------------------------
    // Wave w owns experts [w*32, w*32+32) and, for E > 128, [128 + w*32, ...).
    const int n_et = (E + 31) / 32;  // expert tiles of 32
    f32x16_t acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;

    for (int k0 = 0; k0 < H; k0 += kKc) {
      // x chunk: 32 tokens x 64 k (bf16 -> fp32, exact). 256 threads x 8 elements.
      {
        const int tk = tid >> 3, c = (tid & 7) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (tk < ntok) v = *reinterpret_cast<const uint4*>(x + (int64_t)(t0 + tk) * H + k0 + c);
        float* d = &sx[tk][c];
        d[0] = lo_bf(v.x); d[1] = hi_bf(v.x); d[2] = lo_bf(v.y); d[3] = hi_bf(v.y);
        d[4] = lo_bf(v.z); d[5] = hi_bf(v.z); d[6] = lo_bf(v.w); d[7] = hi_bf(v.w);
      }
      // Wg chunk: E x 64 fp32, 16 floats (4 x float4) per thread-iteration.
      for (int idx = tid; idx < E * (kKc / 4); idx += kRouteThreads) {
        const int e = idx / (kKc / 4), c = (idx % (kKc / 4)) * 4;
        const float4 v = *reinterpret_cast<const float4*>(wg + (int64_t)e * H + k0 + c);
        *reinterpret_cast<float4*>(&sw[e][c]) = v;
      }
      __syncthreads();
      // 64 k per chunk = 16 groups of 4; lane l takes k = 4*(l/32) + {0..3} of an 8-wide group,
      // the same mapping for both operands, so each MFMA sums a consistent pair of k.
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int et = wave + q * 4;
        if (et < n_et) {
          const int e = et * 32 + (lane & 31);
          const bool ev = e < E;
#pragma unroll
          for (int kg = 0; kg < kKc; kg += 8) {
            const int kk = kg + (lane >> 5) * 4;
            const float4 a4 = *reinterpret_cast<const float4*>(&sx[lane & 31][kk]);
            float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
            if (ev) b4 = *reinterpret_cast<const float4*>(&sw[e][kk]);
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(b4.x, a4.x, acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(b4.y, a4.y, acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(b4.z, a4.z, acc[q], 0, 0, 0);
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(b4.w, a4.w, acc[q], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
    // D[e][tok]: lane -> token (lane & 31), registers -> 4 consecutive experts per group of 4.
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int et = wave + q * 4;
      if (et < n_et) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int e = et * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int tk = lane & 31;
          if (e < E) {
            float z = acc[q][r];
            if (logit_bias) z += logit_bias[e];
            score[tk * sstride + e] = z;
          }
        }
      }
    }
    __syncthreads();
    if (logits) {
      for (int idx = tid; idx < ntok * E; idx += kRouteThreads) {
        const int tk = idx / E, e = idx % E;
        logits[(int64_t)(t0 + tk) * E + e] = score[tk * sstride + e];
      }
    }
  } else {
    const float* src = MODE == kFromLogits ? logits : probs;
    for (int idx = tid; idx < ntok * E; idx += kRouteThreads) {
      const int tk = idx / E, e = idx % E;
      score[tk * sstride + e] = src[(int64_t)(t0 + tk) * E + e];
    }
    __syncthreads();
  }

  // ---- 2. per token: softmax, biased top-K, weights, counts (one wavefront per token) --------
  const bool norm = (flags & MOE_NORM_TOPK) != 0;
  float bias[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    bias[s] = (e < E && sel_bias) ? sel_bias[e] : 0.0f;
  }
  for (int tk = wave; tk < ntok; tk += kRouteThreads / 64) {
    const int t = t0 + tk;
    float p[4];
    if (MODE == kFromProbs) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        p[s] = e < E ? score[tk * sstride + e] : 0.0f;
      }
    } else {
      float z[4];
      float m = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        z[s] = e < E ? score[tk * sstride + e] : -INFINITY;
        m = fmaxf(m, z[s]);
      }
      m = wave_max(m);
      float sum = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        p[s] = e < E ? expf(z[s] - m) : 0.0f;
        sum += p[s];
      }
      sum = wave_sum(sum);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        p[s] = p[s] / sum;
        if (probs && e < E) probs[(int64_t)t * E + e] = p[s];
      }
    }
    uint32_t code[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      code[s] = e < E ? key_code(p[s] + bias[s]) : 0u;
    }
    uint32_t taken = 0;  // bit s: expert lane + 64 s already selected
    float wsum = 0.0f, sel_p[8];
    int sel_e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sel_p[j] = 0.0f;
      sel_e[j] = 0;
      if (j < K) {
        // Best local candidate: highest code, then lowest index.
        uint32_t bc = 0, bi = 0xffffffffu;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int e = lane + 64 * s;
          if (e < E && !(taken & (1u << s))) {
            if (bi == 0xffffffffu || code[s] > bc) { bc = code[s]; bi = (uint32_t)e; }
          }
        }
        // Wave arg-max on (code, ~index): a lane without a candidate offers (0, 0), which loses
        // to every real expert, NaN keys (code 0) included.
        uint32_t hi = bc, lo = ~bi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const uint32_t ohi = __shfl_xor(hi, o, 64), olo = __shfl_xor(lo, o, 64);
          if (ohi > hi || (ohi == hi && olo > lo)) { hi = ohi; lo = olo; }
        }
        const int e = (int)(~lo);
        if ((e & 63) == lane) taken |= 1u << (e >> 6);
        const int s = e >> 6;
        const float pv = s == 0 ? p[0] : s == 1 ? p[1] : s == 2 ? p[2] : p[3];
        const float pe = __shfl(pv, e & 63, 64);
        sel_e[j] = e;
        sel_p[j] = pe;
        wsum += pe;  // slot order
      }
    }
    if (lane < K) {
      float pe = sel_p[0];
      int e = sel_e[0];
#pragma unroll
      for (int j = 1; j < 8; ++j)
        if (j == lane) { pe = sel_p[j]; e = sel_e[j]; }
      topk_idx[(int64_t)t * K + lane] = e;
      topk_w[(int64_t)t * K + lane] = norm ? pe / wsum : pe;
      if (counts) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  if (counts)
    for (int e = tid; e < E; e += kRouteThreads)
      if (hist[e]) atomicAdd(&counts[e], hist[e]);
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int th = 256;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + th - 1) / th)), dim3(th), 0, st, p, v, n);
  return hipGetLastError();
}

hipError_t launch_route(const moe_shape_t& s, const uint16_t* x, const float* wg,
                        const float* logit_bias, const float* sel_bias, float* logits,
                        float* probs, int32_t* topk_idx, float* topk_w, int32_t* counts,
                        hipStream_t st) {
  if (counts) {
    hipError_t e = launch_fill_i32(counts, 0, s.E, st);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)((s.T + kTokPerWg - 1) / kTokPerWg)), block(kRouteThreads);
  if (s.flags & MOE_PROBS_IN) {
    hipLaunchKernelGGL(route_kernel<kFromProbs>, grid, block, 0, st, s.T, s.H, s.E, s.K, s.flags,
                       x, wg, logit_bias, sel_bias, logits, probs, topk_idx, topk_w, counts);
  } else if (x) {
    hipLaunchKernelGGL(route_kernel<kFromX>, grid, block, 0, st, s.T, s.H, s.E, s.K, s.flags, x,
                       wg, logit_bias, sel_bias, logits, probs, topk_idx, topk_w, counts);
  } else {
    hipLaunchKernelGGL(route_kernel<kFromLogits>, grid, block, 0, st, s.T, s.H, s.E, s.K, s.flags,
                       x, wg, logit_bias, sel_bias, logits, probs, topk_idx, topk_w, counts);
  }
  return hipGetLastError();
}

}  // namespace moe
