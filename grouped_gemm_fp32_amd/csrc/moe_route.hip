// Router of the MoE layer on gfx950: FP32 gating and biased top-k selection.
//
// dots.llm1 Technical Report, section A2 "Architecture" (MoE paragraph): the gating layer is
// computed in FP32 and picks the top-6 routed experts per token. Section A2, load-balancing
// paragraph: a per-expert bias is added to the affinity scores to decide the top-k, and only there.
//
// Kernels:
//   1. router_logits_kernel: logits = x . Wg^T (+ logit_bias) in fp32 on the bf16 matrix unit. x is
//      bf16, so exact; each fp32 weight is split exactly into three bf16 parts w = hi + mid + lo
//      (24 significand bits), and three v_mfma_f32_32x32x16_bf16 per k-slice accumulate x*hi +
//      x*mid + x*lo in fp32. Every product is exact in fp32, so this is the fp32 dot product up
//      to summation order. One workgroup per 64 tokens (32 for small batches) x 32 experts; its
//      wavefronts split the 64-k steps and their partial sums are added in wavefront order.
//      router_logits_dma_kernel computes the same from 16384 tokens on: 64 tokens and every
//      expert per workgroup, x and Wg staged in LDS by the buffer->LDS DMA.
//   2. route_kernel, one wavefront per token at a time (a few consecutive tokens each): softmax
//      over E, key = p + b, K rounds of a wave-wide arg-max on a 64-bit (key, index) code,
//      weights. Its cross-lane reductions use DPP and permlane swaps, not the LDS crossbar.
//   3. count_kernel: per-expert counts of the selected slots, 16 experts x one chunk of topk_idx
//      per workgroup, reduced across the workgroup and added with one integer atomic per expert
//      and chunk (into counts cleared first); a batch of one chunk (decode) stores its sums
//      directly, with no clear.
#include "moe_common.h"
#include "moe_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = 8192;   // target wavefront count of the routing kernel
constexpr int kMaxE = 256;

enum RouteMode { kFromLogits = 1, kFromProbs = 2 };

// Order-preserving map of a float key to uint32 (larger key -> larger code). -0 and +0 map to the
// same code; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t key_code(float k) {
  if (k != k) return 0u;
  uint32_t u = __float_as_uint(k);
  if (k == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- 1. router logits ---------------------------------------------------------------------------
constexpr int kLgTile = 32;      // experts per workgroup (the MFMA's 32)
constexpr int kLgLargeT = 4096;  // from this many tokens the logits use two token blocks per wave

// logits[t0.., e0..] for TB x 32 tokens and 32 experts. Lanes 0-31 hold token (B) and expert (A)
// rows r = lane; within a 64-k step lane half h = lane >> 5 covers k = 32 h + 8 s .. +8 in slice s
// (the same assignment for both operands, so each MFMA sums matching pairs and four slices cover
// the step). With TB = 2 token blocks every split of Wg feeds two MFMA blocks. Each wavefront
// takes every NW-th 64-k step and loads the next one's operands while the current MFMAs run; the
// NW partial sums are added in wavefront order (deterministic). Large batches use TB = 2 and four
// wavefronts; small ones (decode) one token block and eight, to spread the contraction wider.
template <int TB>
struct LgOps {
  uint4 x[TB][4];   // token blocks: 4 slices of 8 bf16
  float4 w[8];      // the expert row: 4 slices of 8 fp32
};

template <int TB, int NW>
__global__ __launch_bounds__(NW * 64) void router_logits_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ logit_bias, float* __restrict__ logits) {
  constexpr int TOK = 32 * TB;
  __shared__ float red[NW][kLgTile][TOK + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TOK, e0 = blockIdx.y * kLgTile;
  const int r = lane & 31, h = lane >> 5;
  // rows past the end are clamped (read, never stored)
  const uint16_t* xr[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) xr[b] = x + (int64_t)min(t0 + 32 * b + r, T - 1) * H + h * 32;
  const float* wr = wg + (int64_t)min(e0 + r, E - 1) * H + h * 32;
  auto load = [&](int step, LgOps<TB>& o) {
    const int k = step * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int b = 0; b < TB; ++b) o.x[b][i] = *reinterpret_cast<const uint4*>(xr[b] + k + 8 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) o.w[i] = *reinterpret_cast<const float4*>(wr + k + 4 * i);
  };
  f32x16_t acc[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[b][q] = 0.0f;
  const int nstep = H / 64;   // H % 64 == 0
  LgOps<TB> cur;
  if (wave < nstep) load(wave, cur);
  for (int step = wave; step < nstep; step += NW) {
    LgOps<TB> nxt;
    if (step + NW < nstep) load(step + NW, nxt);
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      bf16x8_t a[TB], whi, wmid, wlo;
#pragma unroll
      for (int b = 0; b < TB; ++b) __builtin_memcpy(&a[b], &cur.x[b][sl], 16);
      split3(cur.w[2 * sl], cur.w[2 * sl + 1], whi, wmid, wlo);
#pragma unroll
      for (int b = 0; b < TB; ++b)   // smallest part first
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wlo, a[b], acc[b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < TB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wmid, a[b], acc[b], 0, 0, 0);
#pragma unroll
      for (int b = 0; b < TB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(whi, a[b], acc[b], 0, 0, 0);
    }
    cur = nxt;
  }
  // D[expert][token]: lane -> token 32 b + r, register q -> expert 8 (q / 4) + 4 h + q % 4.
#pragma unroll
  for (int b = 0; b < TB; ++b)
#pragma unroll
    for (int q = 0; q < 16; ++q) red[wave][8 * (q >> 2) + 4 * h + (q & 3)][32 * b + r] = acc[b][q];
  __syncthreads();
  for (int idx = threadIdx.x; idx < kLgTile * TOK; idx += NW * 64) {
    const int el = idx / TOK, tl = idx % TOK;
    if (t0 + tl < T && e0 + el < E) {
      float z = red[0][el][tl];
#pragma unroll
      for (int w = 1; w < NW; ++w) z += red[w][el][tl];
      if (logit_bias) z += logit_bias[e0 + el];
      logits[(int64_t)(t0 + tl) * E + e0 + el] = z;
    }
  }
}

// 16-byte chunk position of chunk c in a 128-byte K-major LDS row r (an involution): the 16 rows
// a 16-lane group reads land on distinct bank slots.
__device__ __forceinline__ int kswz64(int r, int c) { return c ^ ((r >> 1) & 7); }

// ---- 1b. router logits for large batches, operands staged in LDS ---------------------------------
// 64 tokens per workgroup and every expert (E padded to 128 * EBW). Per 64-k step the buffer->LDS
// DMA brings x[64 tokens][64 k] (bf16, 128-byte rows) and Wg[experts][64 k] (fp32, 256-byte rows)
// into a ring of NS stages, whole cache lines per request. Eight wavefronts, two per SIMD: wave
// w takes expert blocks (w & 3) + 4 e for both token blocks, waves 0-3 the first two 16-k slices
// of every step and waves 4-7 the last two. A wavefront reads its experts' fp32 values from LDS
// (32 bytes per lane per slice), splits them exactly into three bf16 parts in registers (split3)
// and runs the three part MFMAs against both token blocks. At the end waves 4-7 hand their sums
// to waves 0-3 through LDS, which add them in that fixed order, so the result is deterministic.
// x is read from HBM once; Wg (at most 4 MiB) comes from L2 for every workgroup.
constexpr int kLgDmaTok = 64;
constexpr int kLgDmaMinT = 16384;   // from this many tokens (256 workgroups of 64)
constexpr int kLgDmaThreads = 512;

template <int EBW>
struct LgDma {
  static constexpr int EP = 32 * 4 * EBW;            // experts covered (padded)
  static constexpr int X_BYTES = kLgDmaTok * 128;    // 8 KiB
  static constexpr int W_BYTES = EP * 256;           // 32 or 64 KiB
  static constexpr int STAGE = X_BYTES + W_BYTES;
  static constexpr int NS = EBW == 1 ? 4 : 2;        // ring slots
  static constexpr int NW = kLgDmaThreads / 64;
  static constexpr int LX = X_BYTES / (NW * 1024), LW = W_BYTES / (NW * 1024), L = LX + LW;
  static_assert(NS * STAGE <= 163840, "LDS budget");
  static_assert(NS <= 5 && (NS - 1) * L < 64, "vmcnt range");
  static_assert(X_BYTES % (NW * 1024) == 0 && W_BYTES % (NW * 1024) == 0, "whole DMA rounds");
  static_assert(4 * EP * kLgDmaTok <= NS * STAGE, "the hand-over of the partial sums fits");
};

template <int EBW>
__global__ __launch_bounds__(kLgDmaThreads, 1) void router_logits_dma_kernel(
    int T, int H, int E, const uint16_t* __restrict__ x, const float* __restrict__ wg,
    const float* __restrict__ logit_bias, float* __restrict__ logits) {
  typedef LgDma<EBW> C;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[C::NS * C::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = (int)uniform((uint32_t)(threadIdx.x >> 6));
  const int eb0 = wave & 3, half = wave >> 2;
  const int t0 = blockIdx.x * kLgDmaTok;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
  // x rows t0.. (rows past T read as zero), all of Wg (rows past E read as zero)
  const v4u32_t rx = make_rsrc(x + (int64_t)t0 * H, (int64_t)(T - t0) * H * 2);
  const v4u32_t rw = make_rsrc(wg, (int64_t)E * H * 4);
  // x: instruction i of wavefront w fills token rows (NW i + w) * 8 + lane / 8, 16-byte chunk
  // position lane % 8 holding chunk position ^ ((row >> 1) & 7) (rows step by 64 between
  // instructions, which keeps that swizzle). Wg: instruction j fills expert rows (NW j + w) * 4 +
  // lane / 16, position lane % 16 holding chunk position ^ (row & 15) (rows step by 32).
  const int xr = wave * 8 + lane / 8, xc = (lane % 8) ^ ((xr >> 1) & 7);
  const uint32_t xoff = (uint32_t)(((int64_t)xr * H + xc * 8) * 2);
  const int wr = wave * 4 + lane / 16, wc = (lane % 16) ^ (wr & 15);
  const uint32_t woff = (uint32_t)(((int64_t)wr * H + wc * 4) * 4);
  auto issue = [&](int kt, int slot) {
    const uint32_t sl = lds_base + slot * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LX; ++i)
      dma16(rx, xoff + uniform((uint32_t)(kt * 128 + i * NW * 8 * H * 2)),
            sl + (i * NW + wave) * 1024);
#pragma unroll
    for (int j = 0; j < C::LW; ++j)
      dma16(rw, woff + uniform((uint32_t)(kt * 256 + j * NW * 4 * H * 4)),
            sl + C::X_BYTES + (j * NW + wave) * 1024);
  };
  f32x16_t acc[EBW][2];
#pragma unroll
  for (int e = 0; e < EBW; ++e)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[e][b][q] = 0.0f;
  const int r = lane & 31, h = lane >> 5;
  const int nst = H / 64;
  for (int s = 0; s < C::NS - 1 && s < nst; ++s) issue(s, s);
  for (int kt = 0; kt < nst; ++kt) {
    // this wavefront's DMA of stage kt has landed (at most NS - 2 later stages are in flight);
    // the barrier makes that true for all, and frees the slot every wavefront used at kt - 1
    wait_stages<C::L, C::NS - 2>(min(C::NS - 2, nst - 1 - kt));
    block_barrier();
    if (kt + C::NS - 1 < nst) issue(kt + C::NS - 1, (kt + C::NS - 1) % C::NS);
    const unsigned char* sx = smem + (kt % C::NS) * C::STAGE;
    const unsigned char* sw = sx + C::X_BYTES;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int sl = 2 * half + s2;
      bf16x8_t xf[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int row = b * 32 + r;
        xf[b] = *reinterpret_cast<const bf16x8_t*>(sx + row * 128 + kswz64(row, 2 * sl + h) * 16);
      }
#pragma unroll
      for (int e = 0; e < EBW; ++e) {
        const int row = (eb0 + 4 * e) * 32 + r;
        const int c0 = 4 * sl + 2 * h;
        const float4 w0 = *reinterpret_cast<const float4*>(sw + row * 256 + ((c0 ^ (row & 15)) * 16));
        const float4 w1 =
            *reinterpret_cast<const float4*>(sw + row * 256 + (((c0 + 1) ^ (row & 15)) * 16));
        bf16x8_t whi, wmid, wlo;
        split3(w0, w1, whi, wmid, wlo);
#pragma unroll
        for (int b = 0; b < 2; ++b)   // smallest part first
          acc[e][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wlo, xf[b], acc[e][b], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[e][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wmid, xf[b], acc[e][b], 0, 0, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[e][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(whi, xf[b], acc[e][b], 0, 0, 0);
      }
    }
  }
  // waves 4-7 hand their partial sums (the last two slices of every step) to waves 0-3
  float* hand = reinterpret_cast<float*>(smem);   // [4][EBW][2][16][64]
  wait_lgkm0();
  block_barrier();
  if (half) {
#pragma unroll
    for (int e = 0; e < EBW; ++e)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int q = 0; q < 16; ++q) hand[(((eb0 * EBW + e) * 2 + b) * 16 + q) * 64 + lane] = acc[e][b][q];
  }
  __syncthreads();
  if (half) return;
  // D[expert][token]: lane -> token 32 b + r, register q -> expert 8 (q / 4) + 4 h + q % 4
#pragma unroll
  for (int e = 0; e < EBW; ++e)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int t = t0 + 32 * b + r;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e4 = (eb0 + 4 * e) * 32 + 8 * g + 4 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ee = e4 + q;
          const float z0 = acc[e][b][4 * g + q] +
                           hand[(((eb0 * EBW + e) * 2 + b) * 16 + 4 * g + q) * 64 + lane];
          if (t < T && ee < E) logits[(int64_t)t * E + ee] = logit_bias ? z0 + logit_bias[ee] : z0;
        }
      }
    }
}

// ---- 2. softmax, biased top-K, weights -----------------------------------------------------------
// Cross-lane steps without the LDS crossbar: DPP for partners within a row of 16 lanes, and
// gfx950's permlane swaps for rows 16 and 32 apart. Each step combines two disjoint, equal-size
// lane groups that are already uniform, so after six steps every lane holds the reduction over
// all 64 lanes (and the same bits on every lane, since the combining order is fixed).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// The two values a permlane swap leaves: (own row group's, partner row group's), 16 or 32 apart.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0]; b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0]; b = r[1];
}

template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, __uint_as_float(dpp<kDppXor1>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kDppXor2>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp<kDppMirror>(__float_as_uint(v))));
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = op(__uint_as_float(a), __uint_as_float(b));
  swap32(__float_as_uint(v), a, b);
  return op(__uint_as_float(a), __uint_as_float(b));
}

// Larger of two (code, ~index) pairs: higher code, then lower expert index.
__device__ __forceinline__ void pair_max(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
  if (ohi > hi || (ohi == hi && olo > lo)) { hi = ohi; lo = olo; }
}
__device__ __forceinline__ void wave_argmax(uint32_t& hi, uint32_t& lo) {
  pair_max(hi, lo, dpp<kDppXor1>(hi), dpp<kDppXor1>(lo));
  pair_max(hi, lo, dpp<kDppXor2>(hi), dpp<kDppXor2>(lo));
  pair_max(hi, lo, dpp<kDppHalfMirror>(hi), dpp<kDppHalfMirror>(lo));
  pair_max(hi, lo, dpp<kDppMirror>(hi), dpp<kDppMirror>(lo));
  uint32_t ah, bh, al, bl;
  swap16(hi, ah, bh); swap16(lo, al, bl);
  hi = ah; lo = al; pair_max(hi, lo, bh, bl);
  swap32(hi, ah, bh); swap32(lo, al, bl);
  hi = ah; lo = al; pair_max(hi, lo, bh, bl);
}

// Each wavefront routes `tpw` consecutive tokens, one at a time, with the next token's scores
// loaded while the current one is processed. Lane l holds experts l, l + 64, l + 128, l + 192.
template <int MODE>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int T, int E, int K, int tpw, uint32_t flags, const float* __restrict__ sel_bias,
    const float* __restrict__ logits, float* __restrict__ probs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const bool norm = (flags & MOE_NORM_TOPK) != 0;
  const float* src = MODE == kFromLogits ? logits : probs;
  float bias[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    bias[s] = (e < E && sel_bias) ? sel_bias[e] : 0.0f;
  }
  const int tb = (blockIdx.x * (kRouteThreads / 64) + wave) * tpw;
  const int tn = min(T, tb + tpw);
  auto load = [&](int t, float (&z)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      z[s] = (t < tn && e < E) ? src[(int64_t)t * E + e] : 0.0f;
    }
  };
  float nxt[4];
  load(tb, nxt);
  for (int t = tb; t < tn; ++t) {
    float p[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) p[s] = nxt[s];
    load(t + 1, nxt);
    if (MODE == kFromLogits) {
      float m = -INFINITY;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (lane + 64 * s < E) m = fmaxf(m, p[s]);
      m = wave_reduce(m, [](float a, float b) { return fmaxf(a, b); });
      float sum = 0.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        p[s] = lane + 64 * s < E ? expf(p[s] - m) : 0.0f;
        sum += p[s];
      }
      sum = wave_reduce(sum, [](float a, float b) { return a + b; });
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
        // A lane without a candidate offers (0, 0), which loses to every real expert, NaN keys
        // (code 0) included.
        uint32_t hi = bc, lo = ~bi;
        wave_argmax(hi, lo);
        const int e = __builtin_amdgcn_readfirstlane((int)(~lo));
        if ((e & 63) == lane) taken |= 1u << (e >> 6);
        const int s = e >> 6;
        const float pv = s == 0 ? p[0] : s == 1 ? p[1] : s == 2 ? p[2] : p[3];
        const float pe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pv), e & 63));
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
    }
  }
}

// ---- 3. expert counts ---------------------------------------------------------------------------
// counts[e] = number of (token, slot) pairs routed to e. Workgroup (g, c) counts experts
// 16 g .. 16 g + 15 over chunk c of topk_idx (2048 entries, 8 per lane, read as two 16-byte
// loads in flight together): each lane keeps 16 counters, the workgroup sums them, and one integer
// atomic per expert and chunk adds the result (a few dozen per address, where an atomic per expert
// from every routing workgroup piled up on the busiest experts). Integer sums do not depend on
// order, so the counts are exact and deterministic.
constexpr int kCntExperts = 16;
constexpr int kCntThreads = 256;
constexpr int kCntPer = 8;                                      // entries per lane
constexpr int64_t kCntChunk = (int64_t)kCntThreads * kCntPer;   // entries per workgroup

// STORE: a single chunk (one workgroup row): its sums are the counts, stored without a prior
// clear; otherwise each chunk adds its sums to counts, which must start at zero.
template <bool STORE>
__global__ __launch_bounds__(kCntThreads) void count_kernel(int64_t n, int E,
                                                            const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ counts) {
  __shared__ int part[kCntThreads / 64][kCntExperts];
  const int e0 = blockIdx.x * kCntExperts;
  const int64_t i0 = (int64_t)blockIdx.y * kCntChunk + (int64_t)threadIdx.x * kCntPer;
  int v[kCntPer];
  if (i0 + kCntPer <= n && (((uintptr_t)(idx + i0)) & 15) == 0) {
    const int4 a = *reinterpret_cast<const int4*>(idx + i0);
    const int4 b = *reinterpret_cast<const int4*>(idx + i0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int u = 0; u < kCntPer; ++u) v[u] = i0 + u < n ? idx[i0 + u] : -1;
  }
  int c[kCntExperts];
#pragma unroll
  for (int j = 0; j < kCntExperts; ++j) c[j] = 0;
#pragma unroll
  for (int u = 0; u < kCntPer; ++u) {
    const int d = v[u] - e0;
#pragma unroll
    for (int j = 0; j < kCntExperts; ++j) c[j] += d == j;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kCntExperts; ++j) {
    int x = c[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    if (lane == 0) part[wave][j] = x;
  }
  __syncthreads();
  if (threadIdx.x < kCntExperts && e0 + (int)threadIdx.x < E) {
    int x = 0;
#pragma unroll
    for (int w = 0; w < kCntThreads / 64; ++w) x += part[w][threadIdx.x];
    if constexpr (STORE) counts[e0 + threadIdx.x] = x;
    else if (x) atomicAdd(&counts[e0 + threadIdx.x], x);
  }
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

namespace {
// One chunk of routed slots (decode-sized batches) is counted and stored by one row of
// workgroups; more are added up, into counts cleared before the routing kernels ran.
bool counts_single_chunk(const moe_shape_t& s) { return (int64_t)s.T * s.K <= kCntChunk; }

hipError_t launch_counts(const moe_shape_t& s, const int32_t* topk_idx, int32_t* counts,
                         hipStream_t st) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !counts) return e;
  const int64_t n = (int64_t)s.T * s.K;
  const dim3 grid((unsigned)((s.E + kCntExperts - 1) / kCntExperts),
                  (unsigned)((n + kCntChunk - 1) / kCntChunk));
  if (counts_single_chunk(s))
    hipLaunchKernelGGL(count_kernel<true>, grid, dim3(kCntThreads), 0, st, n, s.E, topk_idx, counts);
  else
    hipLaunchKernelGGL(count_kernel<false>, grid, dim3(kCntThreads), 0, st, n, s.E, topk_idx, counts);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_route(const moe_shape_t& s, const uint16_t* x, const float* wg,
                        const float* logit_bias, const float* sel_bias, float* logits,
                        float* probs, int32_t* topk_idx, float* topk_w, int32_t* counts,
                        hipStream_t st) {
  if (counts && !counts_single_chunk(s)) {
    hipError_t e = launch_fill_i32(counts, 0, s.E, st);
    if (e != hipSuccess) return e;
  }
  // About 2048 wavefronts (8 per CU) with whole tokens each; at most 512 workgroups, so the
  // per-workgroup count merges stay few.
  const int tpw = (int)((s.T + kRouteWaves - 1) / kRouteWaves);   // T >= 1 here
  const int toks_per_wg = tpw * (kRouteThreads / 64);
  const dim3 grid((unsigned)((s.T + toks_per_wg - 1) / toks_per_wg)), block(kRouteThreads);
  if (s.flags & MOE_PROBS_IN) {
    hipLaunchKernelGGL(route_kernel<kFromProbs>, grid, block, 0, st, s.T, s.E, s.K, tpw, s.flags,
                       sel_bias, logits, probs, topk_idx, topk_w);
    return launch_counts(s, topk_idx, counts, st);
  }
  if (x) {
    const unsigned ge = (unsigned)((s.E + kLgTile - 1) / kLgTile);
    if (s.T >= kLgDmaMinT && s.E <= 128)
      hipLaunchKernelGGL((router_logits_dma_kernel<1>), dim3((unsigned)((s.T + kLgDmaTok - 1) / kLgDmaTok)),
                         dim3(kLgDmaThreads), 0, st, s.T, s.H, s.E, x, wg, logit_bias, logits);
    else if (s.T >= kLgDmaMinT)
      hipLaunchKernelGGL((router_logits_dma_kernel<2>), dim3((unsigned)((s.T + kLgDmaTok - 1) / kLgDmaTok)),
                         dim3(kLgDmaThreads), 0, st, s.T, s.H, s.E, x, wg, logit_bias, logits);
    else if (s.T >= 4 * kLgLargeT)
      hipLaunchKernelGGL((router_logits_kernel<4, 4>), dim3((unsigned)((s.T + 127) / 128), ge), dim3(256),
                         0, st, s.T, s.H, s.E, x, wg, logit_bias, logits);
    else if (s.T >= kLgLargeT)
      hipLaunchKernelGGL((router_logits_kernel<2, 4>), dim3((unsigned)((s.T + 63) / 64), ge), dim3(256),
                         0, st, s.T, s.H, s.E, x, wg, logit_bias, logits);
    else
      hipLaunchKernelGGL((router_logits_kernel<1, 8>), dim3((unsigned)((s.T + 31) / 32), ge),
                         dim3(512), 0, st, s.T, s.H, s.E, x, wg, logit_bias, logits);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(route_kernel<kFromLogits>, grid, block, 0, st, s.T, s.E, s.K, tpw, s.flags,
                     sel_bias, logits, probs, topk_idx, topk_w);
  return launch_counts(s, topk_idx, counts, st);
}

}  // namespace moe
