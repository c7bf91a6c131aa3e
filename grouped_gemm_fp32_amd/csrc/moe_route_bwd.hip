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
//   router_dwg_kernel   dWg[E,H] = dlogits^T x, a contraction over the tokens on the bf16 matrix
//                       unit with dlogits split exactly into three bf16 parts (exact products,
//                       fp32 sums): one workgroup per 32 x 64 tile of dWg, its eight wavefronts
//                       take an eighth of the tokens each and their partial sums are added in
//                       wavefront order (deterministic).
//   router_dx_kernel    dx_router[T,H] = dlogits Wg, an fp32 contraction over the experts on the
//                       fp32 matrix unit (v_mfma_f32_32x32x2_f32): a 64-token tile of dlogits in
//                       LDS, Wg read from L2.
//   balance_hist_kernel, balance_kernel, balance_reduce_kernel
//                       per-chunk selection counts, then the sequence-wise balance loss (per sequence alpha sum_e f_e P_e, f the
//                       normalised selection counts, P the mean probabilities) as per-chunk
//                       partial sums reduced in a fixed order, and its gradient, added to dlogits:
//                       p_e (g_e - sum_i p_i g_i) with g = alpha f / (seq_len n_seq).
//   bias_update_kernel  b_e += gamma * sign(T K - E c_e), one fp32 add per expert.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 2048;   // target wavefront count of the per-token kernel

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
// On the bf16 matrix unit: each fp32 dlogits value is split exactly into three bf16 parts
// (hi + mid + lo, split3), and x is bf16, so every product is exact in fp32. The three parts' sums
// are kept in separate accumulators and added as (lo + mid) + hi at the end: the fp32 contraction
// up to summation order, with no more roundings per element than one fp32 sum over the tokens.
// v_mfma_f32_32x32x16_bf16: lane l supplies A[l % 32][8 (l / 32) .. +7] and B[8 (l / 32) .. +7]
// [l % 32]; D[i][j] sits in lane j (+32 for rows 4..7 of each group of 8), register q -> row
// 8 (q / 4) + 4 (l / 32) + q % 4.
// A workgroup of eight wavefronts covers a 32 x 64 tile of dWg. Wavefront w takes the w-th eighth
// of the 16-token slices. Per slice each lane loads 16 bytes of dlogits (4 experts of one token)
// and 16 bytes of x; the dlogits values are split in registers, and the three bf16 parts and x go
// through the wavefront's own LDS tiles [16 tokens][columns] to come back transposed
// (ds_read_tr16_b64) as the A operand (32 experts) and the B operands (two 32-column blocks). The
// next slices' operands load during the current ones' MFMAs. The wavefronts' partial sums are
// added in wavefront order (deterministic).
constexpr int kDwgThreads = 512;
constexpr int kDwgSlices = 4;        // 16-token slices per batch
// LDS bytes per token row: 64 for a 32-expert bf16 part, 192 for the 64-column x tile (128 used).
// With row strides of 16 or 48 banks the 16 lanes of a transposed read hit distinct banks.
constexpr int kDwgARow = 64, kDwgXRow = 192;
constexpr int kDwgWaveLds = 3 * 16 * kDwgARow + 16 * kDwgXRow;   // 3 KiB of parts + 3 KiB of x
typedef short dwg_v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dwg_v4i16_t dwg_lds_v4i16_t;

// Operand of the 32 columns col0.. of a [16 tokens][columns] bf16 tile with ROW bytes per token:
// within 16 lanes, lane i reads 4 columns of token row (i / 4) and the transposing read hands it
// column col0 + i of 4 consecutive tokens; two reads give 8 (lanes 32-63: tokens 8-15).
template <int ROW>
__device__ __forceinline__ bf16x8_t dwg_frag(const unsigned char* tile, int col0, int lane) {
  const int grp = lane >> 4, li = lane & 15;
  const int col = col0 + (grp & 1) * 16 + 4 * (li & 3);
  const int k0 = (grp >> 1) * 8 + (li >> 2);
  const unsigned char* p0 = tile + k0 * ROW + col * 2;
  const dwg_v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dwg_lds_v4i16_t*)p0);
  const dwg_v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((dwg_lds_v4i16_t*)(p0 + 4 * ROW));
  bf16x8_t r;
  __builtin_memcpy(&r, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi, 8);
  return r;
}

__device__ __forceinline__ uint32_t bf_pair(__bf16 a, __bf16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// VEC: dlogits rows are 16-byte aligned (E % 4 == 0 and an aligned base): one float4 per chunk.
template <bool VEC>
__global__ __launch_bounds__(kDwgThreads) void router_dwg_kernel(int T, int H, int E,
                                                                 const float* __restrict__ dz,
                                                                 const uint16_t* __restrict__ x,
                                                                 float* __restrict__ dwg) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[8][kDwgWaveLds];
  __shared__ float red[8][32][65];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * 32, h0 = blockIdx.y * 64;
  const int r = lane & 31, kh = lane >> 5;
  const int nsl = (T + 15) / 16;
  const int per = (nsl + 7) / 8;
  const int sa = min(nsl, wave * per), sz = min(nsl, sa + per);   // this wave's slices
  unsigned char* ap = lds[wave];                    // parts hi, mid, lo: [16][32] bf16 each
  unsigned char* xt = lds[wave] + 3 * 16 * kDwgARow; // x: [16][64] bf16
  // A lane's chunks of a slice (two of each): dlogits token row (lane >> 3) (+8), experts
  // e0 + 4 (lane & 7) .. +3; x token row (lane >> 3) (+8), columns h0 + 8 (lane & 7) .. +7.
  const int cr = lane >> 3, ce = 4 * (lane & 7), cx = 8 * (lane & 7);
  struct Ops {
    float4 a[kDwgSlices][2];
    uint4 b[kDwgSlices][2];
  };
  auto load = [&](int s0, Ops& o) {
#pragma unroll
    for (int j = 0; j < kDwgSlices; ++j) {
      const int s = s0 + j;
      const bool live = s < sz;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = s * 16 + cr + 8 * i;
        const bool tok = live && t < T;
        const float* row = dz + (int64_t)t * E + e0 + ce;
        if (VEC) {
          o.a[j][i] = (tok && e0 + ce < E) ? *reinterpret_cast<const float4*>(row)
                                            : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        } else {
          const int n = E - (e0 + ce);   // experts of this chunk inside E
          o.a[j][i] = make_float4(tok && n > 0 ? row[0] : 0.0f, tok && n > 1 ? row[1] : 0.0f,
                                  tok && n > 2 ? row[2] : 0.0f, tok && n > 3 ? row[3] : 0.0f);
        }
        o.b[j][i] = tok ? *reinterpret_cast<const uint4*>(x + (int64_t)t * H + h0 + cx)
                        : make_uint4(0, 0, 0, 0);
      }
    }
  };
  f32x16_t acc[3][2];   // [part: hi, mid, lo][32-column block]
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[p][jb][q] = 0.0f;
  Ops cur;
  load(sa, cur);
  for (int s0 = sa; s0 < sz; s0 += kDwgSlices) {
    Ops nxt;
    load(s0 + kDwgSlices, nxt);   // past this wave's slices: zeros, no memory access
#pragma unroll
    for (int j = 0; j < kDwgSlices; ++j) {
      // This wavefront's tiles: its LDS operations run in order, so the transposed reads below
      // see these writes, and the next slice's writes come after these reads.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float4 v = cur.a[j][i];
        bf16x8_t hi, mid, lo;   // elements 0..3 used
        split3(v, make_float4(0.0f, 0.0f, 0.0f, 0.0f), hi, mid, lo);
        const int off = (cr + 8 * i) * kDwgARow + ce * 2;
        *reinterpret_cast<uint2*>(ap + off) = make_uint2(bf_pair(hi[0], hi[1]), bf_pair(hi[2], hi[3]));
        *reinterpret_cast<uint2*>(ap + 16 * kDwgARow + off) =
            make_uint2(bf_pair(mid[0], mid[1]), bf_pair(mid[2], mid[3]));
        *reinterpret_cast<uint2*>(ap + 32 * kDwgARow + off) =
            make_uint2(bf_pair(lo[0], lo[1]), bf_pair(lo[2], lo[3]));
        *reinterpret_cast<uint4*>(xt + (cr + 8 * i) * kDwgXRow + cx * 2) = cur.b[j][i];
      }
      const bf16x8_t b0 = dwg_frag<kDwgXRow>(xt, 0, lane), b1 = dwg_frag<kDwgXRow>(xt, 32, lane);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8_t a = dwg_frag<kDwgARow>(ap + p * 16 * kDwgARow, 0, lane);
        acc[p][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b0, acc[p][0], 0, 0, 0);
        acc[p][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b1, acc[p][1], 0, 0, 0);
      }
    }
    cur = nxt;
  }
  // D[e][h]: lane -> column r of each 32-column block, register q -> e = e0 + 8 (q / 4) + 4 kh + q % 4
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int el = 8 * (q >> 2) + 4 * kh + (q & 3);
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      red[wave][el][32 * jb + r] = (acc[2][jb][q] + acc[1][jb][q]) + acc[0][jb][q];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 32 * 64; idx += kDwgThreads) {
    const int el = idx / 64, hl = idx % 64;
    if (e0 + el < E) {
      float v = red[0][el][hl];
#pragma unroll
      for (int w = 1; w < 8; ++w) v += red[w][el][hl];
      dwg[(int64_t)(e0 + el) * H + h0 + hl] = v;
    }
  }
}

// ---- dx_router = dlogits Wg ---------------------------------------------------------------------
// A workgroup of eight wavefronts covers 64 tokens x 256 columns (one dlogits tile in LDS for all
// of them); each wavefront 64 tokens x 32 columns (two MFMA blocks sharing every Wg operand), with
// the Wg loads of the next batch of experts in flight. Wavefronts past the last column only help
// load the tile.
constexpr int kDxTok = 64;
constexpr int kDxThreads = 512;
constexpr int kDxCols = 32 * (kDxThreads / 64);   // columns per workgroup
constexpr int kDxUnroll = 16;  // expert pairs per batch

__global__ __launch_bounds__(kDxThreads) void router_dx_kernel(int T, int H, int E,
                                                             const float* __restrict__ dz,
                                                             const float* __restrict__ wg,
                                                             float* __restrict__ dx) {
  extern __shared__ float tile[];   // [kDxTok][E + 1], sized at launch
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kDxTok, h0 = blockIdx.y * kDxCols + wave * 32;
  const int nt = min(kDxTok, T - t0);
  const int ld = E + 1;
  // wavefront w fills rows w, w + 8, ...; a row's experts go across the lanes (coalesced)
#pragma unroll 4
  for (int tl = wave; tl < kDxTok; tl += kDxThreads / 64)
    for (int e = lane; e < E; e += 64)
      tile[tl * ld + e] = tl < nt ? dz[(int64_t)(t0 + tl) * E + e] : 0.0f;
  __syncthreads();
  if (h0 >= H) return;   // no barrier follows
  const int r = lane & 31, kh = lane >> 5;
  auto load = [&](int e0, float (&b)[kDxUnroll]) {
#pragma unroll
    for (int u = 0; u < kDxUnroll; ++u) {
      const int e = e0 + 2 * u + kh;
      b[u] = e < E ? wg[(int64_t)e * H + h0 + r] : 0.0f;
    }
  };
  f32x16_t acc0, acc1;
#pragma unroll
  for (int q = 0; q < 16; ++q) { acc0[q] = 0.0f; acc1[q] = 0.0f; }
  // D[t][h] = sum_e A[t][e] B[e][h]: A from the LDS tile, B = Wg rows (128 contiguous bytes)
  float b[kDxUnroll];
  load(0, b);
  for (int e0 = 0; e0 < E; e0 += 2 * kDxUnroll) {
    float bn[kDxUnroll];
    load(e0 + 2 * kDxUnroll, bn);   // past E: zeros, no memory access
#pragma unroll
    for (int u = 0; u < kDxUnroll; ++u) {
      const int e = e0 + 2 * u + kh;
      const float a0 = e < E ? tile[r * ld + e] : 0.0f;
      const float a1 = e < E ? tile[(32 + r) * ld + e] : 0.0f;
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b[u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b[u], acc1, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kDxUnroll; ++u) b[u] = bn[u];
  }
  // lane -> h = h0 + r, register q -> t = t0 + 8 (q / 4) + 4 kh + q % 4 (+32 for the second block)
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int tl = 8 * (q >> 2) + 4 * kh + (q & 3);
    if (tl < nt) dx[(int64_t)(t0 + tl) * H + h0 + r] = acc0[q];
    if (tl + 32 < nt) dx[(int64_t)(t0 + tl + 32) * H + h0 + r] = acc1[q];
  }
}

// ---- sequence-wise balance loss ---------------------------------------------------------------------
// Per sequence of seq_len consecutive tokens: f_e = E / (K seq_len) * (selections of e), P_e = mean
// of p[t, e], loss = alpha sum_e f_e P_e; the batch loss is the mean over the n_seq sequences.
constexpr int kBalTok = 256;       // tokens per workgroup
constexpr int kBalThreads = 1024;  // balance_kernel: 16 wavefronts, 16 tokens each

// Selection counts of chunk c of sequence q (its kBalTok tokens): hc[(q * n_chunk + c) * E + e].
// Entries outside 0..E-1 are not counted.
__global__ __launch_bounds__(kThreads) void balance_hist_kernel(int seq_len, int E, int K,
                                                                const int32_t* __restrict__ topk_idx,
                                                                int32_t* __restrict__ hc) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int q = blockIdx.y, c = blockIdx.x;
  const int t0 = c * kBalTok, t1 = min(seq_len, t0 + kBalTok);
  const int64_t base = ((int64_t)q * seq_len + t0) * K;
  for (int i = threadIdx.x; i < (t1 - t0) * K; i += kThreads) {
    const int e = topk_idx[base + i];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);   // integer adds: order-free
  }
  __syncthreads();
  int32_t* out = hc + ((int64_t)q * gridDim.x + c) * E;
  for (int e = threadIdx.x; e < E; e += kThreads) out[e] = hist[e];
}

// Workgroup (chunk, q) covers kBalTok tokens of sequence q, one wavefront per token. With f the
// sequence's normalised counts, L_seq = alpha sum_e f_e P_e = (alpha / seq_len) sum_t <f, p_t>:
// each token's <f, p_t> goes into the workgroup's partial sum (wavefront order, then token order
// within a wavefront), written to part[q * n_chunk + chunk]. With dlogits, the gradient of the
// mean loss is added: g = alpha f / (seq_len n_seq), dlogits[t, e] += p_e (g_e - <p_t, g>).
__global__ __launch_bounds__(kBalThreads) void balance_kernel(int seq_len, int n_seq, int E, int K,
                                                           float alpha,
                                                           const float* __restrict__ probs,
                                                           const int32_t* __restrict__ hc,
                                                           float* __restrict__ dlogits,
                                                           float* __restrict__ part) {
  __shared__ int hist[256];
  __shared__ float wpart[kBalThreads / 64];
  const int q = blockIdx.y;
  for (int e = threadIdx.x; e < E; e += kBalThreads) hist[e] = 0;
  __syncthreads();
  // the sequence's counts from its chunks' (integer adds: order-free)
  const int64_t hbase = (int64_t)q * gridDim.x * E;
  for (int i = threadIdx.x; i < (int)gridDim.x * E; i += kBalThreads)
    atomicAdd(&hist[i % E], hc[hbase + i]);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float fs = (float)E / (float)(K * seq_len);               // f_e = fs * count_e
  const float gs = alpha / ((float)seq_len * (float)n_seq);        // g_e = gs * f_e
  float f[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    f[s] = e < E ? fs * (float)hist[e] : 0.0f;
  }
  float acc = 0.0f;
  const int t_end = min(seq_len, (blockIdx.x + 1) * kBalTok);
  for (int tl = blockIdx.x * kBalTok + wave; tl < t_end; tl += kBalThreads / 64) {
    const int64_t t = (int64_t)q * seq_len + tl;
    float p[4], dot = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      p[s] = e < E ? probs[t * E + e] : 0.0f;
      dot += p[s] * f[s];
    }
    dot = wave_sum(dot);   // <f, p_t>, the same on every lane
    acc += dot;
    if (dlogits) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        if (e < E) dlogits[t * E + e] += p[s] * (gs * f[s] - gs * dot);
      }
    }
  }
  if (lane == 0) wpart[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.0f;
    for (int w = 0; w < kBalThreads / 64; ++w) v += wpart[w];
    part[(int64_t)q * gridDim.x + blockIdx.x] = v;
  }
}

// seq_loss[q] = alpha / seq_len * (sum of sequence q's partials, in chunk order).
__global__ void balance_reduce_kernel(int n_chunk, int seq_len, float alpha,
                                      const float* __restrict__ part, float* __restrict__ seq_loss) {
  const int q = blockIdx.x;
  if (threadIdx.x != 0) return;
  float v = 0.0f;
  for (int c = 0; c < n_chunk; ++c) v += part[(int64_t)q * n_chunk + c];
  seq_loss[q] = alpha * (v / (float)seq_len);
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
  if (s.T == 0) return launch_router_grads(s, dlogits, x, wg, dw_gate, dx_router, st);
  const int tpw = (s.T + kWaves - 1) / kWaves;
  const int per_wg = tpw * (kThreads / 64);
  const dim3 grid((unsigned)((s.T + per_wg - 1) / per_wg));
  if (norm)
    hipLaunchKernelGGL(route_bwd_kernel<true>, grid, dim3(kThreads), 0, st, s.T, s.E, s.K, tpw,
                       dtopk_w, topk_idx, probs, dlogits);
  else
    hipLaunchKernelGGL(route_bwd_kernel<false>, grid, dim3(kThreads), 0, st, s.T, s.E, s.K, tpw,
                       dtopk_w, topk_idx, probs, dlogits);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_router_grads(s, dlogits, x, wg, dw_gate, dx_router, st);
}

hipError_t launch_router_grads(const moe_shape_t& s, const float* dlogits, const uint16_t* x,
                               const float* wg, float* dw_gate, float* dx_router, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (s.T == 0) {   // an empty batch: the weight gradient is a sum over no tokens
    if (dw_gate) {
      const int64_t n = (int64_t)s.E * s.H;
      hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                         dw_gate, n);
      e = hipGetLastError();
    }
    return e;
  }
  if (dw_gate) {
    const dim3 grid((unsigned)((s.E + 31) / 32), (unsigned)(s.H / 64));
    if (s.E % 4 == 0 && (uintptr_t)dlogits % 16 == 0)
      hipLaunchKernelGGL(router_dwg_kernel<true>, grid, dim3(kDwgThreads), 0, st, s.T, s.H, s.E,
                         dlogits, x, dw_gate);
    else
      hipLaunchKernelGGL(router_dwg_kernel<false>, grid, dim3(kDwgThreads), 0, st, s.T, s.H, s.E,
                         dlogits, x, dw_gate);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dx_router) {
    const size_t lds = sizeof(float) * kDxTok * (s.E + 1);   // at most 64 KiB + 256 B (E <= 256)
    if (lds > 65536) {
      e = hipFuncSetAttribute((const void*)router_dx_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(router_dx_kernel,
                       dim3((unsigned)((s.T + kDxTok - 1) / kDxTok), (unsigned)((s.H + kDxCols - 1) / kDxCols)),
                       dim3(kDxThreads), lds, st, s.T, s.H, s.E, dlogits, wg, dx_router);
    e = hipGetLastError();
  }
  return e;
}

int64_t balance_workspace_floats(int T, int seq_len, int E) {
  if (seq_len < 1) return 0;
  // per chunk of each sequence: one partial loss and E selection counts
  return (int64_t)(T / seq_len) * ((seq_len + kBalTok - 1) / kBalTok) * (1 + E);
}

hipError_t launch_balance_loss(const moe_shape_t& s, int seq_len, float alpha, const float* probs,
                               const int32_t* topk_idx, float* seq_loss, float* dlogits, float* ws,
                               hipStream_t st) {
  const int n_seq = s.T / seq_len;
  if (n_seq == 0) return hipSuccess;
  const int n_chunk = (seq_len + kBalTok - 1) / kBalTok;
  float* part = ws;
  int32_t* hc = reinterpret_cast<int32_t*>(ws + (int64_t)n_seq * n_chunk);
  const dim3 grid((unsigned)n_chunk, (unsigned)n_seq);
  hipLaunchKernelGGL(balance_hist_kernel, grid, dim3(kThreads), 0, st, seq_len, s.E, s.K, topk_idx,
                     hc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(balance_kernel, grid, dim3(kBalThreads), 0, st, seq_len, n_seq, s.E, s.K, alpha,
                     probs, hc, dlogits, part);
  e = hipGetLastError();
  if (e != hipSuccess || !seq_loss) return e;
  hipLaunchKernelGGL(balance_reduce_kernel, dim3((unsigned)n_seq), dim3(64), 0, st, n_chunk,
                     seq_len, alpha, part, seq_loss);
  return hipGetLastError();
}

hipError_t launch_bias_update(const moe_shape_t& s, const int32_t* counts, float gamma, float* bias,
                              hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((unsigned)((s.E + 255) / 256)), dim3(256), 0, st, s.E,
                     (int64_t)s.T * s.K, gamma, counts, bias);
  return hipGetLastError();
}

}  // namespace moe
