// Block-aligned expert segments and the token permutation on gfx950.
//
// dots.llm1 Technical Report, section 3.2 "Efficient grouped GEMM": each expert's token segment is
// padded to a fixed block size (a multiple of the matrix instruction's M), so a workgroup's rows
// always belong to a single expert. Section A2, load-balancing paragraph: no token is dropped, so
// the row capacity covers every routing.
//
// Deterministic and atomic-free in its outputs (integer LDS atomics only build bit masks and
// histograms, whose results do not depend on order):
//   1. hist:    per token block, per-expert counts                        -> ws[nblk][E]
//   2. segment: one workgroup scans ws per expert (block bases, counts), pads and prefix-sums the
//               group sizes (seg_offsets, total_rows) and fills tile_group
//      clear:   row_token = -1 on every row below total_rows (grid-wide)
//   3. scatter: per token block, a [E][TB/32] bit mask of "token routed to e" gives each slot its
//               stable rank (popcounts), hence pos[t,j] and row_token
//   4. gather:  x_perm[r] = x[row_token[r]] or 0, 16-byte vector copies, rows < total_rows.
// A batch of one token block (at most 256 tokens: decode) runs steps 1-3 in a single workgroup
// (perm_small_kernel): the block bases are all zero, so it needs no workspace and saves three
// launches.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

int permute_token_block(int T) {
  // Keep the number of token blocks <= 128 so the segment builder's table fits in LDS.
  const int nb256 = (T + 255) / 256;
  const int mult = (nb256 + 127) / 128;
  return 256 * (mult < 1 ? 1 : mult);
}

int64_t permute_num_blocks(int T) {
  const int tb = permute_token_block(T);
  return (T + tb - 1) / tb;
}

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void perm_hist_kernel(int T, int K, int E, int TB,
                                                             const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ ws) {
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * TB;
  const int t1 = min(T, t0 + TB);
  for (int t = t0 + tid; t < t1; t += kThreads)
    for (int j = 0; j < K; ++j) {
      const int e = idx[(int64_t)t * K + j];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) ws[(int64_t)blockIdx.x * E + e] = hist[e];
}

constexpr int kSegThreads = 1024;

__global__ __launch_bounds__(kSegThreads) void perm_segment_kernel(
    int T, int E, int S, int B, int nblk, int64_t mcap, int32_t* __restrict__ ws,
    int32_t* __restrict__ seg_offsets, int32_t* __restrict__ tile_group,
    int32_t* __restrict__ total_rows, int32_t* __restrict__ row_token) {
  extern __shared__ int smem[];
  int* tab = smem;                        // [nblk][E]
  int* seg = smem + nblk * E;             // [G+1]
  int* cnt = seg + (E + S + 1);           // [E]
  const int tid = threadIdx.x;
  const int G = E + S;
  for (int i = tid; i < nblk * E; i += kSegThreads) tab[i] = ws[i];
  __syncthreads();
  // Per expert: exclusive scan over token blocks (block base of each block) and total count.
  for (int e = tid; e < E; e += kSegThreads) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int v = tab[b * E + e];
      tab[b * E + e] = run;
      run += v;
    }
    cnt[e] = run;
  }
  __syncthreads();
  // Padded group sizes, exclusive prefix sum by the first wavefront, 64 groups per step (shared
  // groups last, T rows each).
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + tid;
      const int c = g < E ? cnt[g] : T;
      const int padded = g < G ? (c + B - 1) / B * B : 0;
      int x = padded;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (tid >= o) x += y;
      }
      if (g < G) seg[g] = run + x - padded;
      run += __shfl(x, 63, 64);
    }
    if (tid == 0) {
      seg[G] = run;
      total_rows[0] = run;
    }
  }
  __syncthreads();
  for (int i = tid; i < nblk * E; i += kSegThreads) ws[i] = tab[i];
  for (int g = tid; g <= G; g += kSegThreads) seg_offsets[g] = seg[g];
  // tile_group: binary search for the group whose segment holds row i*B.
  const int64_t nt = mcap / B;
  const int total = seg[G];
  for (int64_t i = tid; i < nt; i += kSegThreads) {
    const int64_t r = i * B;
    int g = -1;
    if (r < total) {
      int lo = 0, hi = G - 1;  // largest g with seg[g] <= r and a non-empty segment
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid] <= r) lo = mid; else hi = mid - 1;
      }
      g = lo;
    }
    tile_group[i] = g;
  }
}

// Every row below total_rows starts as padding (-1); the scatter then writes the token of each
// routed and shared row. With valid routing that leaves -1 exactly on the padding rows; with
// out-of-range or repeated expert indices (which the contract excludes) a row no slot claims
// stays -1 instead of holding whatever the buffer held. Rows from total_rows on are not written.
__global__ __launch_bounds__(kThreads) void perm_clear_rows_kernel(int64_t mcap,
                                                                   const int32_t* __restrict__ total,
                                                                   int32_t* __restrict__ row_token) {
  const int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (r < mcap && r < total[0]) row_token[r] = -1;
}

__global__ __launch_bounds__(kThreads) void perm_scatter_kernel(
    int T, int K, int E, int S, int TB, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ base, const int32_t* __restrict__ seg_offsets,
    int32_t* __restrict__ pos, int32_t* __restrict__ row_token) {
  extern __shared__ uint32_t sm[];
  const int W = TB / 32;             // mask words per expert
  uint32_t* mask = sm;               // [E][W]
  int* pref = (int*)(sm + E * W);    // [E][W]: set bits in earlier words
  int* segs = pref + E * W;          // [E]
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int t0 = blk * TB;
  const int t1 = min(T, t0 + TB);
  for (int i = tid; i < E * W; i += kThreads) mask[i] = 0u;
  for (int e = tid; e < E; e += kThreads) segs[e] = seg_offsets[e] + base[(int64_t)blk * E + e];
  __syncthreads();
  for (int t = t0 + tid; t < t1; t += kThreads) {
    const int tl = t - t0;
    for (int j = 0; j < K; ++j) {
      const int e = idx[(int64_t)t * K + j];
      if (e >= 0 && e < E) atomicOr(&mask[e * W + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      pref[e * W + w] = run;
      run += __popc(mask[e * W + w]);
    }
  }
  __syncthreads();
  for (int t = t0 + tid; t < t1; t += kThreads) {
    const int tl = t - t0;
    for (int j = 0; j < K; ++j) {
      const int e = idx[(int64_t)t * K + j];
      if (e < 0 || e >= E) {   // out of range (excluded by the contract): no row, pos = -1
        pos[(int64_t)t * K + j] = -1;
        continue;
      }
      const int w = tl >> 5;
      const int rank = pref[e * W + w] + __popc(mask[e * W + w] & ((1u << (tl & 31)) - 1u));
      const int r = segs[e] + rank;
      pos[(int64_t)t * K + j] = r;
      row_token[r] = t;
    }
    for (int s = 0; s < S; ++s) row_token[seg_offsets[E + s] + t] = t;
  }
}

// Steps 1-3 for a batch of one token block (T <= 256), in one workgroup, with the same results as
// the three kernels above: per-expert slot counts (every slot counted, as perm_hist_kernel does),
// the padded prefix sum, tile_group, the padding rows cleared, then each slot's stable rank from
// the [E][8] bit mask of its expert's tokens.
constexpr int kSmallPermThreads = 1024;
constexpr int kSmallPermT = 256;

__global__ __launch_bounds__(kSmallPermThreads) void perm_small_kernel(
    int T, int K, int E, int S, int B, int64_t mcap, const int32_t* __restrict__ idx,
    int32_t* __restrict__ seg_offsets, int32_t* __restrict__ tile_group,
    int32_t* __restrict__ total_rows, int32_t* __restrict__ row_token, int32_t* __restrict__ pos) {
  constexpr int W = kSmallPermT / 32;   // mask words per expert
  __shared__ int cnt[256];              // E <= 256
  __shared__ int seg[256 + 4 + 1];      // G + 1 <= 261
  __shared__ uint32_t mask[256 * W];
  __shared__ int pref[256 * W];
  const int tid = threadIdx.x;
  const int G = E + S, n = T * K;
  for (int i = tid; i < E * W; i += kSmallPermThreads) mask[i] = 0u;
  for (int e = tid; e < E; e += kSmallPermThreads) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kSmallPermThreads) {
    const int t = i / K, e = idx[i];
    if (e >= 0 && e < E) {
      atomicAdd(&cnt[e], 1);
      atomicOr(&mask[e * W + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kSmallPermThreads) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      pref[e * W + w] = run;
      run += __popc(mask[e * W + w]);
    }
  }
  // padded group sizes, exclusive prefix sum by the first wavefront (shared groups last, T rows)
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + tid;
      const int c = g < E ? cnt[g] : T;
      const int padded = g < G ? (c + B - 1) / B * B : 0;
      int x = padded;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (tid >= o) x += y;
      }
      if (g < G) seg[g] = run + x - padded;
      run += __shfl(x, 63, 64);
    }
    if (tid == 0) {
      seg[G] = run;
      total_rows[0] = run;
    }
  }
  __syncthreads();
  const int total = seg[G];
  for (int g = tid; g <= G; g += kSmallPermThreads) seg_offsets[g] = seg[g];
  const int64_t nt = mcap / B;
  for (int64_t i = tid; i < nt; i += kSmallPermThreads) {
    const int64_t r = i * B;
    int g = -1;
    if (r < total) {
      int lo = 0, hi = G - 1;   // largest g with seg[g] <= r
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid] <= r) lo = mid; else hi = mid - 1;
      }
      g = lo;
    }
    tile_group[i] = g;
  }
  for (int64_t r = tid; r < mcap && r < total; r += kSmallPermThreads) row_token[r] = -1;
  __syncthreads();   // the clears are ordered before the scatter's writes of the same rows
  for (int i = tid; i < n; i += kSmallPermThreads) {
    const int t = i / K, e = idx[i];
    if (e < 0 || e >= E) {   // out of range (excluded by the contract): no row, pos = -1
      pos[i] = -1;
      continue;
    }
    const int w = t >> 5;
    const int r = seg[e] + pref[e * W + w] + __popc(mask[e * W + w] & ((1u << (t & 31)) - 1u));
    pos[i] = r;
    row_token[r] = t;
  }
  for (int i = tid; i < S * T; i += kSmallPermThreads) {
    const int sh = i / T, t = i % T;
    row_token[seg[E + sh] + t] = t;
  }
}

// One wavefront per row: x_perm[r] = x[row_token[r]] (or 0), 16 B per lane per step.
constexpr int kGatherU = 8;   // 16-byte chunks per lane per batch (a 4096-wide row in one batch)

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(int T, int H, int64_t mcap,
                                                               const int32_t* __restrict__ total,
                                                               const int32_t* __restrict__ row_token,
                                                               const uint16_t* __restrict__ x,
                                                               uint16_t* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= mcap || r >= total[0]) return;
  const int t = row_token[r];
  const int nv = H / 8;
  uint4* dst = reinterpret_cast<uint4*>(x_perm + r * H);
  if (t < 0 || t >= T) {   // padding (a token index past T never comes from the scatter)
    for (int c = lane; c < nv; c += 64) dst[c] = make_uint4(0, 0, 0, 0);
  } else {
    // all of a batch's loads are issued before its stores, so a wavefront keeps kGatherU 16-byte
    // loads in flight instead of one
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
    for (int c0 = lane; c0 < nv; c0 += 64 * kGatherU) {
      uint4 v[kGatherU];
#pragma unroll
      for (int u = 0; u < kGatherU; ++u) {
        const int c = c0 + 64 * u;
        v[u] = c < nv ? src[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kGatherU; ++u) {
        const int c = c0 + 64 * u;
        if (c < nv) dst[c] = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_permute(const moe_shape_t& s, int64_t mcap, const int32_t* topk_idx,
                          const uint16_t* x, int32_t* seg_offsets, int32_t* tile_group,
                          int32_t* total_rows, int32_t* row_token, int32_t* pos, uint16_t* x_perm,
                          int32_t* ws, hipStream_t st) {
  const int TB = permute_token_block(s.T);
  const int nblk = (int)permute_num_blocks(s.T);
  const int G = s.E + s.S;
  if (s.T <= kSmallPermT) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(kSmallPermThreads), 0, st, s.T, s.K, s.E,
                       s.S, s.block_m, mcap, topk_idx, seg_offsets, tile_group, total_rows,
                       row_token, pos);
    if (x) return launch_gather_rows(s, mcap, total_rows, row_token, x, x_perm, st);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_hist_kernel, dim3(nblk), dim3(kThreads), 0, st, s.T, s.K, s.E, TB,
                     topk_idx, ws);
  const size_t seg_lds = sizeof(int) * ((size_t)nblk * s.E + (G + 1) + s.E);
  const size_t sc_lds = sizeof(int) * ((size_t)2 * s.E * (TB / 32) + s.E);
  // Tables above 64 KiB of dynamic LDS need the per-kernel opt-in (gfx950 has 160 KiB per CU).
  if (seg_lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)perm_segment_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)seg_lds);
    if (e != hipSuccess) return e;
  }
  if (sc_lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)perm_scatter_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)sc_lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(perm_segment_kernel, dim3(1), dim3(kSegThreads), seg_lds, st, s.T, s.E, s.S,
                     s.block_m, nblk, mcap, ws, seg_offsets, tile_group, total_rows, row_token);
  hipLaunchKernelGGL(perm_clear_rows_kernel, dim3((unsigned)((mcap + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, mcap, total_rows, row_token);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblk), dim3(kThreads), sc_lds, st, s.T, s.K, s.E,
                     s.S, TB, topk_idx, ws, seg_offsets, pos, row_token);
  if (x) return launch_gather_rows(s, mcap, total_rows, row_token, x, x_perm, st);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const moe_shape_t& s, int64_t mcap, const int32_t* total_rows,
                              const int32_t* row_token, const uint16_t* x, uint16_t* x_perm,
                              hipStream_t st) {
  const int64_t rows_per_wg = kThreads / 64;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((mcap + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kThreads), 0, st, s.T, s.H, mcap, total_rows, row_token, x, x_perm);
  return hipGetLastError();
}

}  // namespace moe
