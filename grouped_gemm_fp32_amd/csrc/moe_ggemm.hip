// Grouped GEMM engine of the MoE expert FFN on gfx950 (bf16 MFMA, fp32 accumulation).
//
// dots.llm1 Technical Report, section 3.2 "Efficient grouped GEMM": every expert's token segment
// is padded to a fixed block size that is a multiple of the matrix instruction's M, so all rows of
// a workgroup tile belong to one expert and the grouped GEMM is scheduled like an ordinary GEMM.
// Section A2 (MoE paragraph): each expert is a two-layer FFN with SwiGLU.
//
// Three engines, by tile height (which must consist of whole blocks of one segment):
//   - eight wavefronts (two per SIMD), tiles of 128-384 rows x 256 columns, for block_m a multiple
//     of 128, and the persistent weight-gradient kernel (256 x 256 tiles of dW);
//   - four wavefronts, 64 x 256 tiles, for block_m == 64;
//   - four wavefronts with register-staged operands, 16- or 32-row tiles, for block_m 16 and 32.
// The first two stage operands in LDS with the buffer->LDS DMA and read MN-major operands with
// the transposing LDS read; the third loads through registers and transposes 8x8 in registers.
// Tiles are mapped to XCDs so that tiles sharing an operand panel share an L2, and so that every
// XCD gets an equal share of the work when segment lengths differ (skewed routing).
//
// Six kinds of tile share the engines:
//   FwdGateUp   h = x_perm . W1[g]^T, fused a = silu(h_gate) * h_up (and h_save)
//   FwdDown     y_perm = a . W2[g]^T
//   DgradDown   da = dy_perm . W2[g], fused SwiGLU backward -> dh
//   DgradGateUp dx_perm = dh . W1[g]
//   WgradDown   dW2[g] = dy_perm_seg^T . a_seg        (contraction over the segment's rows)
//   WgradGateUp dW1[g] = dh_seg^T . x_perm_seg
// FwdGateUp can also gather its rows from x through the permutation map (row r = x[row_token[r]],
// zero on padding rows) and, on tall tiles, write x_perm from the rows it stages, so the training
// step's permutation copies nothing.
#include <type_traits>

#include "moe_common.h"
#include "moe_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBK = 64;              // k per LDS stage
constexpr int kLdk = kBK + 8;        // padded LDS row (bf16 elements): 144 bytes, conflict-light
constexpr int kThreads = 256;

enum Kind { kFwdGateUp, kFwdDown, kDgradDown, kDgradGateUp, kWgradDown, kWgradGateUp };

template <int KIND> struct KindTraits {
  static constexpr bool a_trans = KIND == kWgradDown || KIND == kWgradGateUp;
  static constexpr bool b_trans = KIND != kFwdGateUp && KIND != kFwdDown;
  static constexpr bool split = KIND == kFwdGateUp;      // B rows: [gate half | up half]
  static constexpr bool grouped_rows = !a_trans;         // rows come from segments
};

struct GemmArgs {
  const uint16_t* a;   // A source
  // Gathered A rows (forward gate/up only): when set, row r of A is row a_rows[r] of `a` (the
  // token rows x[T,H], a_bytes bytes in all), and rows with a_rows[r] < 0 (padding) read as zero.
  const int32_t* a_rows;
  int64_t a_bytes;
  const uint16_t* b;   // B source
  int64_t lda, ldb;
  int64_t b_gstride;   // elements per group of the B source (weights); 0 for wgrad
  const uint16_t* aux; // h_save read by the SwiGLU backward epilogue
  uint16_t* out;
  int64_t ldo;
  int64_t o_gstride;   // elements per group of the output (wgrad)
  uint16_t* out2;      // h_save written by the forward gate/up epilogue (may be null)
  // x_perm written by the gathered gate/up product from its staged A rows (may be null): each
  // column tile's workgroup writes the rows r = nt (mod n_tiles_n) of its row tile
  uint16_t* out3;
  int M, N, K, I;
  int block_m;
  int max_blk;         // tall tiles: at most this many 128-row blocks per tile (2 or 3)
  int tile_chunk;      // tall tiles: consecutive row tiles dealt to one XCD at a time (1..8)
  int n_tiles_n, n_tiles_m;
  int G;
  const int32_t* tile_group;
  const int32_t* total_rows;
  const int32_t* seg;
};

template <int MS> struct Mfma;
template <> struct Mfma<32> {
  typedef f32x16_t acc_t;
  static constexpr int regs = 16, ksub = 16;
  __device__ static acc_t run(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Lane's operand row and k offset inside a sub-step.
  __device__ static int row(int lane) { return lane & 31; }
  __device__ static int kofs(int lane) { return (lane >> 5) * 8; }
  // Output: lane -> column m (the second operand's row), register r -> first-operand row n.
  __device__ static int out_m(int lane) { return lane & 31; }
  __device__ static int out_n(int lane, int q) { return 8 * q + 4 * (lane >> 5); }  // + (r & 3)
  static constexpr int groups = 4;  // groups of 4 consecutive n per lane
};
template <> struct Mfma<16> {
  typedef f32x4_t acc_t;
  static constexpr int regs = 4, ksub = 32;
  __device__ static acc_t run(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int row(int lane) { return lane & 15; }
  __device__ static int kofs(int lane) { return (lane >> 4) * 8; }
  __device__ static int out_m(int lane) { return lane & 15; }
  __device__ static int out_n(int lane, int q) { return 4 * (lane >> 4); }
  static constexpr int groups = 1;
};

// 8x8 transpose of bf16: in[k] holds 8 consecutive m at k; out[m] holds 8 consecutive k at m.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);  // w[k*4 + m/2], half m%2
  uint32_t* o = reinterpret_cast<uint32_t*>(out);             // o[m*4 + k/2], half k%2
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const uint32_t lo = w[(2 * kp) * 4 + (m >> 1)], hi = w[(2 * kp + 1) * 4 + (m >> 1)];
      o[m * 4 + kp] = (m & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
}

// ------------------------------------------------------------------------------------------------
// Operand staging. Each loader fetches one BK-slab of ROWS operand rows from HBM into registers
// (load) and writes it to LDS as [ROWS][kLdk] K-contiguous rows (store).
// ------------------------------------------------------------------------------------------------

// K-contiguous source: element (r, k) at base + row_ofs(r) + k. ROWS*8 16-byte chunks.
template <int ROWS> struct LoaderK {
  static constexpr int kChunks = ROWS * 8;
  static constexpr int kIters = (kChunks + kThreads - 1) / kThreads;
  uint4 v[kIters];
  template <class RowPtr>
  __device__ void load(RowPtr rowptr, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kThreads;
      v[i] = make_uint4(0, 0, 0, 0);
      if (kChunks % kThreads == 0 || idx < kChunks) {
        const uint16_t* p = rowptr(idx >> 3);
        if (p) v[i] = *reinterpret_cast<const uint4*>(p + k0 + (idx & 7) * 8);
      }
    }
  }
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int idx = tid + i * kThreads;
      if (kChunks % kThreads == 0 || idx < kChunks)
        *reinterpret_cast<uint4*>(lds + (idx >> 3) * kLdk + (idx & 7) * 8) = v[i];
    }
  }
};

// Row-contiguous source ([K][rows] in HBM): element (r, k) at base + k*ld + r. Each thread takes
// 8x8 blocks: 8 loads of 8 rows at consecutive k, transposed in registers, 8 LDS row writes.
// Lanes run over the 8 k-blocks of a row block first: a load instruction then reads 128
// contiguous bytes per k row, and the 8 lanes of a row block write one contiguous 128-byte LDS
// span (a row-block-major order would put lanes 1152 bytes apart: 16-way bank conflicts).
template <int ROWS> struct LoaderT {
  static constexpr int kBlocks = (ROWS / 8) * (kBK / 8);
  static constexpr int kIters = (kBlocks + kThreads - 1) / kThreads;
  uint4 v[kIters][8];
  // base points at (k = 0, r = 0) of the slab; rows >= rlim and k >= klim read as zero.
  __device__ void load(const uint16_t* base, int64_t ld, int rlim, int klim, int tid) {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int b = tid + i * kThreads;
      const int kb = b & 7, rb = b >> 3;  // 8 lanes cover one row block's 8 k-blocks
      const bool ok = (kBlocks % kThreads == 0 || b < kBlocks) && rb * 8 < rlim;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = kb * 8 + q;
        v[i][q] = make_uint4(0, 0, 0, 0);
        if (ok && k < klim) v[i][q] = *reinterpret_cast<const uint4*>(base + (int64_t)k * ld + rb * 8);
      }
    }
  }
  __device__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int b = tid + i * kThreads;
      if (kBlocks % kThreads == 0 || b < kBlocks) {
        const int kb = b & 7, rb = b >> 3;
        uint4 t[8];
        transpose8x8(v[i], t);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          *reinterpret_cast<uint4*>(lds + (rb * 8 + m) * kLdk + kb * 8) = t[m];
      }
    }
  }
};

template <bool TRANS, int ROWS> struct LoaderSel { typedef LoaderK<ROWS> type; };
template <int ROWS> struct LoaderSel<true, ROWS> { typedef LoaderT<ROWS> type; };

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

constexpr int64_t kSmallRowsBytes = 32ll << 20;   // activation bytes of a "small batch"

// SwiGLU backward of one accumulator row for the small-tile engines: da -> dh = [da*u*s*(1 +
// g(1-s)) | da*g*s] with g, u read from h_save (bf16). col(k) is the first of the 4 columns of
// group k (at or past N: nothing to do), val(k, e) its da values. The h loads of all NG groups are
// issued before the first dh store: the compiler cannot tell that h_save and dh do not overlap, so
// a load after a store would wait for it.
template <int NG, class Col, class Val>
__device__ __forceinline__ void swiglu_bwd_row(const GemmArgs& p, int64_t m, Col col, Val val) {
  const int64_t hrow = m * (2 * (int64_t)p.I);
  uint2 gw[NG], uw[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int c = col(k);
    const bool in = c < p.N;
    gw[k] = in ? *reinterpret_cast<const uint2*>(p.aux + hrow + c) : make_uint2(0, 0);
    uw[k] = in ? *reinterpret_cast<const uint2*>(p.aux + hrow + p.I + c) : make_uint2(0, 0);
  }
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int c = col(k);
    if (c >= p.N) continue;
    const float gg[4] = {lo_bf(gw[k].x), hi_bf(gw[k].x), lo_bf(gw[k].y), hi_bf(gw[k].y)};
    const float uu[4] = {lo_bf(uw[k].x), hi_bf(uw[k].x), lo_bf(uw[k].y), hi_bf(uw[k].y)};
    float dg[4], du[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = val(k, e);
      const float sg = 1.0f / (1.0f + expf(-gg[e]));
      dg[e] = v * uu[e] * sg * (1.0f + gg[e] * (1.0f - sg));
      du[e] = v * gg[e] * sg;
    }
    *reinterpret_cast<uint2*>(p.out + hrow + c) =
        make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
    *reinterpret_cast<uint2*>(p.out + hrow + p.I + c) =
        make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
  }
}

template <int KIND, int BM, int BN, int MS, int WAVES_M>
__global__ __launch_bounds__(kThreads, 2) void ggemm_kernel(GemmArgs p) {
  typedef KindTraits<KIND> Tr;
  typedef Mfma<MS> Mf;
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int TM = WTM / MS, TN = WTN / MS;
  static_assert(TM >= 1 && TN >= 1 && WTM % MS == 0 && WTN % MS == 0, "tile shape");
  static_assert(!Tr::split || TN % 2 == 0, "split needs gate/up pairs");

  __shared__ __attribute__((aligned(16))) uint16_t lds_a[BM * kLdk];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[BN * kLdk];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // ---- tile decode ------------------------------------------------------------------------------
  int g, m0, n0, kbeg, klen;
  if (Tr::grouped_rows) {
    const int total = p.total_rows[0];
    const int n_mt = total / BM;
    const int64_t n_valid = (int64_t)n_mt * p.n_tiles_n;
    const int64_t L = xcd_remap(blockIdx.x, n_valid);
    if (L < 0) return;
    // Small batches (the activation rows fit the last-level cache many times over): column-tile
    // major, so an expert's row blocks are consecutive workgroups that stream the same weight
    // panel together and share it through L2. Otherwise row-block major, so a row block's column
    // tiles share its activation panel.
    const bool nt_major = (int64_t)total * p.lda * 2 <= kSmallRowsBytes;
    const int mt = nt_major ? (int)(L % n_mt) : (int)(L / p.n_tiles_n);
    const int nt = nt_major ? (int)(L / n_mt) : (int)(L % p.n_tiles_n);
    m0 = mt * BM;
    n0 = nt * (Tr::split ? BN / 2 : BN);
    g = p.tile_group[m0 / p.block_m];
    kbeg = 0;
    klen = p.K;
  } else {
    const int64_t per_g = (int64_t)p.n_tiles_m * p.n_tiles_n;
    const int64_t L = xcd_remap(blockIdx.x, per_g * p.G);
    if (L < 0) return;
    g = (int)(L / per_g);
    const int rem = (int)(L % per_g);
    m0 = (rem / p.n_tiles_n) * BM;
    n0 = (rem % p.n_tiles_n) * BN;
    kbeg = p.seg[g];
    klen = p.seg[g + 1] - kbeg;
  }

  typename Mf::acc_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < Mf::regs; ++r) acc[i][j][r] = 0.0f;

  typename LoaderSel<Tr::a_trans, BM>::type la;
  typename LoaderSel<Tr::b_trans, BN>::type lb;

  // Row pointers of K-contiguous operands (k offset added by the loader).
  const uint16_t* a_tile = p.a + (int64_t)m0 * p.lda;
  const uint16_t* b_grp = p.b + (int64_t)g * p.b_gstride;
  auto a_row = [&](int r) -> const uint16_t* {
    if (p.a_rows) {   // gathered rows: padding rows (token < 0) load as zero
      const int tok = p.a_rows[m0 + r];
      return tok >= 0 ? p.a + (int64_t)tok * p.lda : nullptr;
    }
    return a_tile + (int64_t)r * p.lda;
  };
  auto b_row = [&](int r) -> const uint16_t* {
    if (Tr::split) {
      const int half = BN / 2;
      const int c = n0 + (r % half);
      if (c >= p.I) return nullptr;
      return b_grp + (int64_t)((r < half ? 0 : p.I) + c) * p.ldb;
    }
    if (n0 + r >= p.N) return nullptr;
    return b_grp + (int64_t)(n0 + r) * p.ldb;
  };

  auto load_stage = [&](int k0) {
    if constexpr (Tr::a_trans) {
      la.load(p.a + (int64_t)(kbeg + k0) * p.lda + m0, p.lda, p.M - m0, klen - k0, tid);
    } else {
      la.load(a_row, k0, tid);
    }
    if constexpr (Tr::b_trans) {
      lb.load(b_grp + (int64_t)(kbeg + k0) * p.ldb + n0, p.ldb, p.N - n0, klen - k0, tid);
    } else {
      lb.load(b_row, k0, tid);
    }
  };

  // LDS row of the wave's B sub-tile j.
  auto b_lds_row = [&](int j) {
    if (Tr::split) {
      constexpr int half = TN / 2;
      return (j / half) * (BN / 2) + wn * (WTN / 2) + (j % half) * MS;
    }
    return wn * WTN + j * MS;
  };

  const int nk = (klen + kBK - 1) / kBK;
  if (nk > 0) {
    load_stage(0);
    la.store(lds_a, tid);
    lb.store(lds_b, tid);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load_stage((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK; ks += Mf::ksub) {
      bf16x8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            lds_a + (wm * WTM + i * MS + Mf::row(lane)) * kLdk + ks + Mf::kofs(lane));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t*>(
            lds_b + (b_lds_row(j) + Mf::row(lane)) * kLdk + ks + Mf::kofs(lane));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mf::run(bf[j], af[i], acc[i][j]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      la.store(lds_a, tid);
      lb.store(lds_b, tid);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds row m = m_in, registers hold 4 consecutive columns per group --------
  const int m_in = Mf::out_m(lane);
  if constexpr (Tr::split) {
    constexpr int half = TN / 2;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WTM + i * MS + m_in;
#pragma unroll
      for (int jj = 0; jj < half; ++jj)
#pragma unroll
        for (int q = 0; q < Mf::groups; ++q) {
          const int c = n0 + wn * (WTN / 2) + jj * MS + Mf::out_n(lane, q);
          if (c >= p.I) continue;
          float av[4];
          uint32_t hg[2], hu[2];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[i][jj][4 * q + e], uv = acc[i][jj + half][4 * q + e];
            av[e] = silu_f(gv) * uv;
          }
          hg[0] = pack_bf2(acc[i][jj][4 * q], acc[i][jj][4 * q + 1]);
          hg[1] = pack_bf2(acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]);
          hu[0] = pack_bf2(acc[i][jj + half][4 * q], acc[i][jj + half][4 * q + 1]);
          hu[1] = pack_bf2(acc[i][jj + half][4 * q + 2], acc[i][jj + half][4 * q + 3]);
          *reinterpret_cast<uint2*>(p.out + m * p.ldo + c) =
              make_uint2(pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3]));
          if (p.out2) {
            *reinterpret_cast<uint2*>(p.out2 + m * (2 * (int64_t)p.I) + c) = make_uint2(hg[0], hg[1]);
            *reinterpret_cast<uint2*>(p.out2 + m * (2 * (int64_t)p.I) + p.I + c) =
                make_uint2(hu[0], hu[1]);
          }
        }
    }
  } else {
    uint16_t* out = p.out + (Tr::grouped_rows ? 0 : (int64_t)g * p.o_gstride);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int mloc = wm * WTM + i * MS + m_in;
      const int64_t m = m0 + mloc;
      if (!Tr::grouped_rows && m >= p.M) continue;
      if constexpr (KIND == kDgradDown) {
        constexpr int NQ = Mf::groups;
        swiglu_bwd_row<TN * NQ>(p, m,
            [&](int k) { return n0 + wn * WTN + (k / NQ) * MS + Mf::out_n(lane, k % NQ); },
            [&](int k, int e) { return acc[i][k / NQ][4 * (k % NQ) + e]; });
        continue;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < Mf::groups; ++q) {
          const int c = n0 + wn * WTN + j * MS + Mf::out_n(lane, q);
          if (c >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          *reinterpret_cast<uint2*>(out + m * p.ldo + c) =
              make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
        }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// DMA engine (tiles of 64 to 384 rows). A segment is a whole number of block_m-row blocks of one
// expert, so a tile may span several consecutive 128-row blocks and still belong to one expert.
// The tall kernel cuts every segment into ceil(len / 384) tiles of 128, 256 or 384 rows, as even
// as the 128-row granularity allows; an expert with 384 rows then streams each weight panel once,
// where 128- or 256-row tiles would stream it two or three times.
//
// Operands go from HBM to LDS through the bounds-checked buffer->LDS DMA
// (buffer_load_dwordx4 ... lds): lane l of a wavefront deposits its 16 bytes at LDS M0 + 16 l,
// whatever address it loaded, and reads past the buffer resource's size return zero (tile tails
// and segment ends need no special code). A ring of up to four stages of BK k.
//   K-major operand (K contiguous in HBM): LDS [rows][BK]; 16-byte chunk c of row r sits at
//     position c ^ swz(r) (swz = (r >> 1) & 7 with 8 chunks per row, (r >> 2) & 3 with 4), so
//     the rows of a fragment read spread over all banks.
//   MN-major operand (rows contiguous in HBM, [k][rows]): LDS [BK][rows] as in HBM, chunk cc of
//     k-row k stored at cc ^ ((k & 3) << 2); fragments come from ds_read_b64_tr_b16, which hands
//     each lane 4 consecutive k of one column (within 16 lanes: lane i, item q <- lane 4q + i/4,
//     item i % 4), two reads per 32x32x16 operand.
// Four wavefronts, WM x WN, each (BM/WM) x (BN/WN) of the tile, v_mfma_f32_32x32x16_bf16 with the
// B fragment as the first operand so that a lane ends with 4 consecutive output columns.
//
// Pipeline: the fragments of the next 16-k slice are read from LDS while the MFMAs of the current
// slice run. The one barrier per stage sits before the stage's last slice: every wave then holds
// that slice's fragments in registers, so the barrier both publishes the next stage (whose DMA
// each wave has waited for) and frees the current stage's slot, which is refilled at once with
// the stage STAGES ahead. STAGES - 1 stages are in flight while a stage is computed.
// ------------------------------------------------------------------------------------------------
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
constexpr int kLdsBytes = 163840;   // gfx950: 160 KiB of LDS per workgroup
constexpr int kTallBlk = 128;       // row granularity of tall tiles (block_m % 128 == 0)
constexpr int kTallMaxBlk = 3;      // tallest tile: 3 blocks = 384 rows

template <int BM_, int BN_, int WM_, int BK_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = 4 / WM_, BK = BK_;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32, KK = BK / 16;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int STAGES = kLdsBytes / STAGE >= 4 ? 4 : kLdsBytes / STAGE;
  static constexpr int LA = A_BYTES / 4096, LB = B_BYTES / 4096;  // DMA instr per lane per stage
  static_assert(WM * WN == 4 && TM * 32 == WTM && TN * 32 == WTN, "wave tiling");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(A_BYTES % 4096 == 0 && B_BYTES % 4096 == 0, "whole DMA rounds");
  static_assert(STAGES >= 2, "two stages must fit in LDS");
  static_assert((STAGES - 1) * (LA + LB) < 64, "vmcnt range");
};

// K-major LDS position of 16-byte chunk c of row r (an involution, so it also maps back).
// gfx950 serves a 16-byte LDS read 16 lanes at a time from 64 banks (256 bytes): the 16 rows of
// such a group must land on 16 distinct 16-byte bank slots. With 128-byte rows a slot is
// (r & 1, position), so the position varies with r >> 1; with 64-byte rows it is (r & 3,
// position) and varies with r >> 2. (Measured: keying on r & 7 instead gave 26x the conflict
// cycles on the forward kernels.)
template <int BK>
__device__ __forceinline__ int kswz(int r, int c) {
  if constexpr (BK == 64) return c ^ ((r >> 1) & 7);
  else return c ^ ((r >> 2) & 3);
}

// Epilogue shared by the engines: lane -> row, registers -> 4 consecutive columns per group.

template <int KIND, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const f32x16_t (&acc)[TM][TN], int g,
                                           int m0, int n0, int wm, int wn, int lane) {
  typedef KindTraits<KIND> Tr;
  typedef Mfma<32> Mf;
  const int m_in = Mf::out_m(lane);
  if constexpr (Tr::split) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 32 + m_in;
#pragma unroll
      for (int jj = 0; jj < TN / 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = n0 + wn * (WTN / 2) + jj * 32 + Mf::out_n(lane, q);
          if (c >= p.I) continue;
          const f32x16_t& ga = acc[i][jj];
          const f32x16_t& ua = acc[i][jj + TN / 2];
          float av[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = silu_f(ga[4 * q + e]) * ua[4 * q + e];
          *reinterpret_cast<uint2*>(p.out + m * p.ldo + c) =
              make_uint2(pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3]));
          if (p.out2) {
            uint16_t* hrow = p.out2 + m * (2 * (int64_t)p.I);
            *reinterpret_cast<uint2*>(hrow + c) =
                make_uint2(pack_bf2(ga[4 * q], ga[4 * q + 1]), pack_bf2(ga[4 * q + 2], ga[4 * q + 3]));
            *reinterpret_cast<uint2*>(hrow + p.I + c) =
                make_uint2(pack_bf2(ua[4 * q], ua[4 * q + 1]), pack_bf2(ua[4 * q + 2], ua[4 * q + 3]));
          }
        }
    }
  } else {
    uint16_t* out = p.out + (Tr::grouped_rows ? 0 : (int64_t)g * p.o_gstride);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 32 + m_in;
      if (!Tr::grouped_rows && m >= p.M) continue;
      if constexpr (KIND == kDgradDown) {
        swiglu_bwd_row<TN * 4>(p, m,
            [&](int k) { return n0 + wn * WTN + (k / 4) * 32 + Mf::out_n(lane, k % 4); },
            [&](int k, int e) { return acc[i][k / 4][4 * (k % 4) + e]; });
        continue;
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = n0 + wn * WTN + j * 32 + Mf::out_n(lane, q);
          if (c >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          *reinterpret_cast<uint2*>(out + m * p.ldo + c) =
              make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
        }
    }
  }
}

// One tile: rows m0.. of group g (row-grouped kinds) or weight rows m0.. of group g (wgrad),
// columns n0.., contraction over [kbeg, kbeg + klen).
template <int KIND, class TL>
__device__ __forceinline__ void pipe_tile(const GemmArgs& p, unsigned char* smem, int g, int m0,
                                          int n0, int kbeg, int klen) {
  typedef KindTraits<KIND> Tr;
  typedef Mfma<32> Mf;
  constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, WTM = TL::WTM, WTN = TL::WTN;
  constexpr int TM = TL::TM, TN = TL::TN, KK = TL::KK;
  constexpr int A_BYTES = TL::A_BYTES, STAGE = TL::STAGE, STAGES = TL::STAGES;
  constexpr int LA = TL::LA, LB = TL::LB;
  constexpr bool AMN = Tr::a_trans, BMN = Tr::b_trans;
  static_assert(!Tr::split || TN % 2 == 0, "split needs gate and up sub-tiles in pairs");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / TL::WN, wn = wave % TL::WN;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_u8_t*)smem;
  lds_u8_t* s3 = (lds_u8_t*)smem;

  // ---- buffer resources: each covers exactly the bytes this tile may read ----------------------
  v4u32_t ra, rb;
  const bool gather = !AMN && p.a_rows != nullptr;   // A rows gathered from the token rows
  if (AMN) ra = make_rsrc(p.a + (int64_t)kbeg * p.lda, (int64_t)klen * p.lda * 2);
  else if (gather) ra = make_rsrc(p.a, p.a_bytes);
  else ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (int64_t)BM * p.lda * 2);
  if (Tr::grouped_rows) rb = make_rsrc(p.b + (int64_t)g * p.b_gstride, p.b_gstride * 2);
  else rb = make_rsrc(p.b + (int64_t)kbeg * p.ldb, (int64_t)klen * p.ldb * 2);

  // ---- per-lane DMA byte offsets of stage 0 (a k-step adds a fixed stride) ---------------------
  // K-major: instruction i of wave w fills rows (i*4 + w)*RPI .. +RPI, lane -> (row, position).
  // MN-major: instruction i of wave w fills flat chunks (i*4 + w)*64 + lane of [BK][ROWS].
  constexpr int CPR = BK / 8, RPI = 64 / CPR;
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    if constexpr (!AMN) {
      const int r = (i * 4 + wave) * RPI + lane / CPR;
      const int c = kswz<BK>(r, lane % CPR);
      if (gather) {
        const int tok = p.a_rows[m0 + r];
        a_off[i] = tok >= 0 ? (uint32_t)(((int64_t)tok * p.lda + c * 8) * 2) : kPastEnd;
      } else {
        a_off[i] = (uint32_t)(((int64_t)r * p.lda + c * 8) * 2);
      }
    } else {
      constexpr int CPRM = BM / 8;
      const int f = (i * 4 + wave) * 64 + lane;
      const int k = f / CPRM, cc = (f % CPRM) ^ ((k & 3) << 2);
      a_off[i] = (uint32_t)(((int64_t)k * p.lda + m0 + cc * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    if constexpr (!BMN) {
      const int r = (i * 4 + wave) * RPI + lane / CPR;
      const int c = kswz<BK>(r, lane % CPR);
      int64_t row;
      if (Tr::split) row = r < BN / 2 ? n0 + r : p.I + n0 + (r - BN / 2);
      else row = n0 + r;
      b_off[i] = (uint32_t)((row * p.ldb + c * 8) * 2);
    } else {
      constexpr int CPRM = BN / 8;
      const int f = (i * 4 + wave) * 64 + lane;
      const int k = f / CPRM, cc = (f % CPRM) ^ ((k & 3) << 2);
      b_off[i] = (uint32_t)(((int64_t)k * p.ldb + n0 + cc * 8) * 2);
    }
  }
  const uint32_t a_kstep = AMN ? (uint32_t)(BK * p.lda * 2) : (uint32_t)(BK * 2);
  const uint32_t b_kstep = BMN ? (uint32_t)(BK * p.ldb * 2) : (uint32_t)(BK * 2);

  auto issue = [&](int kt, int slot) {
    const uint32_t sa = lds_base + slot * STAGE;
    const uint32_t sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(ra, a_off[i] + kt * a_kstep, sa + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < LB; ++i) dma16(rb, b_off[i] + kt * b_kstep, sb + (i * 4 + wave) * 1024);
  };

  // ---- fragments ----------------------------------------------------------------------------------
  // LDS row (K-major) or column (MN-major) of the wave's sub-tile j of B.
  auto b_row = [&](int j) {
    if (Tr::split) return (j / (TN / 2)) * (BN / 2) + wn * (WTN / 2) + (j % (TN / 2)) * 32;
    return wn * WTN + j * 32;
  };
  const int l32 = lane & 31, hi = lane >> 5;
  const int grp = lane >> 4, li = lane & 15;
  auto frag_k = [&](int base, int row0, int kk) -> bf16x8_t {
    const int r = row0 + l32;
    return *reinterpret_cast<const bf16x8_t*>(smem + base + r * (BK * 2) +
                                              kswz<BK>(r, 2 * kk + hi) * 16);
  };
  // MN-major: two transposed 8-byte reads give columns col0 + (grp&1)*16 + li,
  // k = kk*16 + (grp>>1)*8 + 0..7.
  auto frag_t = [&](int base, int rows, int col0, int kk) -> bf16x8_t {
    const int col = col0 + (grp & 1) * 16 + 4 * (li & 3);
    const int cc = col >> 3, half = ((col >> 2) & 1) * 8;
    const int k0 = kk * 16 + (grp >> 1) * 8 + (li >> 2);
    const int ad0 = base + k0 * rows * 2 + ((cc ^ ((k0 & 3) << 2)) * 16) + half;
    const int k1 = k0 + 4;
    const int ad1 = base + k1 * rows * 2 + ((cc ^ ((k1 & 3) << 2)) * 16) + half;
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(s3 + ad0));
    const v4i16_t hi2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(s3 + ad1));
    bf16x8_t r;
    __builtin_memcpy(&r, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi2, 8);
    return r;
  };
  struct Frags { bf16x8_t a[TM], b[TN]; };
  auto load = [&](int slot, int kk, Frags& f) {
    const int sa = slot * STAGE, sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (AMN) f.a[i] = frag_t(sa, BM, wm * WTM + i * 32, kk);
      else f.a[i] = frag_k(sa, wm * WTM + i * 32, kk);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if constexpr (BMN) f.b[j] = frag_t(sb, BN, b_row(j), kk);
      else f.b[j] = frag_k(sb, b_row(j), kk);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = Mf::run(f.b[j], f.a[i], acc[i][j]);
  };

  // ---- main loop ----------------------------------------------------------------------------------
  const int nk = (klen + BK - 1) / BK;
  if (nk > 0) {
#pragma unroll
    for (int s0 = 0; s0 < STAGES; ++s0)
      if (s0 < nk) issue(s0, s0);
    wait_stages<LA + LB, STAGES - 1>(min(STAGES - 1, nk - 1));
    block_barrier();
    Frags cur;
    load(0, 0, cur);
    for (int kt = 0; kt < nk; ++kt) {
      const int slot = kt % STAGES;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frags nxt;
        if (kk + 1 < KK) {
          load(slot, kk + 1, nxt);
        } else if (kt + 1 < nk) {
          // Stage kt + 1 must have landed (own DMA: wait; other waves': the barrier) and every
          // wave must be done reading this slot before it is refilled.
          wait_stages<LA + LB, STAGES - 1>(min(STAGES - 2, nk - kt - 2));
          wait_lgkm0();
          block_barrier();
          load((kt + 1) % STAGES, 0, nxt);
          if (kt + STAGES < nk) issue(kt + STAGES, slot);
        }
        mma(cur);
        cur = nxt;
      }
    }
  }

  store_tile<KIND, TM, TN, WTM, WTN>(p, acc, g, m0, n0, wm, wn, lane);
}

// Row-grouped 64-row tiles (block_m == 64) on the four-wavefront engine.
typedef Tile<64, 256, 2, 64> Block64Tile;

// Columns of output one tile covers (gate/up: gate columns; the tile also covers as many up).
template <int KIND> constexpr int tile_cols(int bn) { return KindTraits<KIND>::split ? bn / 2 : bn; }

// ------------------------------------------------------------------------------------------------
// Epilogue of the eight-wavefront engine. An MFMA result gives each lane 4 consecutive columns of
// one row, so storing straight from registers writes 16 bytes to each of 32 rows per instruction.
// Instead every 32-row block goes through a per-wavefront LDS buffer (16-byte chunks XOR-swizzled
// by row) and leaves in 16-byte chunks with a whole 128- or 256-byte row segment per group of
// lanes.
// ------------------------------------------------------------------------------------------------
// Stage a 32 x (NJ*32) block of bf16 values (val(j, q, e): sub-tile j, column group q, element e of
// this lane's row) and hand each 16-byte row chunk to dst(row, col, uint4).
template <int NJ, class Val, class Dst>
__device__ __forceinline__ void stage_bf16(unsigned char* scr, int lane, Val val, Dst dst) {
  constexpr int W = NJ * 32, NCH = W / 8, RS = W * 2, RPI = 64 / NCH;
  static_assert(NCH >= 4 && NCH <= 64 && (NCH & (NCH - 1)) == 0, "row chunks");
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = 4 * j + q;
      const uint2 w = make_uint2(pack_bf2(val(j, q, 0), val(j, q, 1)), pack_bf2(val(j, q, 2), val(j, q, 3)));
      *reinterpret_cast<uint2*>(scr + r * RS + ((ch ^ (r & (NCH - 1))) * 16) + hi * 8) = w;
    }
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + lane / NCH, c = lane % NCH;
    const uint4 d = *reinterpret_cast<const uint4*>(scr + rr * RS + ((c ^ (rr & (NCH - 1))) * 16));
    dst(rr, c * 8, d);
  }
}

// The same for fp32 values: dst(it, row, col, float4) gets 4 consecutive columns of row chunk it.
// The chunks go in batches of B: pre(it, row, col) runs for each chunk of a batch before the
// batch's first dst(), so the loads it issues are in flight together (a dst() that stores would
// otherwise keep the next chunk's loads behind it).
template <int NJ, int B, class Val, class Pre, class Dst>
__device__ __forceinline__ void stage_f32_pre(unsigned char* scr, int lane, Val val, Pre pre, Dst dst) {
  constexpr int W = NJ * 32, NCH = W / 4, RS = W * 4, RPI = 64 / NCH;
  static_assert(NCH >= 4 && NCH <= 64 && (NCH & (NCH - 1)) == 0, "row chunks");
  const int r = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = 8 * j + 2 * q + hi;
      const float4 w = make_float4(val(j, q, 0), val(j, q, 1), val(j, q, 2), val(j, q, 3));
      *reinterpret_cast<float4*>(scr + r * RS + ((ch ^ (r & (NCH - 1))) * 16)) = w;
    }
  static_assert((32 / RPI) % B == 0, "whole batches");
#pragma unroll
  for (int i0 = 0; i0 < 32 / RPI; i0 += B) {
#pragma unroll
    for (int it = i0; it < i0 + B; ++it) pre(it, it * RPI + lane / NCH, (lane % NCH) * 4);
#pragma unroll
    for (int it = i0; it < i0 + B; ++it) {
      const int rr = it * RPI + lane / NCH, c = lane % NCH;
      const float4 d = *reinterpret_cast<const float4*>(scr + rr * RS + ((c ^ (rr & (NCH - 1))) * 16));
      dst(it, rr, c * 4, d);
    }
  }
}

// stage_f32_pre without the pre step: dst(row, col, float4).
template <int NJ, class Val, class Dst>
__device__ __forceinline__ void stage_f32(unsigned char* scr, int lane, Val val, Dst dst) {
  stage_f32_pre<NJ, 1>(scr, lane, val, [](int, int, int) {},
                    [&](int, int rr, int c, float4 d) { dst(rr, c, d); });
}

__device__ __forceinline__ float4 bf4_to_f4(uint2 w) {
  return make_float4(lo_bf(w.x), hi_bf(w.x), lo_bf(w.y), hi_bf(w.y));
}

// scr: this wavefront's LDS buffer of at least 8 KiB.
template <int KIND, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_tile8(const GemmArgs& p, const f32x16_t (&acc)[TM][TN], int g,
                                            int m0, int n0, int wm, int wn, int lane,
                                            unsigned char* scr) {
  typedef KindTraits<KIND> Tr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t mrow = m0 + wm * WTM + i * 32;   // first row of this 32-row block
    if constexpr (Tr::split) {
      // a = silu(gate) * up, columns n0 + wn*WTN/2 .. of [rows, I]; then h = [gate | up] rows.
      constexpr int NJ = TN / 2;
      const int c0 = n0 + wn * (WTN / 2);
      stage_bf16<NJ>(scr, lane,
          [&](int j, int q, int e) { return silu_f(acc[i][j][4 * q + e]) * acc[i][j + NJ][4 * q + e]; },
          [&](int rr, int c, uint4 d) {
            if (c0 + c < p.I) *reinterpret_cast<uint4*>(p.out + (mrow + rr) * p.ldo + c0 + c) = d;
          });
      if (p.out2) {
        uint16_t* h = p.out2;
        const int64_t ldh = 2 * (int64_t)p.I;
        stage_bf16<NJ>(scr, lane, [&](int j, int q, int e) { return acc[i][j][4 * q + e]; },
            [&](int rr, int c, uint4 d) {
              if (c0 + c < p.I) *reinterpret_cast<uint4*>(h + (mrow + rr) * ldh + c0 + c) = d;
            });
        stage_bf16<NJ>(scr, lane, [&](int j, int q, int e) { return acc[i][j + NJ][4 * q + e]; },
            [&](int rr, int c, uint4 d) {
              if (c0 + c < p.I) *reinterpret_cast<uint4*>(h + (mrow + rr) * ldh + p.I + c0 + c) = d;
            });
      }
    } else if constexpr (KIND == kDgradDown) {
      // da (fp32) meets the saved h: dg = da*u*s*(1 + g*(1 - s)), du = da*g*s, s = sigmoid(g).
      // in passes of 64 columns, which keeps the epilogue's registers within budget
      static_assert(TN % 2 == 0, "64-column passes");
#pragma unroll
      for (int h = 0; h < TN / 2; ++h) {
      const int c0 = n0 + wn * WTN + h * 64;
      const int64_t ldh = 2 * (int64_t)p.I;
      // the saved h of 4 row chunks at a time (half the 32 x 64 pass) is loaded before their
      // first dh store: 8 loads in flight instead of 2, within the register budget
      uint2 hg[8], hu[8];
      stage_f32_pre<2, 4>(scr, lane, [&](int j, int q, int e) { return acc[i][2 * h + j][4 * q + e]; },
          [&](int it, int rr, int c) {
            const int64_t hrow = (mrow + rr) * ldh + c0 + c;
            const bool in = c0 + c < p.N;
            hg[it] = in ? *reinterpret_cast<const uint2*>(p.aux + hrow) : make_uint2(0, 0);
            hu[it] = in ? *reinterpret_cast<const uint2*>(p.aux + hrow + p.I) : make_uint2(0, 0);
          },
          [&](int it, int rr, int c, float4 da) {
            if (c0 + c >= p.N) return;
            const int64_t hrow = (mrow + rr) * ldh + c0 + c;
            const float4 gg = bf4_to_f4(hg[it]);
            const float4 uu = bf4_to_f4(hu[it]);
            const float gv[4] = {gg.x, gg.y, gg.z, gg.w}, uv[4] = {uu.x, uu.y, uu.z, uu.w};
            const float av[4] = {da.x, da.y, da.z, da.w};
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = 1.0f / (1.0f + expf(-gv[e]));
              dg[e] = av[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
              du[e] = av[e] * gv[e] * sg;
            }
            *reinterpret_cast<uint2*>(p.out + hrow) =
                make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(p.out + hrow + p.I) =
                make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          });
      }
    } else {
      uint16_t* out = p.out + (Tr::grouped_rows ? 0 : (int64_t)g * p.o_gstride);
      const int c0 = n0 + wn * WTN;
      stage_bf16<TN>(scr, lane, [&](int j, int q, int e) { return acc[i][j][4 * q + e]; },
          [&](int rr, int c, uint4 d) {
            const int64_t m = mrow + rr;
            if (!Tr::grouped_rows && m >= p.M) return;
            if (c0 + c < p.N) *reinterpret_cast<uint4*>(out + m * p.ldo + c0 + c) = d;
          });
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Eight-wavefront engine (two wavefronts per SIMD) for the tall row-grouped tiles: BK = 64, two
// LDS stages. A stage's DMA (128-byte row segments, the request size the texture path serves
// best) is spread over the MFMAs of the slices before the stage is needed: a third of it is
// issued right after the barrier that frees its slot, the rest during the next two slices, so a
// wavefront held up at DMA issue leaves the matrix unit to the other wavefront of its SIMD, and
// the last DMA of a stage still has two slices of MFMAs to land. Each fragment of the next
// 16-k slice is read from LDS as soon as the current slice's last MFMA using its registers has
// issued, so a slice starts with its operands in registers.
// ------------------------------------------------------------------------------------------------
// Q1, Q2: the DMA instructions of a stage issued by the end of the slice right after the freeing
// barrier and by the end of the next one, in twelfths of the stage's L (rounded up); the rest go
// out in the slice after that.
template <int BM_, int BN_, int WM_, int WN_, int Q1 = 4, int Q2 = 8>
struct Tile8 {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = 8, BK = 64, KK = 4, NS = 2;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  static constexpr int LA = A_BYTES / (NW * 1024), LB = B_BYTES / (NW * 1024), L = LA + LB;
  // DMA instructions [0, P1) of a stage go out in slice 0, [P1, P2) in slice 1, [P2, L) in slice 2
  static constexpr int P1 = (Q1 * L + 11) / 12, P2 = (Q2 * L + 11) / 12;
  static_assert(0 < Q1 && Q1 <= Q2 && Q2 <= 12, "DMA parts");
  static_assert(WM * WN == NW && TM * 32 == WTM && TN * 32 == WTN, "wave tiling");
  static_assert(A_BYTES % (NW * 1024) == 0 && B_BYTES % (NW * 1024) == 0, "whole DMA rounds");
  static_assert(NS * STAGE <= kLdsBytes, "two stages must fit in LDS");
};
constexpr int kThreads8 = 512;

// The engine proper: DMA addressing of one tile at a time, fragment reads and the pipelined
// contraction. A persistent kernel may set up the next tile's DMA while the accumulators of the
// current one are still live.
template <int KIND, class TL, bool GA = false>
struct Eng8 {
  typedef KindTraits<KIND> Tr;
  static_assert(!GA || !Tr::a_trans, "gathered rows are a K-major A operand");
  typedef Mfma<32> Mf;
  static constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, WTM = TL::WTM, WTN = TL::WTN;
  static constexpr int TM = TL::TM, TN = TL::TN, NW = TL::NW;
  static constexpr int A_BYTES = TL::A_BYTES, STAGE = TL::STAGE, LA = TL::LA, L = TL::L;
  static constexpr bool AMN = Tr::a_trans, BMN = Tr::b_trans;
  // K-major: instruction i of wave w fills rows (i*NW + w)*RPI .. +RPI (8 lanes per 128-byte row).
  // MN-major: instruction i of wave w fills flat chunks (i*NW + w)*64 + lane of [BK][ROWS].
  static constexpr int CPR = BK / 8, RPI = 64 / CPR;
  static_assert(!Tr::split || TN % 2 == 0, "split needs gate and up sub-tiles in pairs");
  struct Frags { bf16x8_t a[TM], b[TN]; };
  typedef f32x16_t Acc[TM][TN];

  const GemmArgs& p;
  unsigned char* smem;
  lds_u8_t* s3;
  uint32_t lds_base;
  int lane, wave, wm, wn;
  // false when this wavefront's output columns of the current tile all lie at or past N (the
  // ragged last column tile, e.g. N = 1408 = 5.5 x 256): it then still issues its share of the
  // DMA and meets every barrier, but reads no fragments and issues no MFMAs.
  // Only the down projection's gradients have N = I, which need not be a multiple of 256 (1408 is
  // 5.5 tiles); elsewhere the check is compiled out, leaving the hot loop as it was.
  static constexpr bool kRagged = KIND == kDgradDown || KIND == kWgradDown;
  bool mma_on = true;
  // Per tile: where the upper column half lies wholly at or past N, waves w and w + 4 (which share
  // a SIMD) take the same row band and the two halves, so each SIMD keeps one busy wavefront;
  // elsewhere waves 2r and 2r + 1 take row band r (measured faster on whole tiles).
  __device__ __forceinline__ void set_tile_cols(int n0) {
    if constexpr (!kRagged) return;
    constexpr bool split = KindTraits<KIND>::split;
    const int n_lim = split ? p.I : p.N, half = split ? TL::WTN / 2 : TL::WTN;
    if (n0 + half >= n_lim) {
      wm = wave % TL::WM;
      wn = wave / TL::WM;
    } else {
      wm = wave / TL::WN;
      wn = wave % TL::WN;
    }
    mma_on = n0 + wn * half < n_lim;
  }
  // DMA state of one tile: buffer resources and one lane offset per operand; instruction i adds
  // a wave-uniform stride, stage kt adds kt * kstep.
  struct Dma {
    v4u32_t ra, rb;
    uint32_t a_off0, b_off0;
    uint32_t a_offs[GA ? TL::LA : 1];   // gathered A: one lane offset per DMA instruction
    uint32_t a_offs_hi[GA ? TL::LA : 1];   // ... and for the rows of the wave 4 above (HD)
  };
  uint32_t a_kstep, b_kstep;
  // HD: only waves 0-3 (one per SIMD) issue the DMA, each its own instructions and those of the
  // wave 4 above it (LDS 4 KiB further on; K-major operands 32 rows further on, MN-major ones
  // 256 chunks, a whole number of k-rows), so the other wave of each SIMD never waits at a full
  // texture queue. Gathered rows: waves 0-3 hold the lane offsets of both. (false: every wave
  // issues its own share.)
  static constexpr bool HD = true;
  uint32_t a_vs, b_vs;
  // Gathered gate/up with p.out3: per stage each lane of this workgroup copies one 16-byte chunk
  // of its share of the staged rows (read before the stage's barrier, stored after it, so the
  // store waits on nothing and no DMA wait waits on it before the next stage's).
  static constexpr bool CP = GA && Tr::split;
  int cp_m0 = 0, cp_nt = 0;   // the tile's first row and column-tile index (set per tile)

  __device__ __forceinline__ Eng8(const GemmArgs& p_, unsigned char* smem_) : p(p_), smem(smem_) {
    s3 = (lds_u8_t*)smem;
    lds_base = (uint32_t)(uintptr_t)s3;
    lane = threadIdx.x & 63;
    wave = (int)uniform((uint32_t)(threadIdx.x >> 6));
    static_assert(TL::WN == 2 && TL::NW == 8, "two column halves over eight wavefronts");
    wm = wave / TL::WN;
    wn = wave % TL::WN;
    a_kstep = AMN ? (uint32_t)(BK * p.lda * 2) : (uint32_t)(BK * 2);
    b_kstep = BMN ? (uint32_t)(BK * p.ldb * 2) : (uint32_t)(BK * 2);
    a_vs = AMN ? (uint32_t)((4 * 64 / (BM / 8)) * p.lda * 2) : (uint32_t)(4 * RPI * p.lda * 2);
    b_vs = BMN ? (uint32_t)((4 * 64 / (BN / 8)) * p.ldb * 2) : (uint32_t)(4 * RPI * p.ldb * 2);
  }

  // Tile: rows m0.. of group g (row-grouped kinds) or weight rows m0.. of group g (wgrad),
  // columns n0.., contraction over [kbeg, kbeg + klen).
  __device__ __forceinline__ void setup(Dma& st, int g, int m0, int n0, int kbeg, int klen) const {
    if (AMN) st.ra = make_rsrc(p.a + (int64_t)kbeg * p.lda, (int64_t)klen * p.lda * 2);
    else if (GA) st.ra = make_rsrc(p.a, p.a_bytes);
    else st.ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (int64_t)BM * p.lda * 2);
    if (Tr::grouped_rows) st.rb = make_rsrc(p.b + (int64_t)g * p.b_gstride, p.b_gstride * 2);
    else st.rb = make_rsrc(p.b + (int64_t)kbeg * p.ldb, (int64_t)klen * p.ldb * 2);
    if constexpr (GA) {
      // instruction i fills tile rows (i*NW + wave)*RPI + lane/CPR; each reads its token's row
#pragma unroll
      for (int i = 0; i < TL::LA; ++i) {
        const int r = (i * NW + wave) * RPI + lane / CPR;
        const int tok = p.a_rows[m0 + r];
        st.a_offs[i] = tok >= 0
            ? (uint32_t)(((int64_t)tok * p.lda + kswz<BK>(r, lane % CPR) * 8) * 2) : kPastEnd;
        const int r2 = r + 4 * RPI;
        const int tok2 = wave < 4 ? p.a_rows[m0 + r2] : -1;
        st.a_offs_hi[i] = tok2 >= 0
            ? (uint32_t)(((int64_t)tok2 * p.lda + kswz<BK>(r2, lane % CPR) * 8) * 2) : kPastEnd;
      }
      st.a_off0 = 0;
    } else if constexpr (!AMN) {
      const int r = wave * RPI + lane / CPR;
      st.a_off0 = (uint32_t)(((int64_t)r * p.lda + kswz<BK>(r, lane % CPR) * 8) * 2);
    } else {
      constexpr int CPRM = BM / 8;
      static_assert((64 * NW) % (4 * CPRM) == 0, "instruction stride must keep k & 3");
      static_assert(!HD || 256 % (4 * CPRM) == 0, "the upper waves' share must keep k & 3");
      const int f = wave * 64 + lane, k = f / CPRM, cc = (f % CPRM) ^ ((k & 3) << 2);
      st.a_off0 = (uint32_t)(((int64_t)k * p.lda + m0 + cc * 8) * 2);
    }
    if constexpr (!BMN) {
      const int r = wave * RPI + lane / CPR;
      st.b_off0 = (uint32_t)(((int64_t)(n0 + r) * p.ldb + kswz<BK>(r, lane % CPR) * 8) * 2);
    } else {
      constexpr int CPRM = BN / 8;
      static_assert((64 * NW) % (4 * CPRM) == 0, "instruction stride must keep k & 3");
      static_assert(!HD || 256 % (4 * CPRM) == 0, "the upper waves' share must keep k & 3");
      const int f = wave * 64 + lane, k = f / CPRM, cc = (f % CPRM) ^ ((k & 3) << 2);
      st.b_off0 = (uint32_t)(((int64_t)k * p.ldb + n0 + cc * 8) * 2);
    }
  }
  __device__ __forceinline__ uint32_t a_istride(int i) const {
    if constexpr (!AMN) return (uint32_t)((int64_t)i * NW * RPI * p.lda * 2);
    else return (uint32_t)((int64_t)i * (64 * NW / (BM / 8)) * p.lda * 2);
  }
  __device__ __forceinline__ uint32_t b_istride(int i) const {
    if constexpr (!BMN) {
      int64_t row = (int64_t)i * NW * RPI;
      if (Tr::split && row >= BN / 2) row += p.I - BN / 2;   // up rows follow the gate rows
      return (uint32_t)(row * p.ldb * 2);
    } else {
      return (uint32_t)((int64_t)i * (64 * NW / (BN / 8)) * p.ldb * 2);
    }
  }
  // DMA instruction d (0..L-1) of stage kt of tile st into slot. The B operand goes first: for
  // the row-grouped kinds it is the expert weights, streamed once from HBM, so its requests miss
  // L2 and need the longest head start; the A panel is shared by a segment's column tiles and
  // mostly hits L2.
  static constexpr int LB = TL::LB;
  __device__ __forceinline__ void dma_one(const Dma& st, int d, int kt, int slot, int hv = 0) const {
    const uint32_t sl = lds_base + slot * STAGE + hv * 4096;
    if (d < LB) {
      if constexpr (Tr::grouped_rows)   // the expert weights: read once per launch
        dma16_nt(st.rb, st.b_off0 + uniform(kt * b_kstep + b_istride(d) + hv * b_vs),
                 sl + A_BYTES + (d * NW + wave) * 1024);
      else
        dma16(st.rb, st.b_off0 + uniform(kt * b_kstep + b_istride(d) + hv * b_vs),
              sl + A_BYTES + (d * NW + wave) * 1024);
    } else {
      const int i = d - LB;
      if constexpr (GA) dma16(st.ra, (hv ? st.a_offs_hi[i] : st.a_offs[i]) + uniform(kt * a_kstep), sl + (i * NW + wave) * 1024);
      else dma16(st.ra, st.a_off0 + uniform(kt * a_kstep + a_istride(i) + hv * a_vs), sl + (i * NW + wave) * 1024);
    }
  }
  __device__ __forceinline__ void issue_stage(const Dma& st, int kt, int slot) const {
    if constexpr (HD) {
      if (wave < 4) {
#pragma unroll
        for (int d = 0; d < L; ++d) {
          dma_one(st, d, kt, slot, 0);
          dma_one(st, d, kt, slot, 1);
        }
      }
      return;
    }
#pragma unroll
    for (int d = 0; d < L; ++d) dma_one(st, d, kt, slot);
  }

  // ---- fragments ----------------------------------------------------------------------------------
  __device__ __forceinline__ int b_row(int j) const {
    if (Tr::split) return (j / (TN / 2)) * (BN / 2) + wn * (WTN / 2) + (j % (TN / 2)) * 32;
    return wn * WTN + j * 32;
  }
  // K-major: row0 is a multiple of 32, so the row swizzle (r >> 1) & 7 depends on the lane only
  // and slice kk flips bits 5-6 of the lane's offset: one lane offset serves every fragment and
  // slice, the rest is wave-uniform.
  __device__ __forceinline__ uint32_t lane_k() const {
    const int r = lane & 31;
    return (uint32_t)(r * (BK * 2) + (((lane >> 5) ^ ((r >> 1) & 7)) << 4));
  }
  __device__ __forceinline__ bf16x8_t frag_k(int base, int row0, int kk) const {
    return *reinterpret_cast<const bf16x8_t*>(smem + base + row0 * (BK * 2) + (lane_k() ^ (kk << 5)));
  }
  // MN-major: two transposed 8-byte reads give columns col0 + (grp&1)*16 + li,
  // k = kk*16 + (grp>>1)*8 + 0..7. The k-row swizzle uses k & 3, which does not depend on kk, so
  // kk only adds a wave-uniform 32 * rows bytes to a per-fragment lane offset.
  __device__ __forceinline__ bf16x8_t frag_t(int base, int rows, int col0, int kk) const {
    const int grp = lane >> 4, li = lane & 15;
    const int col = col0 + (grp & 1) * 16 + 4 * (li & 3);
    const int cc = col >> 3, half = ((col >> 2) & 1) * 8;
    const int kl = (grp >> 1) * 8 + (li >> 2);
    const int lo_off = kl * rows * 2 + ((cc ^ ((kl & 3) << 2)) * 16) + half;
    const int ad0 = base + kk * 32 * rows + lo_off;
    const int ad1 = ad0 + 8 * rows;   // k + 4
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(s3 + ad0));
    const v4i16_t hi2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(s3 + ad1));
    bf16x8_t r;
    __builtin_memcpy(&r, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &hi2, 8);
    return r;
  }
  // Fragment q of slice kk (q < TM: A block q, else B block q - TM).
  __device__ __forceinline__ void load_one(int slot, int kk, int q, Frags& f) const {
    const int sa = slot * STAGE, sb = sa + A_BYTES;
    if (q < TM) {
      if constexpr (AMN) f.a[q] = frag_t(sa, BM, wm * WTM + q * 32, kk);
      else f.a[q] = frag_k(sa, wm * WTM + q * 32, kk);
    } else {
      if constexpr (BMN) f.b[q - TM] = frag_t(sb, BN, b_row(q - TM), kk);
      else f.b[q - TM] = frag_k(sb, b_row(q - TM), kk);
    }
  }
  __device__ __forceinline__ void load(int slot, int kk, Frags& f) const {
#pragma unroll
    for (int q = 0; q < TM + TN; ++q) load_one(slot, kk, q, f);
  }
  // The slice's MFMAs (A block i against B blocks 0..TN-1, i = 0..TM-1) with DMA instructions
  // [D0, D1) of stage kt_dma of tile st spread evenly among them; with nd < D1 - D0 only the first
  // nd of them are issued. With `nxt` the fragments of the next slice (kk_n of slot_n) are read
  // into fn as those of this one die: A block i after its last MFMA (row i done), B block j after
  // the last row's MFMA with it. So the next slice's first MFMAs find their operands in registers
  // instead of starting with a full LDS round trip.
  // ACT false: a wave with nothing to compute in this tile issues only its DMA share.
  template <int D0, int D1, bool ACT>
  __device__ __forceinline__ void mma_dma(Acc& acc, const Frags& f, bool on, const Dma& st,
                                          int kt_dma, int slot_dma, Frags& fn, int slot_n, int kk_n,
                                          bool nxt, int nd = D1 - D0) const {
    constexpr int N = D1 - D0, T = TM * TN;
    if constexpr (!ACT) {
      if constexpr (N > 0) {
#pragma unroll
        for (int d = 0; d < N; ++d)
          if (on && d < nd) {
            if constexpr (HD) {
              if (wave < 4) {
                dma_one(st, D0 + d, kt_dma, slot_dma, 0);
                dma_one(st, D0 + d, kt_dma, slot_dma, 1);
              }
            } else {
              dma_one(st, D0 + d, kt_dma, slot_dma);
            }
          }
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      acc[t / TN][t % TN] = Mf::run(f.b[t % TN], f.a[t / TN], acc[t / TN][t % TN]);
      if (nxt && (t % TN == TN - 1 || t / TN == TM - 1)) {
        // kept in place: read earlier, a fragment would need registers of its own
        __builtin_amdgcn_sched_barrier(0);
        if (t % TN == TN - 1) load_one(slot_n, kk_n, t / TN, fn);
        if (t / TN == TM - 1) load_one(slot_n, kk_n, TM + t % TN, fn);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (N > 0 && HD) {
        constexpr int N2 = 2 * N;
#pragma unroll
        for (int e2 = 0; e2 < N2; ++e2)
          if (t == e2 * T / N2 && on && e2 / 2 < nd && wave < 4) {
            __builtin_amdgcn_sched_barrier(0);
            dma_one(st, D0 + e2 / 2, kt_dma, slot_dma, e2 & 1);
            __builtin_amdgcn_sched_barrier(0);
          }
      } else if constexpr (N > 0) {
#pragma unroll
        for (int d = 0; d < N; ++d)
          if (t == d * T / N && on && d < nd) {   // d*T/N is in [0, T) for any N
            __builtin_amdgcn_sched_barrier(0);
            dma_one(st, D0 + d, kt_dma, slot_dma);
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    }
  }
  __device__ __forceinline__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
  }

  // Contraction of a tile of nk >= 1 stages, stage kt in slot (s0 + kt) & 1. On entry stage 0
  // is visible to every wavefront and stage 1 (if any) is fully issued. S > 0 with
  // stores_pending: this wave issued S stores after stage 1 (a previous tile's epilogue) that
  // need not wait for it.
  // With `chain` (this tile and the next both have at least two stages) the DMA runs on into the
  // next tile nx: its stage 0 is issued like any other stage during this tile's last two stages
  // and its stage 1 in full during the last slice, so on return the next tile meets the entry
  // condition above with s0' = (s0 + nk) & 1. Without it, at_end() runs once in the last stage,
  // after this wave's last fragment reads are issued and before the last slice's MFMAs.
  // Fragments alternate between two sets: slice kk computes from one while the other receives
  // slice kk + 1 (the next stage's slice 0 after the barrier that makes that stage visible).
  // A wave whose columns of the tile all lie past N (mma_on false) runs the same schedule of DMA
  // and barriers without fragment reads or MFMAs, in a loop of its own, so that neither path
  // keeps the other's registers live.
  template <int S, bool CHAIN, class AtEnd>
  __device__ __forceinline__ void run(Acc& acc, const Dma& cu, int nk, int s0, bool stores_pending,
                                      const Dma& nx, bool chain_, AtEnd at_end) {
    if constexpr (kRagged) {
      if (!mma_on) {
        run_impl<S, CHAIN, false>(acc, cu, nk, s0, stores_pending, nx, chain_, at_end);
        return;
      }
    }
    run_impl<S, CHAIN, true>(acc, cu, nk, s0, stores_pending, nx, chain_, at_end);
  }

  // This wave's DMA instructions per stage (HD: waves 0-3 issue both halves, waves 4-7 none).
  static constexpr int LW = HD ? 2 * L : L;
  // Wait until the DMA of a stage has landed while the `later` stages issued after it (at most
  // one: the ring has two slots) and, with st_out, the S stores issued after those may still be
  // out. vmcnt counts in issue order.
  template <int S>
  __device__ __forceinline__ void wait_later(int later, bool st_out) const {
    static_assert(LW + S < 64, "vmcnt range");
    if constexpr (HD) {
      if (wave >= 4) return;   // issues no DMA
    }
    if (st_out) {
      if constexpr (S > 0) {
        if (later >= 1) wait_vm<LW + S>();
        else wait_vm<S>();
        return;
      }
    }
    if (later >= 1) wait_vm<LW>();
    else wait_vm<0>();
  }
  // The first min(NS, nk) stages of a tile, in full, into slots 0.. (the ring is free).
  __device__ __forceinline__ int issue_first(const Dma& st, int nk) const {
    const int n = min(TL::NS, nk);
#pragma unroll
    for (int s = 0; s < TL::NS; ++s)
      if (s < n) issue_stage(st, s, s);
    return n;
  }

  template <int S, bool CHAIN, bool ACT, class AtEnd>
  __device__ __forceinline__ void run_impl(Acc& acc, const Dma& cu, int nk, int s0,
                                           bool stores_pending, const Dma& nx, bool chain_,
                                           AtEnd at_end) {
    const bool chain = CHAIN && chain_;
    Frags f0, f1;
    if constexpr (ACT) load(s0 & 1, 0, f0);
    for (int kt = 0; kt < nk; ++kt) {
      const int slot = (s0 + kt) & 1;
      // stage kt + 1: this tile's or (chain) the next tile's stage 0; its first DMA part was
      // issued in the previous stage unless it is this tile's stage 1
      const bool nx1 = CHAIN && kt + 1 >= nk;
      const bool pend = kt >= 1 && (kt + 1 < nk || chain);
      const Dma& st1 = nx1 ? nx : cu;
      const int k1 = nx1 ? 0 : kt + 1;
      mma_dma<TL::P1, TL::P2, ACT>(acc, f0, pend, st1, k1, slot ^ 1, f1, slot, 1, true);
      mma_dma<TL::P2, L, ACT>(acc, f1, pend, st1, k1, slot ^ 1, f0, slot, 2, true);
      uint4 cpv = make_uint4(0, 0, 0, 0);
      int cp_r = 0;
      bool cp_on = false;
      if constexpr (CP) {
        const int f = wave * 64 + lane;
        cp_r = cp_nt + (f >> 3) * p.n_tiles_n;
        cp_on = p.out3 != nullptr && cp_r < BM;
        if (cp_on)
          cpv = *reinterpret_cast<const uint4*>(smem + slot * STAGE + cp_r * (BK * 2) +
                                                (kswz<BK>(cp_r, f & 7) << 4));
      }
      mma_dma<0, 0, ACT>(acc, f0, false, cu, 0, 0, f1, slot, 3, true);
      if (kt + 1 < nk || chain) {
        // This wave's DMA of stage kt + 1 has landed and its reads of this slot are done; the
        // barrier makes both true for every wave, so stage kt + 1 is visible and the slot free.
        // (HD: waves 4-7 issue no DMA, and their stores need not land before the barrier)
        if (HD && wave >= 4) {
        } else if (S > 0 && kt == 0 && stores_pending) {
          wait_vm<S>();
        } else {
          wait_vm<0>();
        }
        wait_lgkm0();
        block_barrier();
      }
      if constexpr (CP) {
        if (cp_on)
          *reinterpret_cast<uint4*>(p.out3 + (int64_t)(cp_m0 + cp_r) * p.lda + kt * BK +
                                    ((wave * 64 + lane) & 7) * 8) = cpv;
      }
      // The next stage's slice 0 is read during this slice in every stage: in the last one the
      // reads find whatever the other slot holds and are never used, but made conditional they
      // would keep the old fragments live beside the new ones (a register spill in the loop).
      constexpr bool nxt = true;
      if constexpr (!CHAIN) {
        if (kt + 1 == nk) at_end();
        mma_dma<0, TL::P1, ACT>(acc, f1, kt + 2 < nk, cu, kt + 2, slot, f0, slot ^ 1, 0, nxt);
      } else {
        // stage kt + 2 of the stream: this tile's (first part), the next tile's stage 0 (first
        // part) or the next tile's stage 1 (whole, since that tile starts with it issued)
        if (kt + 1 == nk && !chain) at_end();
        const bool own = kt + 2 < nk;
        mma_dma<0, L, ACT>(acc, f1, own || chain, own ? cu : nx, own ? kt + 2 : kt + 2 - nk, slot,
                      f0, slot ^ 1, 0, nxt, kt + 2 <= nk ? TL::P1 : L);
      }
    }
  }
};

// One tile on the eight-wavefront engine, epilogue through the freed ring.
template <int KIND, class TL, bool GA>
__device__ __forceinline__ void pipe8_tile(const GemmArgs& p, unsigned char* smem, int g, int m0,
                                           int n0, int kbeg, int klen) {
  typedef Eng8<KIND, TL, GA> E;
  E e(p, smem);
  e.set_tile_cols(n0);
  e.cp_m0 = m0;
  e.cp_nt = n0 / tile_cols<KIND>(TL::BN);
  typename E::Dma st;
  e.setup(st, g, m0, n0, kbeg, klen);
  typename E::Acc acc;
  E::zero(acc);
  const int nk = (klen + TL::BK - 1) / TL::BK;
  if (nk > 0) {
    const int n = e.issue_first(st, nk);
    e.template wait_later<0>(n - 1, false);   // stage 0 landed
    block_barrier();
    e.template run<0, false>(acc, st, nk, 0, false, st, false, [] {});
  }
  // Every wavefront is done with the ring: its slots become per-wavefront staging buffers.
  static_assert(TL::NS * TL::STAGE / TL::NW >= 8192, "8 KiB of LDS per wavefront for the epilogue");
  wait_lgkm0();
  block_barrier();
  if (E::kRagged && !e.mma_on) return;   // every column of this wave is at or past N
  store_tile8<KIND, TL::TM, TL::TN, TL::WTM, TL::WTN>(p, acc, g, m0, n0, e.wm, e.wn, e.lane,
                                                      smem + e.wave * (TL::NS * TL::STAGE / TL::NW));
}

// Tall tiles on the eight-wavefront engine: 4 x 2 wavefronts over 256 columns (a ragged last
// column tile, e.g. I = 1408 for the dgrad of the down projection, is cut by the epilogue).
constexpr int kTall8BN = 256;
// Tiles of one or two blocks put a stage's whole DMA out right after the freeing barrier (their
// stage is at most 64 KiB; measured 3-9% faster per kernel on the dense layer's two-block tiles);
// three-block tiles a third per slice (other splits measured within noise there).
template <int ROWS> struct Tall8 {
  static constexpr bool early = ROWS <= 256;
  typedef Tile8<ROWS, kTall8BN, 4, 2, early ? 12 : 4, early ? 12 : 8> type;
};

// Position pos of the dealt order of n row tiles in chunks of q: chunks c = y, y + 8, ... for
// y = 0..7 in turn, rows cq .. cq + q - 1 of each (the last chunk, the only partial one, is the
// last of its class).
__device__ __forceinline__ int dealt_row_tile(int pos, int n, int q) {
  const int nch = (n + q - 1) / q, last = n - (nch - 1) * q;
  int base = 0;
#pragma unroll
  for (int y = 0; y < kNumXcd; ++y) {
    const int cnt = y < nch ? (nch - 1 - y) / kNumXcd + 1 : 0;
    const int rows = cnt * q - ((cnt > 0 && (nch - 1) % kNumXcd == y) ? q - last : 0);
    if (pos < base + rows) {
      const int o = pos - base;
      return (y + kNumXcd * (o / q)) * q + o % q;
    }
    base += rows;
  }
  return n - 1;   // not reached for pos < n
}

// Row-grouped kinds with block_m a multiple of 128: every segment is cut into
// ceil(blocks / max_blk) tiles of whole 128-row blocks, as even as they come (the first `extra`
// tiles one block taller), so no tile is taller than max_blk blocks.
template <int KIND, bool GA>
__global__ __launch_bounds__(kThreads8, 1) void ggemm_tall8_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsBytes];
  int* pref = reinterpret_cast<int*>(smem);   // tiles before group g (reused by the DMA ring)
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = p.G;
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      const int nb = g < G ? (p.seg[g + 1] - p.seg[g]) / kTallBlk : 0;
      int x = (nb + p.max_blk - 1) / p.max_blk;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (g < G) pref[g + 1] = run + x;
      run += __shfl(x, 63, 64);
    }
    if (lane == 0) pref[0] = 0;
  }
  __syncthreads();
  const int64_t n_tiles = pref[G];
  // Each XCD (hardware places workgroup b on XCD b % 8) walks an equal contiguous range of the
  // tiles taken in a dealt order of the row tiles, each row tile with all its column tiles in a
  // row (so the tiles that share its activation panel share that XCD's L2). The dealt order lists
  // chunks of Q = tile_chunk consecutive row tiles (which share a weight panel) class by class:
  // chunks 0, 8, 16, ..., then chunks 1, 9, 17, ..., and so on. Every XCD thus gets about one
  // class, a sample of the whole group order: with skewed routing the segments shrink along that
  // order, and ranges of it would give one XCD the one-block tiles of the rare experts and another
  // the three-block tiles of the popular ones. The ranges are cut by tile count, not at row-tile
  // boundaries, so a few row tiles with many column tiles (a dense layer) still split evenly.
  const int64_t L = xcd_remap(blockIdx.x, n_tiles * p.n_tiles_n);
  int g = 0, ti = 0, nt = 0;
  if (L >= 0) {
    ti = dealt_row_tile((int)(L / p.n_tiles_n), (int)n_tiles, p.tile_chunk);
    nt = (int)(L % p.n_tiles_n);
    int lo = 0, hi = G - 1;   // group of tile ti: largest g with pref[g] <= ti
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= ti) lo = mid; else hi = mid - 1;
    }
    g = lo;
  }
  const int t0 = pref[g], ntg = pref[g + 1] - t0;
  __syncthreads();   // pref is dead from here on: the DMA ring may overwrite it
  if (L < 0) return;
  const int nb = (p.seg[g + 1] - p.seg[g]) / kTallBlk;
  const int local = ti - t0, base = nb / ntg, extra = nb % ntg;
  const int blk0 = local * base + min(local, extra), nblk = base + (local < extra ? 1 : 0);
  const int m0 = p.seg[g] + blk0 * kTallBlk;
  const int n0 = nt * tile_cols<KIND>(kTall8BN);
  if (nblk == 3) pipe8_tile<KIND, Tall8<384>::type, GA>(p, smem, g, m0, n0, 0, p.K);
  else if (nblk == 2) pipe8_tile<KIND, Tall8<256>::type, GA>(p, smem, g, m0, n0, 0, p.K);
  else pipe8_tile<KIND, Tall8<128>::type, GA>(p, smem, g, m0, n0, 0, p.K);
}

// Row-grouped kinds with 64-row tiles (block_m == 64): one block per tile, from tile_group.
template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void ggemm_block64_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[Block64Tile::STAGES * Block64Tile::STAGE];
  const int total = p.total_rows[0];
  const int64_t L = xcd_remap(blockIdx.x, (int64_t)(total / 64) * p.n_tiles_n);
  if (L < 0) return;
  const int mt = (int)(L / p.n_tiles_n), nt = (int)(L % p.n_tiles_n);
  const int m0 = mt * 64;
  const int g = p.tile_group[m0 / p.block_m];
  const int n0 = nt * tile_cols<KIND>(Block64Tile::BN);
  pipe_tile<KIND, Block64Tile>(p, smem, g, m0, n0, 0, p.K);
}

// Weight-gradient kinds: 256 weight rows x 256 columns per tile, contraction over the segment's
// rows (both operands MN-major in HBM). The contraction is short (one segment), so a tile's
// fixed costs (first DMA, 128 KiB of stores) are as large as its MFMAs: the kernel is persistent,
// one workgroup per CU walking its XCD's tiles, and it issues the next tile's first two stages
// before storing the current tile, so the stores drain under the next tile's MFMAs.
// A stage's whole DMA (issued by waves 0-3) goes out in the slice right after the freeing barrier:
// with the stores of the previous tile in the same queues, the earliest start pays (2-4% against
// a third per slice).
typedef Tile8<256, 256, 4, 2, 12, 12> Wgrad8Tile;
constexpr int kStoreNT = 2;   // cache-policy operand of buffer stores: non-temporal
constexpr int kWgradScr = 4096;                     // epilogue staging per wavefront
// A weight-gradient tile's fixed cost in stage times (first DMA latency, 128 KiB of stores): at
// the benchmark shape tiles of 6 stages take about 16 us and tiles of 48 stages about 95 us.
constexpr int kWgradTileFixed = 3;

// Sum and inclusive prefix sum of an int64 over the 64 lanes of a wavefront.
__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}
__device__ __forceinline__ int64_t wave_sum_i64(int64_t x) {
  return __shfl(wave_incl_scan_i64(x), 63, 64);
}
// Stores per wavefront per tile: bf16 dW in 32 x 64 passes (4 stores each); fp32 dW in 32 x 32
// passes (4 stores each, twice as many passes).
template <bool F32> constexpr int wgrad_stores() {
  return Wgrad8Tile::TM * (F32 ? Wgrad8Tile::TN : Wgrad8Tile::TN / 2) * 4;
}
static_assert(Wgrad8Tile::NS * Wgrad8Tile::STAGE + Wgrad8Tile::NW * kWgradScr <= kLdsBytes,
              "LDS budget");
static_assert((Wgrad8Tile::NS - 1) * Wgrad8Tile::L + wgrad_stores<true>() < 64, "vmcnt range");

// Epilogue with 32 x 64 (bf16) or 32 x 32 (fp32) staging passes and bounds-checked buffer stores:
// lanes outside the weight matrix get an offset past the buffer's end, which the hardware drops,
// so every wavefront issues exactly wgrad_stores<F32>() stores per tile (the kernel's vmcnt waits
// count them).
template <bool F32, int TM, int TN, int WTM, int WTN>
__device__ __forceinline__ void store_wgrad8(const GemmArgs& p, const f32x16_t (&acc)[TM][TN],
                                             int g, int m0, int n0, int wm, int wn, int lane,
                                             unsigned char* scr) {
  static_assert(TM * (F32 ? TN : TN / 2) * 4 == wgrad_stores<F32>(), "store count");
  constexpr int EB = F32 ? 4 : 2;   // bytes per element
  unsigned char* out = reinterpret_cast<unsigned char*>(p.out) + (int64_t)g * p.o_gstride * EB;
  const uint32_t bytes = (uint32_t)((int64_t)p.M * p.ldo * EB);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(out, 0, (int)bytes, 0x00020000);
  typedef uint32_t v4_t __attribute__((ext_vector_type(4)));
  auto put = [&](int m, int col, v4_t v) {
    const uint32_t off =
        (m < p.M && col < p.N) ? (uint32_t)(((int64_t)m * p.ldo + col) * EB) : 0x80000000u;
    // non-temporal: dW is written once and read by no later kernel here, so it should not evict
    // the activation panels the next tiles read from L2
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStoreNT);
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mrow = m0 + wm * WTM + i * 32;
    if constexpr (F32) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int c0 = n0 + wn * WTN + j * 32;
        stage_f32<1>(scr, lane, [&](int, int q, int e) { return acc[i][j][4 * q + e]; },
            [&](int rr, int c, float4 d) {
              const v4_t v = {__float_as_uint(d.x), __float_as_uint(d.y), __float_as_uint(d.z),
                              __float_as_uint(d.w)};
              put(mrow + rr, c0 + c, v);
            });
      }
    } else {
#pragma unroll
      for (int h = 0; h < TN / 2; ++h) {
        const int c0 = n0 + wn * WTN + h * 64;
        stage_bf16<2>(scr, lane, [&](int j, int q, int e) { return acc[i][2 * h + j][4 * q + e]; },
            [&](int rr, int c, uint4 d) {
              const v4_t v = {d.x, d.y, d.z, d.w};
              put(mrow + rr, c0 + c, v);
            });
      }
    }
  }
}

// A wave-uniform read of a read-only int array through the scalar data cache (the constant
// address space), so it does not join the vector-memory queue that the DMA waits count.
__device__ __forceinline__ int ld_scalar(const int32_t* a, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)a)[i];
}

template <int KIND, bool F32>
__global__ __launch_bounds__(kThreads8, 1) void ggemm_wgrad8_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsBytes];
  typedef Wgrad8Tile TL;
  typedef Eng8<KIND, TL> E;
  constexpr int S = wgrad_stores<F32>(), L = TL::L;
  const int64_t per_g = (int64_t)p.n_tiles_m * p.n_tiles_n, total = per_g * p.G;
  const int xcd = blockIdx.x % kNumXcd, nwg = gridDim.x / kNumXcd;
  // Each XCD walks a contiguous range of tiles (groups in order, so tiles that share operand
  // panels share its L2), cut so that every XCD gets an eighth of the estimated work: a tile of a
  // segment with nk stages costs nk + kWgradTileFixed stage times (its first DMA and its stores).
  // With skewed routing equal tile counts would leave most of the work to the XCDs that hold the
  // popular experts.
  int64_t lbeg, lend;
  {
    int64_t* sb = reinterpret_cast<int64_t*>(smem);   // [2]; the DMA ring takes the LDS afterwards
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      auto tile_cost = [&](int g) -> int64_t {
        if (g >= p.G) return 0;
        const int klen = ld_scalar(p.seg, g + 1) - ld_scalar(p.seg, g);
        return (klen + TL::BK - 1) / TL::BK + kWgradTileFixed;
      };
      int64_t all = 0;
      for (int base = 0; base < p.G; base += 64) all += wave_sum_i64(per_g * tile_cost(base + lane));
      const int64_t thr0 = all * xcd / kNumXcd, thr1 = all * (xcd + 1) / kNumXcd;
      // the first tile whose preceding work reaches thr, inside the group that spans thr
      int64_t run = 0;
      for (int base = 0; base < p.G; base += 64) {
        const int g = base + lane;
        const int64_t tc = tile_cost(g), c = per_g * tc;
        const int64_t incl = wave_incl_scan_i64(c), pre = run + incl - c;
        if (c > 0 && pre <= thr0 && thr0 < pre + c) sb[0] = g * per_g + (thr0 - pre + tc - 1) / tc;
        if (c > 0 && pre <= thr1 && thr1 < pre + c) sb[1] = g * per_g + (thr1 - pre + tc - 1) / tc;
        run += __shfl(incl, 63, 64);
      }
      if (lane == 0 && thr1 >= all) sb[1] = total;   // the last XCD's range ends with the tiles
    }
    __syncthreads();
    lbeg = sb[0];
    lend = sb[1];
    __syncthreads();
  }
  int64_t l = lbeg + blockIdx.x / kNumXcd;
  if (l >= lend) return;
  struct T { int g, m0, n0, kbeg, klen, nk; };
  const bool m_fast = p.M <= p.N;
  auto decode = [&](int64_t L0) {
    T t;
    t.g = (int)(L0 / per_g);
    const int rem = (int)(L0 % per_g);
    // Within a group the tiles along the smaller of M and N vary fastest: the 32 workgroups of
    // an XCD then cover every panel of the operand with the smaller segment slice, which stays
    // in L2 while the other operand's panels stream past once.
    if (m_fast) {
      t.m0 = (rem % p.n_tiles_m) * TL::BM;
      t.n0 = (rem / p.n_tiles_m) * TL::BN;
    } else {
      t.m0 = (rem / p.n_tiles_n) * TL::BM;
      t.n0 = (rem % p.n_tiles_n) * TL::BN;
    }
    t.kbeg = ld_scalar(p.seg, t.g);
    t.klen = ld_scalar(p.seg, t.g + 1) - t.kbeg;
    t.nk = (t.klen + TL::BK - 1) / TL::BK;
    return t;
  };
  E e(p, smem);
  constexpr int NS = TL::NS;
  unsigned char* scr = smem + NS * TL::STAGE + e.wave * kWgradScr;
  typename E::Dma dc, dn;   // DMA state of the current and the next tile
  T cur = decode(l);
  e.setup(dc, cur.g, cur.m0, cur.n0, cur.kbeg, cur.klen);
  e.issue_first(dc, cur.nk);
  int s0 = 0;             // slot of the current tile's stage 0
  bool stores = false;    // this wave's previous-tile stores are queued after the first stages
  bool ready = false;     // the current tile's stage 0 is already visible (chained DMA)
  for (;;) {
    if (!ready) {
      // stage 0 of this tile has landed (the later first stages and the previous tile's stores
      // may be out)
      if (cur.nk > 0) e.template wait_later<S>(min(NS, cur.nk) - 1, stores);
      block_barrier();
    }
    typename E::Acc acc;
    E::zero(acc);
    e.set_tile_cols(cur.n0);
    const int64_t ln = l + nwg;
    const bool has_next = ln < lend;
    T nxt = cur;
    if (has_next) {
      nxt = decode(ln);
      e.setup(dn, nxt.g, nxt.m0, nxt.n0, nxt.kbeg, nxt.klen);
    }
    // The next tile's first stages follow this tile's in the same DMA stream when both have at
    // least two; otherwise they are issued, whole, once every wave is done with the ring.
    const bool chain = has_next && cur.nk >= NS && nxt.nk >= NS;
    auto at_end = [&] {
      wait_lgkm0();
      block_barrier();
      if (has_next) e.issue_first(dn, nxt.nk);
    };
    if (cur.nk > 0) e.template run<S, true>(acc, dc, cur.nk, s0, stores, dn, chain, at_end);
    else at_end();
    store_wgrad8<F32, TL::TM, TL::TN, TL::WTM, TL::WTN>(p, acc, cur.g, cur.m0, cur.n0, e.wm, e.wn,
                                                   e.lane, scr);
    if (!has_next) break;
    s0 = chain ? (s0 + cur.nk) & (NS - 1) : 0;
    ready = chain;
    l = ln;
    cur = nxt;
    dc = dn;
    stores = true;
  }
}

// Workgroups of a persistent launch: one per CU of MI355X (8 XCDs x 32 CUs), fewer for small
// problems; a multiple of the XCD count so every XCD gets the same number.
constexpr int kPersistentWgs = kNumXcd * 32;
unsigned persistent_grid(int64_t tiles) {
  const int64_t per_xcd = (tiles + kNumXcd - 1) / kNumXcd;
  return (unsigned)(kNumXcd * (per_xcd < kPersistentWgs / kNumXcd ? per_xcd : kPersistentWgs / kNumXcd));
}

template <int KIND, int BM, int BN, int MS, int WAVES_M>
hipError_t launch_kind(const GemmArgs& a, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ggemm_kernel<KIND, BM, BN, MS, WAVES_M>), dim3((unsigned)grid),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// Tallest tile for a row-grouped launch of n_tiles_n column tiles over `rows` real rows in G
// groups. The segment sizes live on the device, so the host prices an even split (rows / G per
// group, rounded up to whole blocks): per choice of at most 3 or 2 blocks a tile, the number of
// waves of 256 tiles times the tallest tile's cost. A 256-row tile does 2/3 of the work of a
// 384-row one at a lower matrix-unit rate (about 1/1.1). The estimate is rough for skewed
// routing, so 2 must win by a tenth. Few long segments choose it: 64 blocks x 16 column tiles
// (a dense layer of 8192 tokens, N = 4096) make 352 tiles of 384 rows, 1.4 waves, or 512 tiles
// of 256 rows, two whole waves.
int tall_max_blk(int64_t rows, int G, int n_tiles_n) {
  if (rows <= 0 || G <= 0) return kTallMaxBlk;
  const int64_t nb = (rows + (int64_t)G * kTallBlk - 1) / ((int64_t)G * kTallBlk);   // >= 1
  auto cost = [&](int mb) {
    const int64_t per_g = (nb + mb - 1) / mb;                 // tiles of one group
    const int64_t tallest = (nb + per_g - 1) / per_g;
    const int64_t waves = (per_g * G * n_tiles_n + kPersistentWgs - 1) / kPersistentWgs;
    return (double)waves * (double)tallest * (tallest >= 3 ? 1.0 : 1.1);
  };
  return cost(2) < 0.9 * cost(kTallMaxBlk) ? 2 : kTallMaxBlk;
}

// Row tiles of one segment share its weight panel, so the tall kernels' dealt order keeps chunks
// of Q consecutive row tiles together: Q is the row tiles of an even split's segment (rows / G,
// whole blocks, at most max_blk a tile), a power of two up to 8, and at most an eighth of all the
// row tiles. Uniform 384-row segments take 1; one GPU's share under 8-way expert parallelism
// (3072-row segments) 8, which keeps each expert on one XCD; the skewed layer (about 8 blocks a
// segment) 2; a dense layer of 8192 rows 2 (22 row tiles) or 4 (32).
int tall_tile_chunk(int64_t rows, int G, int max_blk) {
  if (rows <= 0 || G <= 0) return 1;
  const int64_t nb = (rows + (int64_t)G * kTallBlk - 1) / ((int64_t)G * kTallBlk);   // >= 1
  const int64_t per_g = (nb + max_blk - 1) / max_blk;
  const int64_t cap = per_g * G / kNumXcd;
  int q = 1;
  while (q < 8 && 2 * q <= per_g && 2 * q <= cap) q *= 2;
  return q;
}

// Row-grouped kinds: tall tiles for block_m % 128 == 0, 64-row tiles for block_m == 64, the
// register-staged engine for 16 and 32.
// *rows_copied (if given) tells whether the launch writes a.out3 (the gathered gate/up product
// on tall tiles, where each row tile has enough column tiles to share out its rows).
template <int KIND>
hipError_t launch_rows(GemmArgs a, int64_t mcap, int64_t rows, hipStream_t st,
                       bool* rows_copied = nullptr) {
  if (rows_copied) *rows_copied = false;
  if (a.block_m % kTallBlk == 0) {
    if (a.seg == nullptr) return hipErrorInvalidValue;
    constexpr int cols = tile_cols<KIND>(kTall8BN);
    a.n_tiles_n = (int)((a.N + cols - 1) / cols);
    a.max_blk = tall_max_blk(rows, a.G, a.n_tiles_n);
    // sum over groups of ceil(nb_g / mb) <= (sum nb_g + (mb - 1) G) / mb, sum nb_g <= mcap / 128
    const int64_t tiles = (mcap / kTallBlk + (a.max_blk - 1) * (int64_t)a.G) / a.max_blk + 1;
    a.tile_chunk = tall_tile_chunk(rows, a.G, a.max_blk);
    const int64_t grid = (tiles * a.n_tiles_n + kNumXcd - 1) / kNumXcd * kNumXcd;
    if constexpr (KIND == kFwdGateUp) {
      if (a.a_rows) {
        // each of a row tile's n_tiles_n workgroups copies every n_tiles_n-th row of its stages,
        // at most 64 rows a stage (8 lanes of 16 bytes per 128-byte row stage)
        if (a.out3 && a.n_tiles_n * 64 < a.max_blk * kTallBlk) a.out3 = nullptr;
        if (rows_copied) *rows_copied = a.out3 != nullptr;
        hipLaunchKernelGGL((ggemm_tall8_kernel<KIND, true>), dim3((unsigned)grid), dim3(kThreads8),
                           0, st, a);
        return hipGetLastError();
      }
    } else {
      if (a.a_rows) return hipErrorInvalidValue;   // only the gate/up product gathers its rows
    }
    hipLaunchKernelGGL((ggemm_tall8_kernel<KIND, false>), dim3((unsigned)grid), dim3(kThreads8), 0,
                       st, a);
    return hipGetLastError();
  }
  if (a.tile_group == nullptr || a.total_rows == nullptr) return hipErrorInvalidValue;
  if (a.block_m == 64) {
    a.n_tiles_n = (int)((a.N + tile_cols<KIND>(Block64Tile::BN) - 1) / tile_cols<KIND>(Block64Tile::BN));
    const int64_t grid = ((mcap / 64) * a.n_tiles_n + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL((ggemm_block64_kernel<KIND>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  const int n_per_tile = KindTraits<KIND>::split ? 128 : 256;
  a.n_tiles_n = (int)((a.N + n_per_tile - 1) / n_per_tile);
  const int64_t grid = ((mcap / a.block_m) * a.n_tiles_n + kNumXcd - 1) / kNumXcd * kNumXcd;
  switch (a.block_m) {
    case 32: return launch_kind<KIND, 32, 256, 32, 1>(a, grid, st);
    case 16: return launch_kind<KIND, 16, 256, 16, 1>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_ggemm_fwd(const moe_shape_t& s, uint32_t which, int64_t mcap,
                            const uint16_t* x_perm, const int32_t* row_token,
                            const int32_t* seg_offsets, const int32_t* tile_group,
                            const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                            uint16_t* h_save, uint16_t* a, uint16_t* y_perm, uint16_t* x_perm_out,
                            hipStream_t st) {
  GemmArgs g{};
  g.block_m = s.block_m;
  g.I = s.I;
  g.G = s.E + s.S;
  const int64_t rows = (int64_t)s.T * (s.K + s.S);   // real (unpadded) permuted rows
  g.seg = seg_offsets;
  g.tile_group = tile_group;
  g.total_rows = total_rows;
  // gate/up + SwiGLU: N counts gate columns (I); each tile covers BN/2 gate + BN/2 up columns.
  // With row_token the A operand is x[T,H] itself, each row read through the permutation map.
  g.a = x_perm; g.lda = s.H;
  g.a_rows = row_token;
  g.a_bytes = row_token ? (int64_t)s.T * s.H * 2 : 0;
  g.b = w1; g.ldb = s.H; g.b_gstride = (int64_t)2 * s.I * s.H;
  g.out = a; g.ldo = s.I; g.out2 = h_save;
  g.out3 = row_token ? x_perm_out : nullptr;
  g.N = s.I; g.K = s.H;
  if (which & MOE_FWD_GATEUP) {
    bool copied = false;
    hipError_t e = launch_rows<kFwdGateUp>(g, mcap, rows, st, &copied);
    if (e != hipSuccess) return e;
    if (g.out3 && !copied) {   // the launch could not write x_perm from its stages
      e = launch_gather_rows(s, mcap, total_rows, row_token, x_perm, x_perm_out, st);
      if (e != hipSuccess) return e;
    }
  }
  if (!(which & MOE_FWD_DOWN)) return hipSuccess;
  // down
  g.a = a; g.lda = s.I;
  g.a_rows = nullptr; g.a_bytes = 0; g.out3 = nullptr;
  g.b = w2; g.ldb = s.I; g.b_gstride = (int64_t)s.H * s.I;
  g.out = y_perm; g.ldo = s.H; g.out2 = nullptr;
  g.N = s.H; g.K = s.I;
  return launch_rows<kFwdDown>(g, mcap, rows, st);
}

hipError_t launch_ggemm_dgrad(const moe_shape_t& s, uint32_t which, int64_t mcap,
                              const uint16_t* dy_perm, const uint16_t* h_save,
                              const int32_t* seg_offsets, const int32_t* tile_group,
                              const int32_t* total_rows, const uint16_t* w1, const uint16_t* w2,
                              uint16_t* dh, uint16_t* dx_perm, hipStream_t st) {
  GemmArgs g{};
  g.block_m = s.block_m;
  g.I = s.I;
  g.G = s.E + s.S;
  const int64_t rows = (int64_t)s.T * (s.K + s.S);   // real (unpadded) permuted rows
  g.seg = seg_offsets;
  g.tile_group = tile_group;
  g.total_rows = total_rows;
  // da = dy_perm . W2[g] ([H, I] read as [K=H][N=I]) with the SwiGLU backward epilogue -> dh.
  g.a = dy_perm; g.lda = s.H;
  g.b = w2; g.ldb = s.I; g.b_gstride = (int64_t)s.H * s.I;
  g.aux = h_save; g.out = dh;
  g.N = s.I; g.K = s.H;
  if (which & MOE_DGRAD_DOWN) {
    hipError_t e = launch_rows<kDgradDown>(g, mcap, rows, st);
    if (e != hipSuccess) return e;
  }
  if (!(which & MOE_DGRAD_GATEUP)) return hipSuccess;
  // dx_perm = dh . W1[g] ([2I, H] read as [K=2I][N=H]).
  g.a = dh; g.lda = 2 * (int64_t)s.I;
  g.b = w1; g.ldb = s.H; g.b_gstride = (int64_t)2 * s.I * s.H;
  g.aux = nullptr; g.out = dx_perm; g.ldo = s.H;
  g.N = s.H; g.K = 2 * s.I;
  return launch_rows<kDgradGateUp>(g, mcap, rows, st);
}

namespace {
template <int KIND>
hipError_t launch_wgrad_kind(const GemmArgs& g, bool f32, hipStream_t st) {
  const int64_t tiles = (int64_t)g.G * g.n_tiles_m * g.n_tiles_n;
  if (f32)
    hipLaunchKernelGGL((ggemm_wgrad8_kernel<KIND, true>), dim3(persistent_grid(tiles)),
                       dim3(kThreads8), 0, st, g);
  else
    hipLaunchKernelGGL((ggemm_wgrad8_kernel<KIND, false>), dim3(persistent_grid(tiles)),
                       dim3(kThreads8), 0, st, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_ggemm_wgrad(const moe_shape_t& s, uint32_t which, const uint16_t* x_perm,
                              const uint16_t* a,
                              const uint16_t* dy_perm, const uint16_t* dh,
                              const int32_t* seg_offsets, void* dw1, void* dw2, bool f32,
                              hipStream_t st) {
  GemmArgs g{};
  g.I = s.I;
  g.G = s.E + s.S;
  g.seg = seg_offsets;
  if (which & MOE_WGRAD_DOWN) {
    // dW2[g] [H, I] = dy_perm_seg^T . a_seg
    g.a = dy_perm; g.lda = s.H;
    g.b = a; g.ldb = s.I;
    g.out = static_cast<uint16_t*>(dw2); g.ldo = s.I; g.o_gstride = (int64_t)s.H * s.I;
    g.M = s.H; g.N = s.I;
    g.n_tiles_m = (g.M + Wgrad8Tile::BM - 1) / Wgrad8Tile::BM;
    g.n_tiles_n = (g.N + Wgrad8Tile::BN - 1) / Wgrad8Tile::BN;
    const hipError_t e = launch_wgrad_kind<kWgradDown>(g, f32, st);
    if (e != hipSuccess) return e;
  }
  if (!(which & MOE_WGRAD_GATEUP)) return hipSuccess;
  // dW1[g] [2I, H] = dh_seg^T . x_perm_seg
  g.a = dh; g.lda = 2 * (int64_t)s.I;
  g.b = x_perm; g.ldb = s.H;
  g.out = static_cast<uint16_t*>(dw1); g.ldo = s.H; g.o_gstride = (int64_t)2 * s.I * s.H;
  g.M = 2 * s.I; g.N = s.H;
  g.n_tiles_m = (g.M + Wgrad8Tile::BM - 1) / Wgrad8Tile::BM;
  g.n_tiles_n = (g.N + Wgrad8Tile::BN - 1) / Wgrad8Tile::BN;
  return launch_wgrad_kind<kWgradGateUp>(g, f32, st);
}

}  // namespace moe
