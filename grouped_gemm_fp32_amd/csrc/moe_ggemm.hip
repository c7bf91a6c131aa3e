// Grouped GEMM engine of the MoE expert FFN on gfx950 (bf16 MFMA, fp32 accumulation).
//
// dots.llm1 Technical Report, section 3.2 "Efficient grouped GEMM": every expert's token segment
// is padded to a fixed block size that is a multiple of the matrix instruction's M, so all rows of
// a workgroup tile belong to one expert and the grouped GEMM is scheduled like an ordinary GEMM.
// Section A2 (MoE paragraph): each expert is a two-layer FFN with SwiGLU.
//
// On gfx950 the instruction is v_mfma_f32_32x32x16_bf16 (or 16x16x32 for 16-row tiles); the
// workgroup tile is BM x BN x 64 with BM dividing block_m, four wavefronts, and both operands
// staged through LDS as K-contiguous rows (operands stored the other way round in HBM are
// transposed 8x8 in registers on the way in). Tiles are ordered so that consecutive ones share
// an M-block (and an expert), and mapped to XCDs so that they also share an L2.
//
// Six kinds of tile share the engine:
//   FwdGateUp   h = x_perm . W1[g]^T, fused a = silu(h_gate) * h_up (and h_save)
//   FwdDown     y_perm = a . W2[g]^T
//   DgradDown   da = dy_perm . W2[g], fused SwiGLU backward -> dh
//   DgradGateUp dx_perm = dh . W1[g]
//   WgradDown   dW2[g] = dy_perm_seg^T . a_seg        (contraction over the segment's rows)
//   WgradGateUp dW1[g] = dh_seg^T . x_perm_seg
#include "moe_common.h"
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
  const uint16_t* b;   // B source
  int64_t lda, ldb;
  int64_t b_gstride;   // elements per group of the B source (weights); 0 for wgrad
  const uint16_t* aux; // h_save read by the SwiGLU backward epilogue
  uint16_t* out;
  int64_t ldo;
  int64_t o_gstride;   // elements per group of the output (wgrad)
  uint16_t* out2;      // h_save written by the forward gate/up epilogue (may be null)
  int M, N, K, I;
  int block_m;
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
    const int64_t n_valid = (int64_t)(total / BM) * p.n_tiles_n;
    const int64_t L = xcd_remap(blockIdx.x, n_valid);
    if (L < 0) return;
    const int mt = (int)(L / p.n_tiles_n), nt = (int)(L % p.n_tiles_n);
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
  const uint16_t* a_rows = p.a + (int64_t)m0 * p.lda;
  const uint16_t* b_grp = p.b + (int64_t)g * p.b_gstride;
  auto a_row = [&](int r) -> const uint16_t* { return a_rows + (int64_t)r * p.lda; };
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
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < Mf::groups; ++q) {
          const int c = n0 + wn * WTN + j * MS + Mf::out_n(lane, q);
          if (c >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          if constexpr (KIND == kDgradDown) {
            // da -> dh = [da*u*s*(1 + g(1-s)) | da*g*s] with g, u from h_save (bf16).
            const int64_t hrow = m * (2 * (int64_t)p.I);
            const uint2 gw = *reinterpret_cast<const uint2*>(p.aux + hrow + c);
            const uint2 uw = *reinterpret_cast<const uint2*>(p.aux + hrow + p.I + c);
            const float gg[4] = {lo_bf(gw.x), hi_bf(gw.x), lo_bf(gw.y), hi_bf(gw.y)};
            const float uu[4] = {lo_bf(uw.x), hi_bf(uw.x), lo_bf(uw.y), hi_bf(uw.y)};
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float s = 1.0f / (1.0f + expf(-gg[e]));
              dg[e] = v[e] * uu[e] * s * (1.0f + gg[e] * (1.0f - s));
              du[e] = v[e] * gg[e] * s;
            }
            *reinterpret_cast<uint2*>(p.out + hrow + c) =
                make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(p.out + hrow + p.I + c) =
                make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          } else {
            *reinterpret_cast<uint2*>(out + m * p.ldo + c) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
          }
        }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// DMA engine (tiles of 64 to 256 rows). Taller tiles load fewer bytes per FLOP, and a segment is a
// whole number of 128-row blocks of one expert, so a tile may take two consecutive blocks
// (256 rows) and still belong to a single expert. Each workgroup derives its tile from
// seg_offsets: group g has ceil(len_g / 256) tiles of 256 rows, the last one 128 or 256.
// (Measured on MI355X at 8192 tokens x 128 experts: 384-row tiles, which only fit two LDS
// stages and 384 accumulators, ran 1.7x slower than 256-row tiles.)
// Weight-gradient tiles are 256 weight rows.
//
// Every operand goes from HBM to LDS through the bounds-checked buffer->LDS DMA
// (buffer_load_dwordx4 ... lds): lane l of a wavefront deposits its 16 bytes at LDS base + 16 l,
// whatever address it loaded, and reads past the buffer resource's size return zero (tile tails
// and segment ends need no special code). A ring of two or three LDS stages, one barrier per
// k-step.
//   K-major operand (K contiguous in HBM): LDS [rows][64], 16-byte chunk c of row r stored at
//     position c ^ (r & 7) so the MFMA fragment reads (32 rows, one chunk) hit 8 distinct bank
//     groups.
//   MN-major operand (rows contiguous in HBM, [k][rows]): LDS [64][rows] as in HBM, chunk cc of
//     k-row k stored at cc ^ ((k & 3) << 2); fragments come from ds_read_tr16_b64, which hands
//     each lane 4 consecutive k of one column (within 16 lanes: lane i, item q <- lane 4q + i/4,
//     item i % 4), two reads per 32x32x16 operand.
// Four wavefronts in 2 x 2, each (BM/2) x 128 of the BM x 256 tile.
// ------------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));

// Buffer resource (gfx9 layout): 48-bit base, stride 0, num_records = bytes, raw dword format.
__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ v4u32_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes);
  const uint64_t a = (uint64_t)(uintptr_t)base;
  v4u32_t r;
  r.x = uniform((uint32_t)a);
  r.y = uniform((uint32_t)(a >> 32) & 0xffffu);
  r.z = uniform(n);
  r.w = 0x00020000u;
  return r;
}

// Bounds-checked DMA of 16 bytes per lane from a buffer resource into LDS at lds_wave + 16 * lane. Issued from asm: the instruction has no register result (it
// writes LDS through M0), and hiding it from the compiler keeps it from draining every DMA
// before unrelated LDS reads; the kernel's own vmcnt waits and barriers order the data.
__device__ __forceinline__ void dma16(v4u32_t r, uint32_t voff, uint32_t lds_wave) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(uniform(lds_wave)), "v"(voff), "s"(r) : "memory", "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) (LDS reads retired), vmcnt and expcnt left at their maxima.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));

// N transposed 8-byte LDS reads (ds_read_b64_tr_b16) in one asm block that also waits for them,
// so the results are complete when the block ends. addr: LDS byte addresses.
template <int N>
__device__ __forceinline__ void tr_read(v2u32_t (&v)[N], const uint32_t (&addr)[N]);

template <>
__device__ __forceinline__ void tr_read<8>(v2u32_t (&v)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

template <>
__device__ __forceinline__ void tr_read<12>(v2u32_t (&v)[12], const uint32_t (&a)[12]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %12\n\tds_read_b64_tr_b16 %1, %13\n\t"
      "ds_read_b64_tr_b16 %2, %14\n\tds_read_b64_tr_b16 %3, %15\n\t"
      "ds_read_b64_tr_b16 %4, %16\n\tds_read_b64_tr_b16 %5, %17\n\t"
      "ds_read_b64_tr_b16 %6, %18\n\tds_read_b64_tr_b16 %7, %19\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\tds_read_b64_tr_b16 %9, %21\n\t"
      "ds_read_b64_tr_b16 %10, %22\n\tds_read_b64_tr_b16 %11, %23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
        "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11])
      : "memory");
}

template <>
__device__ __forceinline__ void tr_read<4>(v2u32_t (&v)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\tds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

constexpr int kLdsBytes = 163840;   // gfx950: 160 KiB of LDS per workgroup
constexpr int kTallRows = 256;      // tallest row-grouped tile (two 128-row blocks)

template <int BM> struct DmaCfg {
  static constexpr int BN = 256, WTM = BM / 2, WTN = BN / 2, TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_BYTES = BM * kBK * 2, B_BYTES = BN * kBK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int STAGES = 3 * STAGE <= kLdsBytes ? 3 : 2;
  static constexpr int LA = A_BYTES / 4096, LB = B_BYTES / 4096;  // DMA instr per lane per stage
  static_assert(2 * STAGE <= kLdsBytes, "two stages must fit in LDS");
};

// One BM x 256 output tile: rows m0.. of group g (row-grouped kinds) or weight rows m0.. of group
// g (wgrad), contraction over [kbeg, kbeg + klen).
template <int KIND, int BM>
__device__ __forceinline__ void dma_tile(const GemmArgs& p, unsigned char* smem, uint32_t lds_base,
                                         int g, int m0, int n0, int kbeg, int klen) {
  typedef KindTraits<KIND> Tr;
  typedef Mfma<32> Mf;
  typedef DmaCfg<BM> C;
  constexpr int BN = C::BN, WTM = C::WTM, WTN = C::WTN, TM = C::TM, TN = C::TN;
  constexpr int A_BYTES = C::A_BYTES, STAGE = C::STAGE, STAGES = C::STAGES;
  constexpr int LA = C::LA, LB = C::LB;
  constexpr bool AMN = Tr::a_trans, BMN = Tr::b_trans;
  static_assert(!Tr::split || TN == 4, "split needs 2 gate + 2 up sub-tiles");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- buffer resources: each covers exactly the bytes this tile may read ----------------------
  v4u32_t ra, rb;
  if (AMN) ra = make_rsrc(p.a + (int64_t)kbeg * p.lda, (int64_t)klen * p.lda * 2);
  else ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (int64_t)BM * p.lda * 2);
  const uint16_t* b_grp = p.b + (int64_t)g * p.b_gstride;
  if (Tr::grouped_rows) rb = make_rsrc(b_grp, p.b_gstride * 2);
  else rb = make_rsrc(p.b + (int64_t)kbeg * p.ldb, (int64_t)klen * p.ldb * 2);

  // ---- per-lane DMA byte offsets of stage 0 (a k-step adds a fixed stride) ---------------------
  // K-major: instruction i of wave w fills rows (i*4 + w)*8 .. +8; lane -> row + chunk position.
  // MN-major: instruction i of wave w fills flat chunks (i*4 + w)*64 + lane of [64][ROWS].
  uint32_t a_off[LA], b_off[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    if (!AMN) {
      const int r = (i * 4 + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      a_off[i] = (uint32_t)(((int64_t)r * p.lda + c * 8) * 2);
    } else {
      constexpr int CPR = BM / 8;
      const int f = (i * 4 + wave) * 64 + lane;
      const int k = f / CPR, cc = (f % CPR) ^ ((k & 3) << 2);
      a_off[i] = (uint32_t)(((int64_t)k * p.lda + m0 + cc * 8) * 2);
    }
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    if (!BMN) {
      const int r = (i * 4 + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);
      int64_t row;
      if (Tr::split) row = r < BN / 2 ? n0 + r : p.I + n0 + (r - BN / 2);
      else row = n0 + r;
      b_off[i] = (uint32_t)((row * p.ldb + c * 8) * 2);
    } else {
      constexpr int CPR = BN / 8;
      const int f = (i * 4 + wave) * 64 + lane;
      const int k = f / CPR, cc = (f % CPR) ^ ((k & 3) << 2);
      b_off[i] = (uint32_t)(((int64_t)k * p.ldb + n0 + cc * 8) * 2);
    }
  }
  const uint32_t a_kstep = AMN ? (uint32_t)(kBK * p.lda * 2) : (uint32_t)(kBK * 2);
  const uint32_t b_kstep = BMN ? (uint32_t)(kBK * p.ldb * 2) : (uint32_t)(kBK * 2);

  auto issue = [&](int kt, int slot) {
    const uint32_t sa = lds_base + slot * STAGE;
    const uint32_t sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(ra, a_off[i] + kt * a_kstep, sa + (i * 4 + wave) * 1024);
#pragma unroll
    for (int i = 0; i < LB; ++i) dma16(rb, b_off[i] + kt * b_kstep, sb + (i * 4 + wave) * 1024);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // LDS row (K-major) or column (MN-major) of the wave's sub-tile j.
  auto b_row = [&](int j) {
    if (Tr::split) return (j >> 1) * (BN / 2) + wn * (WTN / 2) + (j & 1) * 32;
    return wn * WTN + j * 32;
  };
  const int l32 = lane & 31, hi = lane >> 5;
  const int grp = lane >> 4, li = lane & 15;
  auto frag_k = [&](const unsigned char* base, int row0, int kk) -> bf16x8_t {
    const int r = row0 + l32;
    const int c = (2 * kk + hi) ^ (r & 7);
    return *reinterpret_cast<const bf16x8_t*>(base + r * 128 + c * 16);
  };
  // MN-major fragment addresses: two transposed 8-byte reads give columns col0 + (grp&1)*16 + li,
  // k = kk*16 + (grp>>1)*8 + 0..7.
  auto tr_addr = [&](int rows, int col0, int kk, int h) -> uint32_t {
    const int col = col0 + (grp & 1) * 16 + 4 * (li & 3);
    const int k = kk * 16 + (grp >> 1) * 8 + (li >> 2) + 4 * h;
    const int cc = (col >> 3) ^ ((k & 3) << 2);
    return (uint32_t)(k * rows * 2 + cc * 16 + ((col >> 2) & 1) * 8);
  };

  const int nk = (klen + kBK - 1) / kBK;
  constexpr int AHEAD = STAGES - 1;   // stages in flight ahead of the one computed
#pragma unroll
  for (int s0 = 0; s0 < AHEAD; ++s0)
    if (s0 < nk) issue(s0, s0);
  for (int kt = 0; kt < nk; ++kt) {
    // This wave's DMA for stage kt is done once only the stages issued after it remain; the
    // barrier then publishes every wave's stage kt and retires every wave's reads of stage
    // kt - 1, whose slot the next DMA reuses. A bare s_barrier: __syncthreads() would add a
    // fence that also drains the DMA still in flight.
    const int later = min(AHEAD - 1, nk - 1 - kt);   // stages issued after kt
    if (later >= 2) wait_vm<2 * (LA + LB)>();
    else if (later == 1) wait_vm<LA + LB>();
    else wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    if (kt + AHEAD < nk) issue(kt + AHEAD, (kt + AHEAD) % STAGES);
    const unsigned char* sa = smem + (kt % STAGES) * STAGE;
    const unsigned char* sb = sa + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8_t af[TM], bf[TN];
      // Transposed reads are issued from inline asm blocks that wait for them: the builtin form
      // makes the compiler drain every outstanding DMA first.
      if constexpr (AMN) {
        static_assert(TM % 4 == 0, "transposed A in groups of four sub-tiles");
#pragma unroll
        for (int i0 = 0; i0 < TM; i0 += 4) {
          uint32_t ad[8];
          v2u32_t v[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t base = lds_base + (uint32_t)(sa - smem);
            ad[2 * i] = base + tr_addr(BM, wm * WTM + (i0 + i) * 32, kk, 0);
            ad[2 * i + 1] = base + tr_addr(BM, wm * WTM + (i0 + i) * 32, kk, 1);
          }
          tr_read<8>(v, ad);
#pragma unroll
          for (int i = 0; i < 4; ++i) __builtin_memcpy(&af[i0 + i], &v[2 * i], 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = frag_k(sa, wm * WTM + i * 32, kk);
      }
      if constexpr (BMN) {
        uint32_t ad[8];
        v2u32_t v[8];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const uint32_t base = lds_base + (uint32_t)(sb - smem);
          ad[2 * j] = base + tr_addr(BN, b_row(j), kk, 0);
          ad[2 * j + 1] = base + tr_addr(BN, b_row(j), kk, 1);
        }
        tr_read<8>(v, ad);
#pragma unroll
        for (int j = 0; j < TN; ++j) __builtin_memcpy(&bf[j], &v[2 * j], 16);
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = frag_k(sb, b_row(j), kk);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Mf::run(bf[j], af[i], acc[i][j]);
    }
  }

  // ---- epilogue (lane -> row, registers -> 4 consecutive columns per group) --------------------
  const int m_in = Mf::out_m(lane);
  if constexpr (Tr::split) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 32 + m_in;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = n0 + wn * (WTN / 2) + jj * 32 + Mf::out_n(lane, q);
          if (c >= p.I) continue;
          float av[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = silu_f(acc[i][jj][4 * q + e]) * acc[i][jj + 2][4 * q + e];
          *reinterpret_cast<uint2*>(p.out + m * p.ldo + c) =
              make_uint2(pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3]));
          if (p.out2) {
            uint16_t* hrow = p.out2 + m * (2 * (int64_t)p.I);
            *reinterpret_cast<uint2*>(hrow + c) =
                make_uint2(pack_bf2(acc[i][jj][4 * q], acc[i][jj][4 * q + 1]),
                           pack_bf2(acc[i][jj][4 * q + 2], acc[i][jj][4 * q + 3]));
            *reinterpret_cast<uint2*>(hrow + p.I + c) =
                make_uint2(pack_bf2(acc[i][jj + 2][4 * q], acc[i][jj + 2][4 * q + 1]),
                           pack_bf2(acc[i][jj + 2][4 * q + 2], acc[i][jj + 2][4 * q + 3]));
          }
        }
    }
  } else {
    uint16_t* out = p.out + (Tr::grouped_rows ? 0 : (int64_t)g * p.o_gstride);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 32 + m_in;
      if (!Tr::grouped_rows && m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = n0 + wn * WTN + j * 32 + Mf::out_n(lane, q);
          if (c >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          if constexpr (KIND == kDgradDown) {
            const int64_t hrow = m * (2 * (int64_t)p.I);
            const uint2 gw = *reinterpret_cast<const uint2*>(p.aux + hrow + c);
            const uint2 uw = *reinterpret_cast<const uint2*>(p.aux + hrow + p.I + c);
            const float gg[4] = {lo_bf(gw.x), hi_bf(gw.x), lo_bf(gw.y), hi_bf(gw.y)};
            const float uu[4] = {lo_bf(uw.x), hi_bf(uw.x), lo_bf(uw.y), hi_bf(uw.y)};
            float dg[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sg = 1.0f / (1.0f + expf(-gg[e]));
              dg[e] = v[e] * uu[e] * sg * (1.0f + gg[e] * (1.0f - sg));
              du[e] = v[e] * gg[e] * sg;
            }
            *reinterpret_cast<uint2*>(p.out + hrow + c) =
                make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(p.out + hrow + p.I + c) =
                make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          } else {
            *reinterpret_cast<uint2*>(out + m * p.ldo + c) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
          }
        }
    }
  }
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// Row-grouped kinds with block_m a multiple of 128: tiles of up to kTallRows rows per group.
template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void ggemm_tall_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsBytes];
  int* pref = reinterpret_cast<int*>(smem);   // tiles before group g (reused by the DMA ring)
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = p.G;
  if (tid < 64) {
    int run = 0;
    for (int base = 0; base < G; base += 64) {
      const int g = base + lane;
      const int len = g < G ? p.seg[g + 1] - p.seg[g] : 0;
      int x = (len + kTallRows - 1) / kTallRows;
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
  const int64_t L = xcd_remap(blockIdx.x, n_tiles * p.n_tiles_n);
  if (L < 0) return;
  const int ti = (int)(L / p.n_tiles_n), nt = (int)(L % p.n_tiles_n);
  int lo = 0, hi = G - 1;   // group of tile ti: largest g with pref[g] <= ti
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pref[mid] <= ti) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int m0 = p.seg[g] + (ti - pref[g]) * kTallRows;
  const int rows = min(kTallRows, p.seg[g + 1] - m0);
  const int n0 = nt * (KindTraits<KIND>::split ? DmaCfg<128>::BN / 2 : DmaCfg<128>::BN);
  __syncthreads();   // pref is dead from here on: the DMA ring may overwrite it
  const uint32_t lb = lds_addr_of(smem);
  if (rows == 256) dma_tile<KIND, 256>(p, smem, lb, g, m0, n0, 0, p.K);
  else dma_tile<KIND, 128>(p, smem, lb, g, m0, n0, 0, p.K);
}

// Row-grouped kinds with 64-row tiles (block_m == 64): one block per tile, from tile_group.
template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void ggemm_block64_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DmaCfg<64>::STAGES * DmaCfg<64>::STAGE];
  const int total = p.total_rows[0];
  const int64_t L = xcd_remap(blockIdx.x, (int64_t)(total / 64) * p.n_tiles_n);
  if (L < 0) return;
  const int mt = (int)(L / p.n_tiles_n), nt = (int)(L % p.n_tiles_n);
  const int m0 = mt * 64;
  const int g = p.tile_group[m0 / p.block_m];
  const int n0 = nt * (KindTraits<KIND>::split ? DmaCfg<64>::BN / 2 : DmaCfg<64>::BN);
  dma_tile<KIND, 64>(p, smem, lds_addr_of(smem), g, m0, n0, 0, p.K);
}

// Weight-gradient kinds: 256 weight rows x 256 columns per tile, contraction over the segment.
template <int KIND>
__global__ __launch_bounds__(kThreads, 1) void ggemm_wgrad_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[DmaCfg<256>::STAGES * DmaCfg<256>::STAGE];
  const int64_t per_g = (int64_t)p.n_tiles_m * p.n_tiles_n;
  const int64_t L = xcd_remap(blockIdx.x, per_g * p.G);
  if (L < 0) return;
  const int g = (int)(L / per_g);
  const int rem = (int)(L % per_g);
  const int m0 = (rem / p.n_tiles_n) * 256, n0 = (rem % p.n_tiles_n) * 256;
  const int kbeg = p.seg[g], klen = p.seg[g + 1] - kbeg;
  dma_tile<KIND, 256>(p, smem, lds_addr_of(smem), g, m0, n0, kbeg, klen);
}

template <int KIND, int BM, int BN, int MS, int WAVES_M>
hipError_t launch_kind(const GemmArgs& a, int64_t grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((ggemm_kernel<KIND, BM, BN, MS, WAVES_M>), dim3((unsigned)grid),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

// Row-grouped kinds: pick the tile height from block_m (it must divide block_m).
template <int KIND>
hipError_t launch_rows(GemmArgs a, int64_t mcap, int n_per_tile, hipStream_t st) {
  const int bm = a.block_m >= 128 ? 128 : a.block_m;
  a.n_tiles_n = (int)((a.N + n_per_tile - 1) / n_per_tile);
  const int64_t tiles = (mcap / bm) * a.n_tiles_n;
  const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (a.block_m % 128 == 0) {
    if (a.seg == nullptr || a.total_rows == nullptr) return hipErrorInvalidValue;
    // Tall tiles: at most mcap/256 + G tiles (each group adds at most one short tile).
    const int64_t tall = (mcap / kTallRows + a.G) * a.n_tiles_n;
    const int64_t g2 = (tall + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL((ggemm_tall_kernel<KIND>), dim3((unsigned)g2), dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  if (a.tile_group == nullptr || a.total_rows == nullptr) return hipErrorInvalidValue;
  if (a.block_m == 64) {
    hipLaunchKernelGGL((ggemm_block64_kernel<KIND>), dim3((unsigned)grid), dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  switch (bm) {
    case 32: return launch_kind<KIND, 32, 256, 32, 1>(a, grid, st);
    case 16: return launch_kind<KIND, 16, 256, 16, 1>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_ggemm_fwd(const moe_shape_t& s, uint32_t which, int64_t mcap,
                            const uint16_t* x_perm, const int32_t* seg_offsets,
                            const int32_t* tile_group, const int32_t* total_rows,
                            const uint16_t* w1, const uint16_t* w2, uint16_t* h_save, uint16_t* a,
                            uint16_t* y_perm, hipStream_t st) {
  GemmArgs g{};
  g.block_m = s.block_m;
  g.I = s.I;
  g.G = s.E + s.S;
  g.seg = seg_offsets;
  g.tile_group = tile_group;
  g.total_rows = total_rows;
  // gate/up + SwiGLU: N counts gate columns (I); each tile covers BN/2 gate + BN/2 up columns.
  g.a = x_perm; g.lda = s.H;
  g.b = w1; g.ldb = s.H; g.b_gstride = (int64_t)2 * s.I * s.H;
  g.out = a; g.ldo = s.I; g.out2 = h_save;
  g.N = s.I; g.K = s.H;
  if (which & MOE_FWD_GATEUP) {
    hipError_t e = launch_rows<kFwdGateUp>(g, mcap, 128, st);
    if (e != hipSuccess) return e;
  }
  if (!(which & MOE_FWD_DOWN)) return hipSuccess;
  // down
  g.a = a; g.lda = s.I;
  g.b = w2; g.ldb = s.I; g.b_gstride = (int64_t)s.H * s.I;
  g.out = y_perm; g.ldo = s.H; g.out2 = nullptr;
  g.N = s.H; g.K = s.I;
  return launch_rows<kFwdDown>(g, mcap, 256, st);
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
  g.seg = seg_offsets;
  g.tile_group = tile_group;
  g.total_rows = total_rows;
  // da = dy_perm . W2[g] ([H, I] read as [K=H][N=I]) with the SwiGLU backward epilogue -> dh.
  g.a = dy_perm; g.lda = s.H;
  g.b = w2; g.ldb = s.I; g.b_gstride = (int64_t)s.H * s.I;
  g.aux = h_save; g.out = dh;
  g.N = s.I; g.K = s.H;
  if (which & MOE_DGRAD_DOWN) {
    hipError_t e = launch_rows<kDgradDown>(g, mcap, 256, st);
    if (e != hipSuccess) return e;
  }
  if (!(which & MOE_DGRAD_GATEUP)) return hipSuccess;
  // dx_perm = dh . W1[g] ([2I, H] read as [K=2I][N=H]).
  g.a = dh; g.lda = 2 * (int64_t)s.I;
  g.b = w1; g.ldb = s.H; g.b_gstride = (int64_t)2 * s.I * s.H;
  g.aux = nullptr; g.out = dx_perm; g.ldo = s.H;
  g.N = s.H; g.K = 2 * s.I;
  return launch_rows<kDgradGateUp>(g, mcap, 256, st);
}

hipError_t launch_ggemm_wgrad(const moe_shape_t& s, uint32_t which, const uint16_t* x_perm,
                              const uint16_t* a,
                              const uint16_t* dy_perm, const uint16_t* dh,
                              const int32_t* seg_offsets, uint16_t* dw1, uint16_t* dw2,
                              hipStream_t st) {
  GemmArgs g{};
  g.I = s.I;
  g.G = s.E + s.S;
  g.seg = seg_offsets;
  // dW2[g] [H, I] = dy_perm_seg^T . a_seg
  g.a = dy_perm; g.lda = s.H;
  g.b = a; g.ldb = s.I;
  g.out = dw2; g.ldo = s.I; g.o_gstride = (int64_t)s.H * s.I;
  g.M = s.H; g.N = s.I;
  g.n_tiles_m = (g.M + 255) / 256;
  g.n_tiles_n = (g.N + 255) / 256;
  int64_t tiles = (int64_t)g.G * g.n_tiles_m * g.n_tiles_n;
  if (which & MOE_WGRAD_DOWN) {
    hipLaunchKernelGGL((ggemm_wgrad_kernel<kWgradDown>),
                       dim3((unsigned)((tiles + kNumXcd - 1) / kNumXcd * kNumXcd)), dim3(kThreads),
                       0, st, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(which & MOE_WGRAD_GATEUP)) return hipSuccess;
  // dW1[g] [2I, H] = dh_seg^T . x_perm_seg
  g.a = dh; g.lda = 2 * (int64_t)s.I;
  g.b = x_perm; g.ldb = s.H;
  g.out = dw1; g.ldo = s.H; g.o_gstride = (int64_t)2 * s.I * s.H;
  g.M = 2 * s.I; g.N = s.H;
  g.n_tiles_m = (g.M + 255) / 256;
  g.n_tiles_n = (g.N + 255) / 256;
  tiles = (int64_t)g.G * g.n_tiles_m * g.n_tiles_n;
  hipLaunchKernelGGL((ggemm_wgrad_kernel<kWgradGateUp>),
                     dim3((unsigned)((tiles + kNumXcd - 1) / kNumXcd * kNumXcd)), dim3(kThreads), 0,
                     st, g);
  return hipGetLastError();
}

}  // namespace moe
