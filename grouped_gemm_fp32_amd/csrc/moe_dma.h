// Buffer->LDS DMA and wait helpers shared by the gfx950 kernels that stage operands in LDS (the
// grouped GEMM engines and the router's logits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

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

// A lane offset past the end of every buffer resource the gathering kernels build (their sources
// hold at most 2^31 bytes, which the host checks): the DMA then deposits zeros.
constexpr uint32_t kPastEnd = 0x80000000u;

// Bounds-checked DMA of 16 bytes per lane from a buffer resource into LDS at lds_wave + 16 * lane.
// Issued from asm: the instruction has no register result (it writes LDS through M0), and hiding
// it from the compiler keeps it from draining every DMA before unrelated LDS reads; the kernel's
// own vmcnt waits and barriers order the data.
// M0 is a reserved register, so the compiler would not honour it in a clobber list: the block
// saves and restores it. On GFX9-family hardware an LDS DMA that reads M0 right after a scalar
// write of M0 needs one wait state in between, hence the s_nop.
__device__ __forceinline__ void dma16(v4u32_t r, uint32_t voff, uint32_t lds_wave) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(uniform(lds_wave)), "v"(voff), "s"(r) : "memory");
}
// The same with the non-temporal hint, for operands read exactly once (the expert weights): L2
// then keeps the activation panels that the tiles of a segment share.
__device__ __forceinline__ void dma16_nt(v4u32_t r, uint32_t voff, uint32_t lds_wave) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
               "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "s"(uniform(lds_wave)), "v"(voff), "s"(r) : "memory");
}

// Waits, each also a compiler memory barrier so that no LDS access moves across them.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Wait until at most `later` of this wave's DMA stages (PER instructions each) are in flight.
template <int PER, int MAXL>
__device__ __forceinline__ void wait_stages(int later) {
  if constexpr (MAXL >= 3) {
    if (later >= 3) { wait_vm<3 * PER>(); return; }
  }
  if constexpr (MAXL >= 2) {
    if (later == 2) { wait_vm<2 * PER>(); return; }
  }
  if constexpr (MAXL >= 1) {
    if (later == 1) { wait_vm<PER>(); return; }
  }
  wait_vm<0>();
}

}  // namespace moe
