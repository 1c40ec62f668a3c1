// Device helpers shared by the bf16 GEMM and the block-scaled GEMM: LDS DMA
// staging (buffer descriptors, the DMA instruction, explicit vector-memory
// waits), the conflict-free swizzle of 64-byte LDS rows, and the XCD-aware
// tile order.
#pragma once

#include "stg_internal.h"

namespace stg {
namespace {

// s_waitcnt immediate: vmcnt <= n, other counters unconstrained (gfx9 layout).
#define STG_VMCNT(n) (((n)&0xF) | (((n) >> 4) << 14) | 0x0F70)

// Physical 16-byte chunk of logical chunk c in A row r (4 chunks per row):
// the 16 rows one ds_read_b128 phase touches cover all 16 bank groups of the
// 256-byte LDS bank sweep (and any 8 consecutive rows cover a 128-byte one).
__device__ __forceinline__ int a_phys(int r, int c) { return c ^ (((r >> 2) ^ (r >> 1)) & 3); }
// XOR applied to the chunk index of B row k: the 4 rows x 64 bytes that one
// ds_read_b64_tr_b16 phase of 32 lanes touches land in distinct bank groups.
template <int CPR>
__device__ __forceinline__ int b_swz(int k) {
  return CPR >= 16 ? 4 * (k & 3) : CPR >= 8 ? 2 * (k & 3) : 2 * ((k >> 1) & 1);
}

// Wait until at most n (0..63) vector-memory operations of this wave are
// outstanding; n is only known at run time here, the instruction needs it as
// an immediate.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define STG_W(i) case i: __builtin_amdgcn_s_waitcnt(STG_VMCNT(i)); break;
#define STG_W8(b) STG_W(b) STG_W(b + 1) STG_W(b + 2) STG_W(b + 3) STG_W(b + 4) STG_W(b + 5) STG_W(b + 6) STG_W(b + 7)
    STG_W8(0) STG_W8(8) STG_W8(16) STG_W8(24) STG_W8(32) STG_W8(40) STG_W8(48) STG_W8(56)
#undef STG_W8
#undef STG_W
    default: __builtin_amdgcn_s_waitcnt(STG_VMCNT(0));
  }
}


// Tile (tm, tn) of logical id t: consecutive ids on one XCD, grouped by 4
// row panels so neighbouring workgroups share A and B panels in L2.
__device__ __forceinline__ void tile_of(uint32_t t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int group = t / per_group;
  const int first = group * G;
  const int gm = min(G, tiles_m - first);
  const int in = t - group * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

typedef uint32_t u32x4_s __attribute__((ext_vector_type(4)));

// Raw-buffer descriptor words (gfx9 layout, stride 0) over [base, base+bytes),
// made wave-uniform so they live in SGPRs.
__device__ __forceinline__ u32x4_s rsrc_words(const char* base, int64_t avail) {
  const uint32_t bytes = (uint32_t)(avail <= 0 ? 0 : avail < (int64_t)kOOB ? avail : (int64_t)kOOB - 1);
  const uint64_t a = (uint64_t)base;
  u32x4_s w;
  w[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  w[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
  w[2] = __builtin_amdgcn_readfirstlane(bytes);
  w[3] = 0x00020000u;
  return w;
}

// LDS DMA of 16 bytes per lane: lane L's chunk at buffer offset `off` lands at
// LDS byte lds_base + 16 L; an offset past num_records writes zeros.  Issued
// through inline asm so the compiler does not guard every later LDS read with
// a wait on all outstanding loads; completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes the stage.
__device__ __forceinline__ void dma16(const u32x4_s& rs, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(off), "s"(rs)
               : "memory", "m0");
}

// The same at buffer offset off + soff, soff and lds_addr wave-uniform: soff
// is the instruction's scalar offset, so a descriptor can stay fixed while
// soff walks along K.  The operand takes an SGPR only, never a literal: a
// caller whose soff may fold to a constant passes it through
// uniform_sgpr() first.
__device__ __forceinline__ void dma16s(const u32x4_s& rs, uint32_t off, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(off), "s"(rs), "s"(soff)
               : "memory", "m0");
}

// v made wave-uniform and held in an SGPR as far as the compiler knows
__device__ __forceinline__ uint32_t uniform_sgpr(uint32_t v) {
  v = __builtin_amdgcn_readfirstlane(v);
  asm volatile("" : "+s"(v));
  return v;
}

}  // namespace
}  // namespace stg
