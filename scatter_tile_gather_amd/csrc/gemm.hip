// Bounded-edge GEMM  C = A . B  (bf16 operands, fp32 accumulation).
//
// Semantics (cuTile.jl Operations, muladd: bf16 x bf16 accumulates in f32;
// Tylo.jl Boundary tiles, "Accumulator stores and GEMM": ceiling-division
// output grid and K loop, boundary stages zero-filled, an epilogue that
// converts the f32 accumulator to the destination type and suppresses invalid
// coordinates, leaving padding untouched).
//
// gfx950 design (the template kernel below; the two main kernels further down
// keep its staging and differ in waves and MFMA shape):
//  * Workgroup tile BM x BN x 32, waves WM x WN, each wave owning a
//    (BM/WM) x (BN/WN) block of v_mfma_f32_32x32x16_bf16 accumulators.  Every
//    lane issues every MFMA; bounds only select the data that was staged.
//  * Staging (Tylo.jl Boundary tiles, opening section and "A concrete edge",
//    recast for gfx950): the A and B stages are filled by LDS DMA
//    (buffer_load_dwordx4 ... lds), which writes each lane's 16 bytes straight
//    into LDS without passing through registers.  A lane whose 16-byte chunk
//    (eight bf16 values, at any 2-byte alignment) lies fully inside the
//    logical extent gets its offset; a chunk with no valid value gets an offset
//    past the buffer's num_records and lands as zeros.  Only a stage that holds
//    a chunk straddling the K or N edge is patched afterwards, element by
//    element, by the lane that owns the chunk.  No address is formed for an
//    invalid coordinate.
//  * LDS layout: a DMA instruction writes 64 lanes x 16 bytes linearly, so the
//    swizzle is realised by choosing which chunk each lane fetches.  A rows are
//    64 bytes (K contiguous, the MFMA A operand is eight consecutive K of one
//    row) with chunk c stored at c ^ (((row >> 2) ^ (row >> 1)) & 3); B rows are N
//    contiguous with chunk pairs XOR-ed by the row, and the MFMA B operand
//    (eight consecutive K of one column) is read with ds_read_b64_tr_b16, the
//    gfx950 LDS transpose read.  Both swizzles are functions of the
//    tile-local (window) coordinate and zero-filled chunks take the same
//    mapping, so an edge never disturbs the swizzle phase (Tylo.jl Boundary
//    tiles, "A concrete edge", swizzled windows).  Operand reads are
//    bank-conflict free.
//  * Pipeline: a ring of NSTAGE stages; the DMA for stage k+NSTAGE-1 is
//    issued while stage k feeds the MFMAs, one instruction after every few
//    MFMAs (a wave issues in order, and a burst of DMA that fills the memory
//    queue would stall the MFMAs behind it); the first operands of stage k+1
//    are read before the barrier that ends step k, and each step waits only
//    for stage k+2.  One barrier per 32 K values.
//  * Grid: a main launch of 256 x 256 tiles over the columns that fill whole
//    tiles -- the 4-wave kernel for 16-byte aligned rows, otherwise the
//    8-wave kernel on 16 x 16 x 32 MFMAs (both below) --; the remaining
//    columns go to an edge launch of 64 x 32 tiles (the template kernel
//    here), or, when at most 8 remain (N = 8193 leaves one), to a skinny
//    vector kernel.
//    Tile ids are renumbered so that consecutive ids run on one XCD and walk
//    4-row-panel groups, keeping A and B panels resident in that XCD's L2.
#include <type_traits>

#include "gemm_common.h"

namespace stg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4y __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BK = 32;  // K values per stage

struct GemmParams {
  const char* A;  // bf16 (M, K), row stride lda elements
  const char* B;  // bf16 (K, N), row stride ldb elements
  char* C;
  const float* acc;  // fp32 output only: (M, N) added to the product, row stride ldacc, or null
  int64_t lda, ldb, ldc, ldacc;
  int64_t M, N, K;
  int64_t n_base;  // first column covered by this launch
  int32_t tiles_m, tiles_n;
  int32_t c_f32;  // 1: fp32 output, 0: bf16
};

template <int BM_, int BN_, int WM_, int WN_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NSTAGE = NS_;  // LDS ring depth; stage k+NSTAGE-1 is in flight during step k
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_STAGE_B = BM * BK * 2;  // 64-byte rows
  static constexpr int B_STAGE_B = BK * BN * 2;
  static constexpr int STAGE_B = A_STAGE_B + B_STAGE_B;
  static constexpr int A_DMA_W = A_STAGE_B / 1024 / NW;  // DMA instructions per wave and stage
  static constexpr int B_DMA_W = B_STAGE_B / 1024 / NW;
  static constexpr int DMA_W = A_DMA_W + B_DMA_W;
  static constexpr int B_CPR = BN / 8;  // 16-byte chunks per B row
  static constexpr int EPI_PITCH_B = WTN * 2 + 16;  // bytes per row of a wave's bf16 output tile
  static constexpr int EPI_WAVE_B = WTM * EPI_PITCH_B;
  static constexpr int LDS_B = NSTAGE * STAGE_B > NW * EPI_WAVE_B ? NSTAGE * STAGE_B : NW * EPI_WAVE_B;
  static_assert(NSTAGE >= 3 && (NSTAGE - 3) * DMA_W <= 63, "ring depth vs vmcnt range");
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 MFMA blocks");
  static_assert(A_DMA_W * NW * 1024 == A_STAGE_B && B_DMA_W * NW * 1024 == B_STAGE_B,
                "stages must split into whole 1 KiB DMA instructions per wave");
  static_assert(BN == 32 || BN % 64 == 0, "B swizzle assumes 64-byte rows or multiples of 128 bytes");
};

template <class CF>
__global__ __launch_bounds__(CF::NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CF::WN, wn = wave % CF::WN;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * CF::BM;
  const int64_t n0 = p.n_base + (int64_t)tn * CF::BN;
  const int nk = (int)((p.K + BK - 1) / BK);

  f32x16 acc[CF::FM][CF::FN];
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int j = 0; j < CF::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8 fa[2][CF::FM], fb[2][CF::FN];

  // chunk owned by this lane in DMA instruction q of the A / B stage
  auto a_chunk = [&](int q, int& r, int& c) {
    const int pos = (wave * CF::A_DMA_W + q) * 64 + lane;
    r = pos >> 2;
    c = a_phys(r, pos & 3);
  };
  auto b_chunk = [&](int q, int& k, int& c) {
    const int pos = (wave * CF::B_DMA_W + q) * 64 + lane;
    k = pos / CF::B_CPR;
    c = (pos % CF::B_CPR) ^ b_swz<CF::B_CPR>(k);
  };

  // Per-lane DMA offsets are the same for every stage (the descriptors move
  // with k0): rows of A past M and columns of B past N are folded in once
  // here; only a stage reaching past K needs a per-chunk test.
  uint32_t a_off[CF::A_DMA_W], b_off[CF::B_DMA_W];
  int a_kc[CF::A_DMA_W], b_k[CF::B_DMA_W];
#pragma unroll
  for (int q = 0; q < CF::A_DMA_W; ++q) {
    int r, c;
    a_chunk(q, r, c);
    a_kc[q] = 8 * c;
    a_off[q] = m0 + r < p.M ? (uint32_t)(r * p.lda * 2 + c * 16) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < CF::B_DMA_W; ++q) {
    int k, c;
    b_chunk(q, k, c);
    b_k[q] = k;
    b_off[q] = n0 + 8 * c + 8 <= p.N ? (uint32_t)(k * p.ldb * 2 + c * 16) : kOOB;
  }

  // 32-bit LDS address of the dynamic shared memory (wave-uniform)
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  // issue the LDS DMA of stage kt into ring slot kt % NSTAGE
  auto issue_stage = [&](int kt) {
    const uint32_t st = smem_lds + (kt % CF::NSTAGE) * CF::STAGE_B;
    const int64_t k0 = (int64_t)kt * BK;
    const u32x4_s rsa = rsrc_words(p.A + (m0 * p.lda + k0) * 2, ((p.M - 1 - m0) * p.lda + (p.K - k0)) * 2);
    const u32x4_s rsb = rsrc_words(p.B + (k0 * p.ldb + n0) * 2, ((p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2);
    if (k0 + BK <= p.K) {
#pragma unroll
      for (int q = 0; q < CF::A_DMA_W; ++q) dma16(rsa, a_off[q], st + (wave * CF::A_DMA_W + q) * 1024);
#pragma unroll
      for (int q = 0; q < CF::B_DMA_W; ++q) dma16(rsb, b_off[q], st + CF::A_STAGE_B + (wave * CF::B_DMA_W + q) * 1024);
    } else {
      const int kleft = (int)(p.K - k0);  // valid K values in this stage, 1..BK-1
#pragma unroll
      for (int q = 0; q < CF::A_DMA_W; ++q)
        dma16(rsa, a_kc[q] + 8 <= kleft ? a_off[q] : kOOB, st + (wave * CF::A_DMA_W + q) * 1024);
#pragma unroll
      for (int q = 0; q < CF::B_DMA_W; ++q)
        dma16(rsb, b_k[q] < kleft ? b_off[q] : kOOB, st + CF::A_STAGE_B + (wave * CF::B_DMA_W + q) * 1024);
    }
  };

  // after this lane's DMA of stage kt completed: write the chunks that
  // straddle the K edge (A) or the N edge (B), which the DMA left zero
  auto fix_stage = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    const bool a_edge = k0 + BK > p.K && (p.K & 7);
    const bool b_edge = n0 + CF::BN > p.N && (p.N & 7);
    if (!a_edge && !b_edge) return;
    char* st = smem + (kt % CF::NSTAGE) * CF::STAGE_B;
    if (a_edge) {
#pragma unroll
      for (int q = 0; q < CF::A_DMA_W; ++q) {
        int r, c;
        a_chunk(q, r, c);
        const int64_t col = k0 + 8 * c, left = p.K - col;
        if (m0 + r < p.M && left > 0 && left < 8) {
          const uint16_t* src = (const uint16_t*)(p.A + ((m0 + r) * p.lda + col) * 2);
          u32x4 v = {0, 0, 0, 0};
          for (int e = 0; e < 8; ++e)
            if (e < left) vec_set<2>(v, e, src[e]);
          *(u32x4*)(st + (wave * CF::A_DMA_W + q) * 1024 + lane * 16) = v;
        }
      }
    }
    if (b_edge) {
#pragma unroll
      for (int q = 0; q < CF::B_DMA_W; ++q) {
        int k, c;
        b_chunk(q, k, c);
        const int64_t col = n0 + 8 * c, left = p.N - col;
        if (k0 + k < p.K && left > 0 && left < 8) {
          const uint16_t* src = (const uint16_t*)(p.B + ((k0 + k) * p.ldb + col) * 2);
          u32x4 v = {0, 0, 0, 0};
          for (int e = 0; e < 8; ++e)
            if (e < left) vec_set<2>(v, e, src[e]);
          *(u32x4*)(st + CF::A_STAGE_B + (wave * CF::B_DMA_W + q) * 1024 + lane * 16) = v;
        }
      }
    }
  };

  // MFMA operands of K sub-step ks (16 K values) of stage kt into slot s
  auto read_frags = [&](int kt, int ks, int s) {
    const char* as = smem + (kt % CF::NSTAGE) * CF::STAGE_B;
    const char* bs = as + CF::A_STAGE_B;
#pragma unroll
    for (int i = 0; i < CF::FM; ++i) {
      const int r = wm * CF::WTM + i * 32 + (lane & 31);
      fa[s][i] = *(const bf16x8*)(as + r * (BK * 2) + (a_phys(r, 2 * ks + (lane >> 5)) << 4));
    }
#pragma unroll
    for (int j = 0; j < CF::FN; ++j) {
      // transpose read: lane t of 16-lane group g points at row
      // 16ks + 8(g/2) + 4h + t/4, columns nb + 16(g%2) + 4(t%4) .. +3
      const int g = lane >> 4, t = lane & 15;
      const int col = wn * CF::WTN + j * 32 + 16 * (g & 1) + 4 * (t & 3);
      const int row = 16 * ks + 8 * (g >> 1) + (t >> 2);
      const int off = ((col >> 3) ^ b_swz<CF::B_CPR>(row)) * 16 + (col & 7) * 2;  // rows 4 apart share the XOR
      const char* p0 = bs + row * (CF::BN * 2) + off;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * CF::BN * 2));
      const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      fb[s][j] = __builtin_bit_cast(bf16x8, both);
    }
  };
  auto mfmas = [&](int s) {
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  };

  // DMA instruction q (the A instructions first, then B) of stage kt; a
  // stage reaching past K sends its chunks with no valid value out of range
  auto stage_rsrc = [&](int kt, u32x4_s& rsa, u32x4_s& rsb) {
    const int64_t k0 = (int64_t)kt * BK;
    rsa = rsrc_words(p.A + (m0 * p.lda + k0) * 2, ((p.M - 1 - m0) * p.lda + (p.K - k0)) * 2);
    rsb = rsrc_words(p.B + (k0 * p.ldb + n0) * 2, ((p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2);
  };
  auto dma_one = [&](int kt, int q, const u32x4_s& rsa, const u32x4_s& rsb) {
    const uint32_t st = smem_lds + (kt % CF::NSTAGE) * CF::STAGE_B;
    const int kleft = (int)(p.K - (int64_t)kt * BK);
    if (q < CF::A_DMA_W) {
      dma16(rsa, a_kc[q] + 8 <= kleft ? a_off[q] : kOOB, st + (wave * CF::A_DMA_W + q) * 1024);
    } else {
      const int qb = q - CF::A_DMA_W;
      dma16(rsb, b_k[qb] < kleft ? b_off[qb] : kOOB, st + CF::A_STAGE_B + (wave * CF::B_DMA_W + qb) * 1024);
    }
  };
  // MFMAs of operand slot s with DMA instructions q0 .. q0+nq-1 of stage kd
  // spread evenly among them: a wave whose memory instructions cannot issue
  // (the vector-memory queue is full) stalls in order, so a burst of DMA
  // would hold back the MFMAs queued behind it.  The scheduling barriers keep
  // the compiler from regrouping them.
  auto mfmas_dma = [&](int s, int kd, int q0, int nq, const u32x4_s& rsa, const u32x4_s& rsb) {
    constexpr int NM = CF::FM * CF::FN;
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
        const int m = i * CF::FN + j;
#pragma unroll
        for (int d = 0; d < nq; ++d) {
          // instruction d goes after MFMA max(0, (d + 1) NM / nq - 1)
          const int after = ((d + 1) * NM) / nq - 1;
          if ((after < 0 ? 0 : after) == m) {
            __builtin_amdgcn_sched_barrier(0);
            dma_one(kd, q0 + d, rsa, rsb);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
  };
  // one K step: operands of stage kt (second half) and kt + 1 (first half)
  // feed the MFMAs while stage kt + NSTAGE - 1 is issued (when `dma`)
  auto step = [&](int kt, bool dma) {
    constexpr int H = CF::DMA_W / 2;
    u32x4_s rsa, rsb;
    if (dma) stage_rsrc(kt + CF::NSTAGE - 1, rsa, rsb);
    read_frags(kt, 1, 1);
    mfmas_dma(0, kt + CF::NSTAGE - 1, 0, dma ? H : 0, rsa, rsb);
    // stage kt + 1 became visible at the previous barrier
    if (kt + 1 < nk) read_frags(kt + 1, 0, 0);
    mfmas_dma(1, kt + CF::NSTAGE - 1, H, dma ? CF::DMA_W - H : 0, rsa, rsb);
    if (kt + 2 < nk) {
      // stage kt + 2 must have landed; the stages issued after it may fly on
      wait_vmcnt((min(nk - 1, kt + CF::NSTAGE - 1) - (kt + 2)) * CF::DMA_W);
      fix_stage(kt + 2);
    }
    // ring slot (kt + NSTAGE) % NSTAGE = kt % NSTAGE is free after this
    __syncthreads();
  };
  // the same for a step in the middle of a tile that is whole in N: the DMA
  // of stage kt + NSTAGE - 1 in flight and stage kt + 2 not the last, so no
  // edge to patch -- kept out of the loop, the patch code no longer takes
  // registers and issue slots from every step (1.5% faster)
  auto step_inner = [&](int kt) {
    constexpr int H = CF::DMA_W / 2;
    u32x4_s rsa, rsb;
    stage_rsrc(kt + CF::NSTAGE - 1, rsa, rsb);
    read_frags(kt, 1, 1);
    mfmas_dma(0, kt + CF::NSTAGE - 1, 0, H, rsa, rsb);
    read_frags(kt + 1, 0, 0);
    mfmas_dma(1, kt + CF::NSTAGE - 1, H, CF::DMA_W - H, rsa, rsb);
    wait_vmcnt((CF::NSTAGE - 3) * CF::DMA_W);
    __syncthreads();
  };

  // prologue: NSTAGE - 1 stages in flight, wait for the first two
  for (int s = 0; s < CF::NSTAGE - 1 && s < nk; ++s) issue_stage(s);
  wait_vmcnt(max(0, min(nk, CF::NSTAGE - 1) - 2) * CF::DMA_W);
  if (nk > 0) fix_stage(0);
  if (nk > 1) fix_stage(1);
  __syncthreads();
  if (nk > 0) read_frags(0, 0, 0);
  // ring slot (kt + NSTAGE - 1) % NSTAGE, written during step kt, was last
  // read in step kt - 1 and released by its barrier
  int kt = 0;
  if (n0 + CF::BN <= p.N)
    for (; kt + CF::NSTAGE - 1 < nk && kt + 3 < nk; ++kt) step_inner(kt);
  for (; kt + CF::NSTAGE - 1 < nk; ++kt) step(kt, true);
  for (; kt < nk; ++kt) step(kt, false);

  // clipped epilogue: lane l, accumulator r of block (i, j) is
  // row 8(r/4) + 4(l/32) + r%4, column l%32 of that 32x32 block
  if (p.c_f32) {
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) {
        const int64_t col = n0 + wn * CF::WTN + j * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * CF::WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M)
            *(float*)(p.C + (row * p.ldc + col) * 4) = p.acc ? acc[i][j][r] + p.acc[row * p.ldacc + col] : acc[i][j][r];
        }
      }
    return;
  }
  // bf16: round to nearest even, stage the wave's tile in LDS (every wave has
  // its own region; the ring is no longer read after the last barrier), then
  // write whole 16-byte row chunks; only chunks crossing column N are written
  // element by element
  char* ep = smem + wave * CF::EPI_WAVE_B;
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int j = 0; j < CF::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = j * 32 + (lane & 31);
        *(__bf16*)(ep + row * CF::EPI_PITCH_B + col * 2) = (__bf16)acc[i][j][r];
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = CF::WTN / 8;  // 16-byte chunks per wave-tile row
  for (int c = lane; c < CF::WTM * CPR; c += 64) {
    const int row = c / CPR, ch = c % CPR;
    const int64_t grow = m0 + wm * CF::WTM + row;
    const int64_t gcol = n0 + wn * CF::WTN + ch * 8;
    if (grow >= p.M || gcol >= p.N) continue;
    const u32x4 v = *(const u32x4*)(ep + row * CF::EPI_PITCH_B + ch * 16);
    char* dst = p.C + (grow * p.ldc + gcol) * 2;
    if (gcol + 8 <= p.N) {
      st16(dst, v);
    } else {
      for (int e = 0; e < 8; ++e)
        if (gcol + e < p.N) store_elem<2>(dst + e * 2, vec_get<2>(v, e));
    }
  }
}

// Skinny strip: C[:, n_base + j] for j < R <= 8 remaining columns.  The strip
// is a matrix-vector shape (all of A against a few columns of B), bound by
// reading A once, so it runs on the vector ALUs.  B's R columns of each K block
// are staged once per workgroup in LDS as fp32; a wave owns SK_RPW rows and
// covers a block's K with its 64 lanes, one 16-byte chunk of A (eight bf16)
// per lane and row at a time (element loads only for the chunk crossing K),
// issuing all of its rows' loads before the arithmetic; each lane keeps R fp32
// partial sums per row, reduced across the wave with cross-lane shuffles
// before the clipped write.
constexpr int SK_KB = 1024;                 // K values per LDS block
constexpr int SK_CPL = SK_KB / 8 / 64;      // 16-byte chunks per lane and row in a block (2)
constexpr int SK_RPW = 4;                   // rows per wave
constexpr int SK_ROWS = SK_RPW * 4;         // rows per workgroup (4 waves)

template <int R>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p) {
  __shared__ float sb[8 * SK_KB];  // [j][k] of the current K block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * SK_ROWS + wave * SK_RPW;
  float acc[SK_RPW][R];
#pragma unroll
  for (int r = 0; r < SK_RPW; ++r)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[r][j] = 0.f;
  for (int64_t k0 = 0; k0 < p.K; k0 += SK_KB) {
    const int kb = (int)(p.K - k0 < SK_KB ? p.K - k0 : SK_KB);
    __syncthreads();  // the previous block's B is no longer read
    for (int i = tid; i < R * SK_KB; i += 256) {
      const int j = i / SK_KB, k = i - j * SK_KB;
      float v = 0.f;
      if (k < kb) {
        const uint16_t h = *(const uint16_t*)(p.B + ((k0 + k) * p.ldb + p.n_base + j) * 2);
        v = __uint_as_float((uint32_t)h << 16);
      }
      sb[j * SK_KB + k] = v;
    }
    __syncthreads();
    u32x4 a[SK_RPW][SK_CPL];
#pragma unroll
    for (int r = 0; r < SK_RPW; ++r) {
      const int64_t row = row0 + r;
      const char* arow = p.A + (row * p.lda + k0) * 2;
#pragma unroll
      for (int q = 0; q < SK_CPL; ++q) {
        const int c = (lane + 64 * q) * 8;  // first K value of the chunk within the block
        a[r][q] = (u32x4){0, 0, 0, 0};
        if (row < p.M) {
          if (c + 8 <= kb) {
            a[r][q] = ld16(arow + c * 2);
          } else if (c < kb) {
            for (int e = 0; e < 8; ++e)
              if (c + e < kb) vec_set<2>(a[r][q], e, load_elem<2>(arow + (c + e) * 2));
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < SK_CPL; ++q) {
      const int c = (lane + 64 * q) * 8;
      if (c >= kb) continue;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float4 b0 = *(const float4*)(sb + j * SK_KB + c);
        const float4 b1 = *(const float4*)(sb + j * SK_KB + c + 4);
#pragma unroll
        for (int r = 0; r < SK_RPW; ++r) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = __uint_as_float((uint32_t)vec_get<2>(a[r][q], e) << 16);
          acc[r][j] += x[0] * b0.x + x[1] * b0.y + x[2] * b0.z + x[3] * b0.w + x[4] * b1.x + x[5] * b1.y +
                       x[6] * b1.z + x[7] * b1.w;
        }
      }
    }
  }
  // reduce over the wave's 64 lanes; lane j (< R) writes column j of each row
#pragma unroll
  for (int r = 0; r < SK_RPW; ++r) {
    const int64_t row = row0 + r;
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      float v = acc[r][j];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == j) mine = v;
    }
    if (row < p.M && lane < R) {
      const int64_t col = p.n_base + lane;
      if (p.c_f32)
        *(float*)(p.C + (row * p.ldc + col) * 4) = p.acc ? mine + p.acc[row * p.ldacc + col] : mine;
      else
        *(__bf16*)(p.C + (row * p.ldc + col) * 2) = (__bf16)mine;
    }
  }
}

// Main kernel for 16-byte aligned operand rows: 4 waves, one per SIMD, each
// owning a 128 x 128 block of the 256 x 256 tile as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators per lane, held in the
// accumulation registers).  Against 8 waves of 128 x 64 it reads a third
// fewer operand bytes from LDS per MFMA, and the 16 x 16 x 32 instruction
// costs less power per flop than 32 x 32 x 16 (alone on random register
// operands: 2.17 against 1.90 PFLOP/s).  At 8192 x 8192 x 4096: 1.36-1.37
// PFLOP/s, against 1.30-1.32 for the same kernel on 32 x 32 x 16, 1.27-1.30
// for the 8-wave kernel below and 1.34 for hipBLASLt.  With one wave per SIMD
// a DMA instruction that cannot issue holds back the MFMAs behind it, so when
// the operand feed itself is the bound -- rows not 16-byte aligned, where
// every 16-byte chunk straddles two -- 8 waves, whose SIMD partner keeps
// issuing, are faster (odd strides: 1.03-1.04 here against 1.10-1.15), and
// the host picks this kernel only for aligned rows.
//  * Same stages, swizzles, zero-fill and ring as the 8-wave kernel (4 slots of
//    32 K values; stage k+3 in flight during step k, spread 8 DMA instructions
//    per wave among the step's 64 MFMAs); one descriptor per operand panel
//    for the whole K loop, the stage selected by the instruction's scalar
//    offset, so a DMA costs no vector arithmetic.
//  * Operands: the next stage's B blocks are read into a second register set
//    during the current stage (16 transposed reads, one after every 4 MFMAs);
//    A blocks just in time, two 16-row blocks ahead through four rolling
//    registers.  The loop is unrolled over the 4 ring slots (and the last
//    steps over the 2 register sets), so every LDS address is a per-lane
//    base plus an immediate and every register-array index a constant.
//  * The MFMAs are written out as inline assembly with the accumulator in
//    accumulation registers: through the builtin, the compiler kept some of
//    the 64 blocks in VGPRs and copied them after every MFMA behind a 6-cycle
//    wait.  Nothing else reads an accumulator inside the loop, each block is
//    rewritten only 64 MFMAs later, and the operand reads feeding an MFMA
//    are awaited by the compiler (it sees the asm's inputs); after the loop
//    an explicit wait covers the results' latency.
//  * Epilogue through LDS in 32-row passes, also for fp32 output, so rows
//    leave as 16-byte chunks.
constexpr int W4_NS = 4;                           // ring stages
constexpr int W4_ASTAGE = 256 * BK * 2;            // 256 rows of 64 bytes
constexpr int W4_BSTAGE = BK * 256 * 2;            // 32 rows of 512 bytes
constexpr int W4_STAGE = W4_ASTAGE + W4_BSTAGE;
constexpr int W4_DMA = 8;                          // DMA instructions per wave and stage (4 A, then 4 B)
constexpr int W4_EPI_PITCH = 128 * 2 + 16;         // bf16 staging: bytes per row of a wave's block
constexpr int W4_EPI_WAVE = 128 * W4_EPI_PITCH;
constexpr int W4_F32_PITCH = 128 * 4 + 32;         // fp32 staging: rows 4 apart land 32 banks apart
constexpr int W4_F32_WAVE = 32 * W4_F32_PITCH;
constexpr int W4_LDS = W4_NS * W4_STAGE > 4 * W4_EPI_WAVE ? W4_NS * W4_STAGE : 4 * W4_EPI_WAVE;
static_assert(4 * W4_F32_WAVE <= W4_LDS, "fp32 staging fits");

template <int V>
using Slot = std::integral_constant<int, V>;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * 256;
  const int64_t n0 = p.n_base + (int64_t)tn * 256;
  const int nk = (int)((p.K + BK - 1) / BK);
  const int nkf = (int)(p.K / BK);  // stages wholly inside K

  // whole panels: A rows m0 .., B columns n0 .. (the host bounds both below 2^31 bytes)
  const u32x4_s rsa = rsrc_words(p.A + m0 * p.lda * 2, ((p.M - 1 - m0) * p.lda + p.K) * 2);
  const u32x4_s rsb = rsrc_words(p.B + n0 * 2, ((p.K - 1) * p.ldb + (p.N - n0)) * 2);
  const uint32_t bstep = (uint32_t)(BK * p.ldb * 2);

  // chunk of DMA instruction q: A row r, logical chunk c (swizzled slot pos & 3);
  // B row k, logical chunk cb (slot pos & 31)
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int pos = (wave * 4 + q) * 64 + lane;
    const int r = pos >> 2, c = a_phys(r, pos & 3);
    a_off[q] = m0 + r < p.M ? (uint32_t)(r * p.lda * 2 + c * 16) : kOOB;
    const int k = pos >> 5, cb = (pos & 31) ^ b_swz<32>(k);
    b_off[q] = n0 + 8 * cb + 8 <= p.N ? (uint32_t)(k * p.ldb * 2 + cb * 16) : kOOB;
  }
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  // DMA instruction q of stage kt into ring slot `slot`; a stage reaching past K
  // (part) sends its chunks with no valid value out of range
  auto dma = [&](int kt, int slot, int q, bool part) {
    const uint32_t st = smem_lds + slot * W4_STAGE;
    const int kleft = part ? (int)(p.K - (int64_t)kt * BK) : BK;
    const int pos = (wave * 4 + (q & 3)) * 64 + lane;
    if (q < 4) {
      const uint32_t off = part && 8 * a_phys(pos >> 2, pos & 3) + 8 > kleft ? kOOB : a_off[q];
      dma16s(rsa, off, (uint32_t)kt * (BK * 2), st + (wave * 4 + q) * 1024);
    } else {
      const uint32_t off = part && (pos >> 5) >= kleft ? kOOB : b_off[q - 4];
      dma16s(rsb, off, (uint32_t)kt * bstep, st + W4_ASTAGE + (wave * 4 + q - 4) * 1024);
    }
  };
  // after this lane's DMA of stage kt landed: A chunks straddling K, which the
  // DMA left zero, written element by element (the main launch has no N edge)
  auto fix_stage = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    if (!(k0 + BK > p.K && (p.K & 7))) return;
    char* st = smem + (kt % W4_NS) * W4_STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = (wave * 4 + q) * 64 + lane;
      const int r = pos >> 2, c = a_phys(r, pos & 3);
      const int64_t col = k0 + 8 * c, left = p.K - col;
      if (m0 + r < p.M && left > 0 && left < 8) {
        const uint16_t* src = (const uint16_t*)(p.A + ((m0 + r) * p.lda + col) * 2);
        u32x4 v = {0, 0, 0, 0};
        for (int e = 0; e < 8; ++e)
          if (e < left) vec_set<2>(v, e, src[e]);
        *(u32x4*)(st + (wave * 4 + q) * 1024 + lane * 16) = v;
      }
    }
  };

  f32x4y acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  bf16x8 fa[4], fb[2][8];

  // per-lane LDS offsets within a stage.  A block i: row ar + 16 i, chunk
  // lane / 16 (rows 16 apart share the swizzle: i adds 1024).  B block j
  // (transposed reads): lane t of 16-lane group g reads row 8 g + 4 h + t / 4
  // at columns wn 128 + 16 j + 4 (t % 4) .. + 3 and receives column 16 j + t,
  // K values 8 g + 4 h .. + 3 (h adds 2048)
  const int ar = wm * 128 + (lane & 15);
  const uint32_t a_lds = ar * 64 + (a_phys(ar, lane >> 4) << 4);
  uint32_t b_lds[8];
  {
    const int g = lane >> 4, t = lane & 15;
    const int row = 8 * g + (t >> 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = wn * 128 + j * 16 + 4 * (t & 3);
      b_lds[j] = W4_ASTAGE + row * 512 + ((col >> 3) ^ b_swz<32>(row)) * 16 + (col & 7) * 2;
    }
  }
  auto rd_a = [&](const char* base, int i) __attribute__((always_inline)) {
    fa[i & 3] = *(const bf16x8*)(base + a_lds + i * 1024);
  };
  auto rd_b = [&](const char* base, int s, int e) __attribute__((always_inline)) {
    const int j = e >> 1, h = e & 1;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + b_lds[j] + h * 2048));
    s16x8 cur = __builtin_bit_cast(s16x8, fb[s][j]);
#pragma unroll
    for (int x = 0; x < 4; ++x) cur[4 * h + x] = v[x];
    fb[s][j] = __builtin_bit_cast(bf16x8, cur);
  };
  // the 64 MFMAs of stage kt (A rolling, B in set s), row by row: A block
  // i + 2 read at the start of row i (the next stage's blocks 0, 1 at rows 6,
  // 7); B read e of the next stage into the other set after MFMA 4 e + 2; DMA
  // instruction d of stage dkt after MFMA 8 d + 7
  auto phase = [&](int s, const char* cbase, bool nxt, const char* nbase, bool dmado, int dkt, int dslot, bool part)
      __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 64; ++m) {
      const int i = m >> 3, j = m & 7;
      // written out so the accumulator stays in its accumulation registers
      // (through the builtin, the compiler routed some of the 64 blocks
      // through VGPRs with a copy and a 6-cycle wait after each MFMA)
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(fa[i & 3]), "v"(fb[s][j]));
      if (j == 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 2 < 8) rd_a(cbase, i + 2);
        else if (nxt) rd_a(nbase, i + 2 - 8);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nxt && (m & 3) == 2) {
        __builtin_amdgcn_sched_barrier(0);
        rd_b(nbase, s ^ 1, m >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dmado && (m & 7) == 7) {
        __builtin_amdgcn_sched_barrier(0);
        dma(dkt, dslot, m >> 3, part);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // prologue: stages 0 .. 2 in flight, wait for 0 and 1; stage 0's B blocks
  // and its first two A blocks into registers
  for (int s = 0; s < W4_NS - 1 && s < nk; ++s)
    for (int q = 0; q < W4_DMA; ++q) dma(s, s, q, s >= nkf);
  wait_vmcnt(max(0, min(nk, W4_NS - 1) - 2) * W4_DMA);
  if (nk > 0) fix_stage(0);
  if (nk > 1) fix_stage(1);
  __syncthreads();
  if (nk > 0) {
    rd_a(smem, 0);
    rd_a(smem, 1);
#pragma unroll
    for (int e = 0; e < 16; ++e) rd_b(smem, 0, e);
  }
  // step kt: stage kt + 1 (visible since the last barrier) is read, stage
  // kt + 3 issued into the slot of stage kt - 1, whose last reads completed
  // before step kt - 1's MFMAs used them (so a bare s_barrier suffices); at
  // the end, stage kt + 2 must have landed.  Steady steps: every stage they
  // issue is whole in K.
  auto step_steady = [&](int kt, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    phase(slot & 1, smem + slot * W4_STAGE, true, smem + ((slot + 1) % W4_NS) * W4_STAGE, true, kt + 3,
          (slot + 3) % W4_NS, false);
    wait_vmcnt(W4_DMA);
    __builtin_amdgcn_s_barrier();
  };
  // the last steps, register sets by compile-time parity (kt is even here)
  auto step_tail = [&](int kt, auto PAR) __attribute__((always_inline)) {
    constexpr int par = decltype(PAR)::value;
    const bool dmado = kt + 3 < nk;
    phase(par, smem + (kt % W4_NS) * W4_STAGE, kt + 1 < nk, smem + ((kt + 1) % W4_NS) * W4_STAGE, dmado, kt + 3,
          (kt + 3) % W4_NS, kt + 3 >= nkf);
    if (kt + 2 < nk) {
      wait_vmcnt(dmado ? W4_DMA : 0);
      fix_stage(kt + 2);
    }
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 6 < nkf; kt += 4) {
    step_steady(kt, Slot<0>());
    step_steady(kt + 1, Slot<1>());
    step_steady(kt + 2, Slot<2>());
    step_steady(kt + 3, Slot<3>());
  }
  for (; kt < nk; kt += 2) {
    step_tail(kt, Slot<0>());
    if (kt + 1 < nk) step_tail(kt + 1, Slot<1>());
  }
  // the MFMAs were written out, so the compiler does not know that the
  // accumulators are MFMA results: wait out their latency (24 wait states,
  // above what a 16x16x32 result needs) before the epilogue reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // clipped epilogue, 32 rows (two block rows) of the wave's block per pass:
  // lane l's accumulator r of 16x16 block (i, j) is row 4 (l / 16) + r,
  // column l % 16 of that block
  if (p.c_f32) {
    char* ep = smem + wave * W4_F32_WAVE;
#pragma unroll
    for (int pss = 0; pss < 4; ++pss) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            *(float*)(ep + (ii * 16 + 4 * (lane >> 4) + r) * W4_F32_PITCH + (j * 16 + (lane & 15)) * 4) =
                acc[2 * pss + ii][j][r];
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
#pragma unroll 2
      for (int c = lane; c < 32 * 32; c += 64) {
        const int row = c >> 5, ch = c & 31;
        const int64_t grow = m0 + wm * 128 + pss * 32 + row;
        const int64_t gcol = n0 + wn * 128 + ch * 4;
        if (grow >= p.M) continue;
        u32x4 v = *(const u32x4*)(ep + row * W4_F32_PITCH + ch * 16);
        if (p.acc) {
          const u32x4 a = ld16((const char*)(p.acc + grow * p.ldacc + gcol));
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(__uint_as_float(v[e]) + __uint_as_float(a[e]));
        }
        st16(p.C + (grow * p.ldc + gcol) * 4, v);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    return;
  }
  char* ep = smem + wave * W4_EPI_WAVE;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(__bf16*)(ep + (i * 16 + 4 * (lane >> 4) + r) * W4_EPI_PITCH + (j * 16 + (lane & 15)) * 2) =
            (__bf16)acc[i][j][r];
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (int c = lane; c < 128 * 16; c += 64) {
    const int row = c >> 4, ch = c & 15;
    const int64_t grow = m0 + wm * 128 + row;
    if (grow >= p.M) continue;
    st16(p.C + (grow * p.ldc + n0 + wn * 128 + ch * 8) * 2, *(const u32x4*)(ep + row * W4_EPI_PITCH + ch * 16));
  }
}

// main tile shape (the 8-wave kernel's: 128 x 64 accumulators per wave, two
// waves per SIMD, 4-stage ring; its stage sizes and LDS footprint come from
// here); edge strip: the template kernel on small stages, so a deep ring
// hides the load latency of its long K loop
using MainCfg = Cfg<256, 256, 2, 4, 4>;
using EdgeCfg = Cfg<64, 32, 2, 1, 16>;

template <class CF>
int launch(const char* name, GemmParams p, int64_t cols, hipStream_t s) {
  p.tiles_m = (int32_t)((p.M + CF::BM - 1) / CF::BM);
  p.tiles_n = (int32_t)((cols + CF::BN - 1) / CF::BN);
  const int64_t n_wg = (int64_t)p.tiles_m * p.tiles_n;
  if (n_wg == 0) return STG_OK;
  launch_kernel(name, gemm_kernel<CF>, dim3((unsigned)n_wg), dim3(CF::NT), (uint32_t)CF::LDS_B, s, p);
  return check_launch(name);
}

// Main kernel for operand rows that are not 16-byte aligned: 8 waves, two per
// SIMD, each owning a 128 x 64 block of the 256 x 256 tile as 8 x 4 blocks of
// v_mfma_f32_16x16x32_bf16 (16 x 16 outputs, 32 K values per instruction).
// At the power limit the 16 x 16 x 32 instruction costs less per flop than
// the 32 x 32 x 16 one (alone, on random operands held in registers: 2.17
// against 1.90 PFLOP/s), and at (8191, 8193, 4097) this kernel runs 7-9%
// faster than the same kernel on 32 x 32 x 16 (1101-1153 against 1030-1060
// TFLOP/s, with identical output bits in every case compared).
//  * Stages, ring, swizzles, zero-fill and K-edge patch as the 4-wave kernel
//    (descriptors rebased per stage, so any stride works); 4 DMA
//    instructions per wave and stage, one after every 8 MFMAs.
//  * Operands: a 32-K stage feeds each 16 x 16 x 32 MFMA whole, so the B
//    blocks of the next stage are read into a second register set during the
//    current one (8 transposed reads, one after every 4 MFMAs), and A blocks
//    are read just in time, two 16-row blocks ahead through four rolling
//    registers (the next stage's first two at the end of the current one):
//    double-buffering A as well would need 96 operand registers, past what
//    two waves per SIMD leave beside 128 accumulators.
//  * The loop is unrolled over the ring's four slots (and the last steps over
//    the two register sets), so every index into the register arrays is a
//    constant: a run-time index would put them in scratch memory.
typedef float f32x4a __attribute__((ext_vector_type(4)));
template <int V>
using Ix = std::integral_constant<int, V>;
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_w8_kernel(GemmParams p) {
  using CF = Cfg<256, 256, 2, 4, 4>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CF::WN, wn = wave % CF::WN;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * CF::BM;
  const int64_t n0 = p.n_base + (int64_t)tn * CF::BN;
  const int nk = (int)((p.K + BK - 1) / BK);
  const int nkf = (int)(p.K / BK);

  auto a_chunk = [&](int q, int& r, int& c) __attribute__((always_inline)) {
    const int pos = (wave * CF::A_DMA_W + q) * 64 + lane;
    r = pos >> 2;
    c = a_phys(r, pos & 3);
  };
  auto b_chunk = [&](int q, int& k, int& c) __attribute__((always_inline)) {
    const int pos = (wave * CF::B_DMA_W + q) * 64 + lane;
    k = pos / CF::B_CPR;
    c = (pos % CF::B_CPR) ^ b_swz<CF::B_CPR>(k);
  };
  uint32_t a_off[CF::A_DMA_W], b_off[CF::B_DMA_W];
  int a_kc[CF::A_DMA_W], b_k[CF::B_DMA_W];
#pragma unroll
  for (int q = 0; q < CF::A_DMA_W; ++q) {
    int r, c;
    a_chunk(q, r, c);
    a_kc[q] = 8 * c;
    a_off[q] = m0 + r < p.M ? (uint32_t)(r * p.lda * 2 + c * 16) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < CF::B_DMA_W; ++q) {
    int k, c;
    b_chunk(q, k, c);
    b_k[q] = k;
    b_off[q] = n0 + 8 * c + 8 <= p.N ? (uint32_t)(k * p.ldb * 2 + c * 16) : kOOB;
  }
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);
  auto stage_rsrc = [&](int kt, u32x4_s& rsa, u32x4_s& rsb) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)kt * BK;
    rsa = rsrc_words(p.A + (m0 * p.lda + k0) * 2, ((p.M - 1 - m0) * p.lda + (p.K - k0)) * 2);
    rsb = rsrc_words(p.B + (k0 * p.ldb + n0) * 2, ((p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2);
  };
  auto dma_one = [&](int kt, int slot, int q, const u32x4_s& rsa, const u32x4_s& rsb) __attribute__((always_inline)) {
    const uint32_t st = smem_lds + slot * CF::STAGE_B;
    const int kleft = kt < nkf ? BK : (int)(p.K - (int64_t)kt * BK);
    if (q < CF::A_DMA_W) {
      dma16(rsa, a_kc[q] + 8 <= kleft ? a_off[q] : kOOB, st + (wave * CF::A_DMA_W + q) * 1024);
    } else {
      const int qb = q - CF::A_DMA_W;
      dma16(rsb, b_k[qb] < kleft ? b_off[qb] : kOOB, st + CF::A_STAGE_B + (wave * CF::B_DMA_W + qb) * 1024);
    }
  };
  auto fix_stage = [&](int kt) __attribute__((always_inline)) {
    const int64_t k0 = (int64_t)kt * BK;
    if (!(k0 + BK > p.K && (p.K & 7))) return;
    char* st = smem + (kt % CF::NSTAGE) * CF::STAGE_B;
#pragma unroll
    for (int q = 0; q < CF::A_DMA_W; ++q) {
      int r, c;
      a_chunk(q, r, c);
      const int64_t col = k0 + 8 * c, left = p.K - col;
      if (m0 + r < p.M && left > 0 && left < 8) {
        const uint16_t* src = (const uint16_t*)(p.A + ((m0 + r) * p.lda + col) * 2);
        u32x4 v = {0, 0, 0, 0};
        for (int e = 0; e < 8; ++e)
          if (e < left) vec_set<2>(v, e, src[e]);
        *(u32x4*)(st + (wave * CF::A_DMA_W + q) * 1024 + lane * 16) = v;
      }
    }
  };

  f32x4a acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  constexpr int ALOOK = 2, FAN = 4;  // A blocks read this many rows ahead; rolling registers
  bf16x8 fa[FAN], fb[2][4];
  // per-lane LDS offsets within a stage.  A block i: row ar + 16 i, chunk
  // lane / 16 (rows 16 apart share the swizzle: i adds 1024).  B block j
  // (transposed reads): lane t of 16-lane group g reads row 8 g + 4 h + t / 4
  // at columns wn 64 + 16 j + 4 (t % 4) .. + 3 and receives column 16 j + t,
  // K values 8 g + 4 h .. + 3 (h adds 2048).  The 16x16x32 operand layout:
  // lane l holds row (column) l % 16, K values 8 (l / 16) .. + 7.
  const int ar = wm * 128 + (lane & 15);
  const uint32_t a_lds = ar * 64 + (a_phys(ar, lane >> 4) << 4);
  uint32_t b_lds[4];
  {
    const int g = lane >> 4, t = lane & 15;
    const int row = 8 * g + (t >> 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 64 + j * 16 + 4 * (t & 3);
      b_lds[j] = CF::A_STAGE_B + row * 512 + ((col >> 3) ^ b_swz<32>(row)) * 16 + (col & 7) * 2;
    }
  }
  auto rd_a = [&](const char* base, int i) __attribute__((always_inline)) {
    fa[i % FAN] = *(const bf16x8*)(base + a_lds + i * 1024);
  };
  auto rd_b = [&](const char* base, int s, int e) __attribute__((always_inline)) {
    const int j = e >> 1, h = e & 1;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + b_lds[j] + h * 2048));
    s16x8 cur = __builtin_bit_cast(s16x8, fb[s][j]);
#pragma unroll
    for (int x = 0; x < 4; ++x) cur[4 * h + x] = v[x];
    fb[s][j] = __builtin_bit_cast(bf16x8, cur);
  };
  // the 32 MFMAs of stage kt (A rolling, B in set s), row by row: A block
  // i + 2 read at the start of row i (the next stage's blocks 0, 1 at rows 6,
  // 7); B read e of the next stage into the other set after MFMA 4 e + 1; DMA
  // instruction d of stage dkt after MFMA 8 d + 7 (scheduling barriers pin
  // the order: a wave issues in order, and a burst of DMA would hold back the
  // MFMAs behind it)
  auto phase = [&](int s, const char* cbase, bool nxt, const char* nbase, bool dmado, int dkt, int dslot,
                   const u32x4_s& rsa, const u32x4_s& rsb) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int i = m >> 2, j = m & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i % FAN], fb[s][j], acc[i][j], 0, 0, 0);
      if (j == 0) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + ALOOK < 8) rd_a(cbase, i + ALOOK);
        else if (nxt) rd_a(nbase, i + ALOOK - 8);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (nxt && (m & 3) == 1) {
        __builtin_amdgcn_sched_barrier(0);
        rd_b(nbase, s ^ 1, m >> 2);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dmado && (m & 7) == 7) {
        __builtin_amdgcn_sched_barrier(0);
        dma_one(dkt, dslot, m >> 3, rsa, rsb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  for (int s = 0; s < CF::NSTAGE - 1 && s < nk; ++s) {
    u32x4_s rsa, rsb;
    stage_rsrc(s, rsa, rsb);
    for (int q = 0; q < CF::DMA_W; ++q) dma_one(s, s, q, rsa, rsb);
  }
  wait_vmcnt(max(0, min(nk, CF::NSTAGE - 1) - 2) * CF::DMA_W);
  if (nk > 0) fix_stage(0);
  if (nk > 1) fix_stage(1);
  __syncthreads();
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < ALOOK; ++i) rd_a(smem, i);
#pragma unroll
    for (int e = 0; e < 8; ++e) rd_b(smem, 0, e);
  }
  // step kt: stage kt + 1 (visible since the last barrier) is read, stage
  // kt + 3 issued into the slot of stage kt - 1 (its last reads completed
  // before step kt - 1's MFMAs used them); at the end stage kt + 2 must have
  // landed.  Steady steps: every stage they issue is whole in K.
  auto step_steady = [&](int kt, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    u32x4_s rsa, rsb;
    stage_rsrc(kt + 3, rsa, rsb);
    phase(slot & 1, smem + slot * CF::STAGE_B, true, smem + ((slot + 1) % 4) * CF::STAGE_B, true, kt + 3,
          (slot + 3) % 4, rsa, rsb);
    wait_vmcnt(CF::DMA_W);
    __builtin_amdgcn_s_barrier();
  };
  // the last steps, register sets by compile-time parity (kt is even here)
  auto step_tail = [&](int kt, auto PAR) __attribute__((always_inline)) {
    constexpr int par = decltype(PAR)::value;
    const bool dmado = kt + 3 < nk;
    u32x4_s rsa, rsb;
    stage_rsrc(kt + 3, rsa, rsb);
    phase(par, smem + (kt % 4) * CF::STAGE_B, kt + 1 < nk, smem + ((kt + 1) % 4) * CF::STAGE_B, dmado, kt + 3,
          (kt + 3) % 4, rsa, rsb);
    if (kt + 2 < nk) {
      wait_vmcnt(dmado ? CF::DMA_W : 0);
      fix_stage(kt + 2);
    }
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 6 < nkf; kt += 4) {
    step_steady(kt, Ix<0>());
    step_steady(kt + 1, Ix<1>());
    step_steady(kt + 2, Ix<2>());
    step_steady(kt + 3, Ix<3>());
  }
  for (; kt < nk; kt += 2) {
    step_tail(kt, Ix<0>());
    if (kt + 1 < nk) step_tail(kt + 1, Ix<1>());
  }

  // clipped epilogue: lane l's accumulator r of 16x16 block (i, j) is row
  // 4 (l / 16) + r, column l % 16 of that block
  if (p.c_f32) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (col >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = m0 + wm * 128 + i * 16 + 4 * (lane >> 4) + r;
          if (row < p.M)
            *(float*)(p.C + (row * p.ldc + col) * 4) = p.acc ? acc[i][j][r] + p.acc[row * p.ldacc + col] : acc[i][j][r];
        }
      }
    return;
  }
  char* ep = smem + wave * CF::EPI_WAVE_B;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *(__bf16*)(ep + (i * 16 + 4 * (lane >> 4) + r) * CF::EPI_PITCH_B + (j * 16 + (lane & 15)) * 2) =
            (__bf16)acc[i][j][r];
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = CF::WTN / 8;
  for (int c = lane; c < CF::WTM * CPR; c += 64) {
    const int row = c / CPR, ch = c % CPR;
    const int64_t grow = m0 + wm * CF::WTM + row;
    const int64_t gcol = n0 + wn * CF::WTN + ch * 8;
    if (grow >= p.M || gcol >= p.N) continue;
    const u32x4 v = *(const u32x4*)(ep + row * CF::EPI_PITCH_B + ch * 16);
    char* dst = p.C + (grow * p.ldc + gcol) * 2;
    if (gcol + 8 <= p.N) {
      st16(dst, v);
    } else {
      for (int e = 0; e < 8; ++e)
        if (gcol + e < p.N) store_elem<2>(dst + e * 2, vec_get<2>(v, e));
    }
  }
}

// Raises the kernels' dynamic LDS limit once on each device.
bool lds_configured() {
  static OncePerDevice once;
  return once.run([] {
    return hipFuncSetAttribute((const void*)gemm_w8_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               MainCfg::LDS_B) == hipSuccess &&
           hipFuncSetAttribute((const void*)gemm_w4_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, W4_LDS) ==
               hipSuccess &&
           hipFuncSetAttribute((const void*)gemm_kernel<EdgeCfg>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               EdgeCfg::LDS_B) == hipSuccess;
  });
}

}  // namespace
}  // namespace stg

using namespace stg;

namespace stg {

int gemm_bf16(const GemmNames& names, const void* A, int64_t lda, const void* B, int64_t ldb, const float* acc,
              int64_t ldacc, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t c_dtype, hipStream_t s) {
  const char* name = names.entry;
  if (M < 0 || N < 0 || K < 0) return fail(STG_ERR_INVALID, "%s: negative size", name);
  if (c_dtype != STG_BF16 && c_dtype != STG_F32)
    return fail(STG_ERR_UNSUPPORTED, "%s: c_dtype must be STG_BF16 or STG_F32", name);
  if (lda < (K > 0 ? K : 1) || ldb < (N > 0 ? N : 1) || ldc < (N > 0 ? N : 1) || (acc && ldacc < N))
    return fail(STG_ERR_INVALID, "%s: row strides must be >= the row lengths", name);
  if (acc && c_dtype != STG_F32) return fail(STG_ERR_UNSUPPORTED, "%s: an accumulator input needs fp32 output", name);
  if (M == 0 || N == 0) return STG_OK;
  if (!C || (K > 0 && (!A || !B))) return fail(STG_ERR_INVALID, "%s: null operand", name);
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return fail(STG_ERR_RANGE, "%s: size too large", name);
  // 32-bit buffer offsets within one stage: BM rows of A, BK rows of B
  if ((int64_t)MainCfg::BM * lda * 2 + 256 >= kMaxOffset32 || (int64_t)BK * ldb * 2 + 512 >= kMaxOffset32)
    return fail(STG_ERR_RANGE, "%s: a stage of A or B spans more than 2^31 bytes", name);
  if (!lds_configured())
    return fail(STG_ERR_LAUNCH, "%s: cannot reserve LDS for the GEMM kernels", name);
  GemmParams p{};
  p.A = (const char*)A;
  p.B = (const char*)B;
  p.C = (char*)C;
  p.acc = acc;
  p.lda = lda, p.ldb = ldb, p.ldc = ldc, p.ldacc = ldacc;
  p.M = M, p.N = N, p.K = K;
  p.c_f32 = c_dtype == STG_F32;
  const int64_t n_main = (N / MainCfg::BN) * MainCfg::BN;
  int rc;
  p.n_base = 0;
  // 16-byte aligned rows take the 4-wave kernel (its whole-panel descriptors
  // also need the B panel, read up to a stage past K, below 2^31 bytes)
  const bool w4 = (lda & 7) == 0 && (ldb & 7) == 0 && ((uintptr_t)A & 15) == 0 && ((uintptr_t)B & 15) == 0 &&
                  (K + 2 * BK) * ldb * 2 < kMaxOffset32;
  if (n_main > 0 && w4) {
    p.tiles_m = (int32_t)((M + 255) / 256);
    p.tiles_n = (int32_t)(n_main / 256);
    launch_kernel(names.main, gemm_w4_kernel, dim3((unsigned)((int64_t)p.tiles_m * p.tiles_n)), dim3(256),
                  (uint32_t)W4_LDS, s, p);
    if ((rc = check_launch(names.main))) return rc;
  } else if (n_main > 0) {
    p.tiles_m = (int32_t)((M + MainCfg::BM - 1) / MainCfg::BM);
    p.tiles_n = (int32_t)(n_main / MainCfg::BN);
    launch_kernel(names.main, gemm_w8_kernel, dim3((unsigned)((int64_t)p.tiles_m * p.tiles_n)), dim3(MainCfg::NT),
                  (uint32_t)MainCfg::LDS_B, s, p);
    if ((rc = check_launch(names.main))) return rc;
  }
  p.n_base = n_main;
  const int64_t rem = N - n_main;
  if (rem > 8) return launch<EdgeCfg>(names.edge, p, rem, s);
  if (rem > 0) {
    const unsigned grid = (unsigned)((M + SK_ROWS - 1) / SK_ROWS);
    switch (rem) {
#define STG_SK(r) case r: launch_kernel(names.skinny, gemm_skinny_kernel<r>, dim3(grid), dim3(256), 0, s, p); break;
      STG_SK(1) STG_SK(2) STG_SK(3) STG_SK(4) STG_SK(5) STG_SK(6) STG_SK(7) STG_SK(8)
#undef STG_SK
    }
    return check_launch(names.skinny);
  }
  return STG_OK;
}

}  // namespace stg

extern "C" int gemm_bounded(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                            int64_t M, int64_t N, int64_t K, int32_t c_dtype, void* stream) {
  clear_error();
  static const GemmNames names{"gemm_bounded", "gemm_bounded/main", "gemm_bounded/edge", "gemm_bounded/skinny"};
  return gemm_bf16(names, A, lda, B, ldb, nullptr, 0, C, ldc, M, N, K, c_dtype, as_stream(stream));
}
