// Block-scaled GEMM  C = (A . a_scale) (B . b_scale) + acc  (fp8 / fp4
// operands, e8m0 block scales, fp32 accumulation).
//
// Semantics (cuTile.jl Operations, muladd_scaled: each scale element
// multiplies a contiguous block of K / K_s values along K of its operand;
// a / b in f8e4m3fn, f8e5m2 or f4e2m1fn, accumulator f32; reinterpret: FP4
// travels two values per byte).  Layout read here: A is (M, K) and B is given
// K-major as Bt (N, K), so every scale block and every FP4 pair is a
// contiguous run of its row; the even FP4 element sits in the low nibble.
//
// gfx950 design: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies a 32 x 64 by a
// 64 x 32 block with one e8m0 scale per row (column) and 32 K values, which
// is the block-scaled product itself when the scale block is a multiple of 32
// K values.  Lane l of an operand holds row (column) l % 32; the scale that
// lane l supplies covers the 32-value K block l / 32 of the step, and that
// block is (measured with one-hot operands) fp8: bytes 0-15 of every lane for
// block 0 and bytes 16-31 for block 1; fp4 (16 bytes, two values per byte,
// even element low): all of lane half l / 32.  The order of K inside a block
// does not matter as long as both operands use the same one, so a lane takes
// the 16-byte chunks 2p + l / 32 (p = 0, 1) of a stage's 64-byte K run: for
// fp8 the two halves of the stage's one MFMA step (K values 32 p + 16 (l / 32)
// .. +15), for fp4 its 16 bytes of MFMA step p (K values 64 p + 32 (l / 32)
// .. +31).  The accumulator layout is the 32x32 MFMA layout.
//  * Tiles 256 x 256 on 4 waves, one per SIMD, each with 128 x 128
//    accumulators: with a SIMD to itself a wave has 512 registers, enough to
//    hold the next stage's operands while the current ones feed the MFMAs,
//    and a 128 x 128 wave tile reads a third less LDS per MFMA than 128 x 64.
//  * Both operands are staged by LDS DMA into 64-byte rows -- 64 fp8 or 128
//    fp4 K values per stage -- with the conflict-free chunk swizzle of the bf16
//    GEMM, out-of-range rows and K chunks landing as zeros; a 4-slot ring, the
//    DMA of stage k+4 spread among stage k's MFMAs (stage k itself was read
//    into registers during step k-1).
//  * The scale bytes travel the same way, once per group of 4 stages: per
//    row the 16-byte aligned 32-byte window that holds the row's (at most
//    16) scale bytes of the group is DMA'd into one of two window buffers,
//    and each lane reads its bytes from LDS: with 32-value blocks and scale
//    rows that start 16-byte aligned, a whole group's bytes at once, packed
//    into one register per block row and selected per MFMA with op_sel;
//    otherwise one byte per MFMA step.  (Per-stage windows would cost
//    one L2 request per row and stage for a few bytes, doubling the requests
//    of the whole kernel.)  No load the compiler can see is in flight in the
//    K loop, so its own waits never force a later stage's DMA to land early;
//    one explicit wait per step (all but the two newest stages, and the window
//    issued among them) publishes stage k+2 while stage k+1 is read into the
//    second register set.  Scale bytes of K blocks past K are capped to a
//    finite value, so a NaN byte beyond the matrix cannot reach the zero data
//    there.
//  * Clipped fp32 epilogue adding the optional accumulator input.
//  * Columns past the last whole 256-column tile, when at most 8, go to a
//    skinny kernel instead of a tile column of their own.
#include "gemm_common.h"

#include <type_traits>

namespace stg {
namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16_s __attribute__((ext_vector_type(16)));
typedef float f32x2_s __attribute__((ext_vector_type(2)));

struct ScaledParams {
  const char* A;      // (M, K), row stride lda bytes
  const char* B;      // Bt (N, K), row stride ldb bytes
  const char* sa;     // e8m0 (M, K / block) at sa + sa_delta, row stride lds_a; sa 16-byte aligned
  const char* sb;     // e8m0 (N, K / block) at sb + sb_delta, row stride lds_b; sb 16-byte aligned
  const float* acc;   // (M, N) f32, row stride ldacc, or null
  float* C;           // (M, N) f32, row stride ldc
  int64_t lda, ldb, lds_a, lds_b, ldacc, ldc;
  int64_t M, N, K;
  int64_t sa_bytes, sb_bytes;  // readable bytes from sa / sb (whole 16-byte chunks)
  int32_t sa_delta, sb_delta;  // 0..15
  int32_t lg_bq;               // log2(block / 32)
  int32_t nkb;                 // K / block
  int32_t tiles_m, tiles_n;
};

constexpr int kSBM = 256, kSBN = 256, kSWN = 2, kSNW = 4, kSNT = kSNW * 64;
constexpr int kSFM = 4, kSFN = 4;  // 32x32 blocks per wave: 128 x 128
constexpr int kSNS = 4;            // ring slots
constexpr int kRowB = 64;          // bytes per operand row per stage
constexpr int kSG = 4;             // stages per scale window group
constexpr int kSWin = 32;          // bytes of scale window per row and group
constexpr int kAStage = kSBM * kRowB, kBStage = kSBN * kRowB;
constexpr int kSlot = kAStage + kBStage;  // 32 KiB
constexpr int kASc = kSBM * kSWin, kBSc = kSBN * kSWin;
constexpr int kScBuf = kASc + kBSc;  // 16 KiB per window buffer, two of them
constexpr int kADma = kAStage / 1024 / kSNW, kBDma = kBStage / 1024 / kSNW;
constexpr int kDma = kADma + kBDma;         // operand DMA instructions per thread and stage
constexpr int kWDmaOp = kASc / 1024 / kSNW;  // window DMA instructions per thread and operand
constexpr int kWDma = 2 * kWDmaOp;
constexpr int kScaledLds = kSNS * kSlot + 2 * kScBuf;  // 160 KiB
static_assert(kWDmaOp * kSNT * 16 == kASc && kASc == kBSc, "whole windows per DMA round");
static_assert(kScaledLds <= 160 * 1024, "LDS");

// FA / FB: operand format codes of the scaled MFMA (0 e4m3, 1 e5m2, 4 e2m1);
// BITS: 8 for fp8 operands, 4 for fp4 (both operands of one width).  PK: the
// packed-scale path, for 32-value blocks whose scale rows start 16-byte
// aligned (row strides and bases multiples of 16): each lane reads the scale
// bytes of a whole group of 4 stages with one 8-byte LDS read per block row
// (fp4: two), gathers its own into one register, and each MFMA selects its
// byte with op_sel; otherwise one byte is read per MFMA step.
template <int FA, int FB, int BITS, bool PK>
__global__ __launch_bounds__(kSNT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_scaled_kernel(
    ScaledParams p) {
  constexpr int KS = kRowB * 8 / BITS;    // K values per stage: 64 (fp8) / 128 (fp4)
  constexpr int S = KS / 64;              // MFMA steps per stage
  constexpr int CHUNK_K = 16 * 8 / BITS;  // K values per 16-byte chunk
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kSWN, wn = wave % kSWN;
  const int half = lane >> 5;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kSBM, n0 = (int64_t)tn * kSBN;
  const int nk = (int)((p.K + KS - 1) / KS);
  const int64_t row_bytes = p.K * BITS / 8;

  f32x16_s acc[kSFM][kSFN];
#pragma unroll
  for (int i = 0; i < kSFM; ++i)
#pragma unroll
    for (int j = 0; j < kSFN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // operand DMA chunks of this lane (row r of the stage, logical chunk c):
  // offsets are the same for every stage (the descriptors move with K)
  uint32_t a_off[kADma], b_off[kBDma];
  int a_kc[kADma], b_kc[kBDma];  // first K value of the chunk within its stage
#pragma unroll
  for (int q = 0; q < kADma; ++q) {
    const int pos = (wave * kADma + q) * 64 + lane;
    const int r = pos >> 2, c = a_phys(r, pos & 3);
    a_kc[q] = c * CHUNK_K;
    a_off[q] = m0 + r < p.M ? (uint32_t)(r * p.lda + c * 16) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < kBDma; ++q) {
    const int pos = (wave * kBDma + q) * 64 + lane;
    const int r = pos >> 2, c = a_phys(r, pos & 3);
    b_kc[q] = c * CHUNK_K;
    b_off[q] = n0 + r < p.N ? (uint32_t)(r * p.ldb + c * 16) : kOOB;
  }
  // window DMA q of this thread: LDS chunk t & 1 of the window of row t / 2,
  // t = (wave * kWDmaOp + q) * 64 + lane, which holds the window's chunk
  // (t & 1) ^ bit 3 of the row: the 32 rows whose scale bytes one read
  // instruction fetches (same byte of each window, windows 32 bytes apart)
  // then fall on 16 banks instead of 8.  Byte offsets of the rows' first
  // scales from the 16-byte aligned bases (below 2^31).
  uint32_t sa_row[kWDmaOp], sb_row[kWDmaOp], s_ch[kWDmaOp];
  bool sa_ok[kWDmaOp], sb_ok[kWDmaOp];
#pragma unroll
  for (int q = 0; q < kWDmaOp; ++q) {
    const int t = (wave * kWDmaOp + q) * 64 + lane, srow = t >> 1;
    s_ch[q] = 16 * ((t & 1) ^ ((srow >> 3) & 1));
    sa_ok[q] = m0 + srow < p.M;
    sb_ok[q] = n0 + srow < p.N;
    sa_row[q] = sa_ok[q] ? (uint32_t)(p.sa_delta + (m0 + srow) * p.lds_a) : 0u;
    sb_row[q] = sb_ok[q] ? (uint32_t)(p.sb_delta + (n0 + srow) * p.lds_b) : 0u;
  }
  const u32x4_s rs_sa = rsrc_words(p.sa, p.sa_bytes), rs_sb = rsrc_words(p.sb, p.sb_bytes);
  // where this lane's scale rows start within their windows: (row offset) mod 16
  int a_ph[kSFM], b_ph[kSFN];
#pragma unroll
  for (int i = 0; i < kSFM; ++i) {
    const int64_t r = m0 + wm * 128 + i * 32 + (lane & 31);
    a_ph[i] = (int)((p.sa_delta + (r < p.M ? r : 0) * p.lds_a) & 15);
  }
#pragma unroll
  for (int j = 0; j < kSFN; ++j) {
    const int64_t r = n0 + wn * 128 + j * 32 + (lane & 31);
    b_ph[j] = (int)((p.sb_delta + (r < p.N ? r : 0) * p.lds_b) & 15);
  }
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  auto first_block = [&](int kt) { return (int)(((uint32_t)kt * (KS / 32)) >> p.lg_bq); };
  // K values of stage kt still inside K (clamped to the int range)
  auto k_left = [&](int kt) {
    const int64_t kl = p.K - (int64_t)kt * KS;
    return (int)(kl < 0 ? 0 : kl > INT32_MAX ? INT32_MAX : kl);
  };
  // Descriptors of stage kt's operand bytes.  fp8: one descriptor per
  // operand panel for the whole K loop, the stage chosen by the DMA
  // instruction's scalar offset kt * kRowB (rows past M or N still start
  // past num_records, since a row stride is at least a row; with the host's
  // 2^31 bound on 256 row strides, vector plus scalar offset of every chunk
  // inside the matrix stays below num_records, whether or not the range
  // check counts the scalar offset); fp4: one
  // descriptor per stage starting at the stage's bytes.  The same bytes land
  // either way; each is the faster one for its width (measured at 8191 x
  // 8193 x 4096: fp8 2% faster on panels, fp4 3% slower).
  constexpr bool kPanel = BITS == 8;
  auto stage_rsrc = [&](int kt, u32x4_s& rsa, u32x4_s& rsb) {
    const int64_t kb = kPanel ? 0 : (int64_t)kt * kRowB;  // byte offset of the descriptor in a row
    rsa = rsrc_words(p.A + m0 * p.lda + kb, (p.M - 1 - m0) * p.lda + (row_bytes - kb));
    rsb = rsrc_words(p.B + n0 * p.ldb + kb, (p.N - 1 - n0) * p.ldb + (row_bytes - kb));
  };
  // DMA instruction q of stage kt into its ring slot (A chunks, then B);
  // chunks at or past K land as zeros
  auto dma_one = [&](int slot, int kt, int kleft, int q, const u32x4_s& rsa, const u32x4_s& rsb) {
    const uint32_t st = smem_lds + slot * kSlot;
    if (q < kADma) {
      const uint32_t off = a_kc[q] < kleft ? a_off[q] : kOOB;
      const uint32_t dst = st + (wave * kADma + q) * 1024;
      if constexpr (kPanel)
        dma16s(rsa, off, uniform_sgpr((uint32_t)kt * kRowB), uniform_sgpr(dst));
      else
        dma16(rsa, off, dst);
    } else {
      const int qb = q - kADma;
      const uint32_t off = b_kc[qb] < kleft ? b_off[qb] : kOOB;
      const uint32_t dst = st + kAStage + (wave * kBDma + qb) * 1024;
      if constexpr (kPanel)
        dma16s(rsb, off, uniform_sgpr((uint32_t)kt * kRowB), uniform_sgpr(dst));
      else
        dma16(rsb, off, dst);
    }
  };
  // window DMA instruction q (A, then B) of group g into buffer g % 2; kb0:
  // first scale block of the group; windows of groups past K and of rows past
  // the matrix land as zeros
  auto wdma_one = [&](int g, int kb0, int q) {
    const uint32_t wb = smem_lds + kSNS * kSlot + (g & 1) * kScBuf;
    const bool is_a = q < kWDmaOp;
    const int qq = is_a ? q : q - kWDmaOp;
    const uint32_t win = ((is_a ? sa_row[qq] : sb_row[qq]) + (uint32_t)kb0) & ~15u;
    const uint32_t off = (is_a ? sa_ok[qq] : sb_ok[qq]) && kb0 < p.nkb ? win + s_ch[qq] : kOOB;
    dma16(is_a ? rs_sa : rs_sb, off, wb + (is_a ? 0 : kASc) + (wave * kWDmaOp + qq) * 1024);
  };

  // Operand registers, double-buffered by step parity P; dwords 4h .. 4h+3
  // of fa[P][i] / fb[P][j] hold the lane's 16-byte chunk 2h + half: fp8 --
  // the one MFMA step's 32 bytes (scale blocks 0 and 1 of the step), in the
  // register order the instruction takes; fp4 -- the 16 bytes of MFMA step h.
  i32x8 fa[2][kSFM], fb[2][kSFN];
  int sca[2][kSFM][S], scb[2][kSFN][S];
  // packed path: byte i of scp[w][h] is the scale of K block kbg + 8 h +
  // 2 i + half of the current group (kbg: its first block) for block row w
  // (A rows, then B rows); scr[w]: the 8 raw window bytes just read
  uint32_t scp[kSFM + kSFN][S];
  uint64_t scr[kSFM + kSFN];
  // v_perm selector gathering window bytes half, 2 + half, 4 + half, 6 + half
  const uint32_t s_sel = (uint32_t)half | (uint32_t)(2 + half) << 8 | (uint32_t)(4 + half) << 16 |
                         (uint32_t)(6 + half) << 24;
  // LDS byte offsets of this lane's chunks half and 2 + half of its first A
  // and B rows; rows 32 i further on keep the swizzle (bits 1-2 of r/2 and
  // r/4 do not change), so the other blocks are at fixed distances
  const int ra0 = wm * 128 + (lane & 31), rb0 = wn * 128 + (lane & 31);
  // window chunks are swapped in rows with bit 3 set (rows 32 i further on
  // keep it): a scale byte at window position x sits at x ^ s_swz
  const int s_swz = 16 * (((lane & 31) >> 3) & 1);
  const int a_l0 = ra0 * kRowB + (a_phys(ra0, half) << 4), a_l1 = ra0 * kRowB + (a_phys(ra0, 2 + half) << 4);
  const int b_l0 = rb0 * kRowB + (a_phys(rb0, half) << 4), b_l1 = rb0 * kRowB + (a_phys(rb0, 2 + half) << 4);
  // Read instruction q of stage kt (ring slot SLOT) into buffer P: q <
  // NRD_A: half q % 2 of A block q / 2 (chunk half, then 2 + half); then the
  // same for B; then the scale bytes, A blocks then B blocks for each MFMA
  // step s.  The scale of 32-value K block kb is byte (phase + kb - kbg) of
  // its row's window of group kt / 4 (kbg: the group's first block).  The
  // 16-byte halves land in ta / tb and are joined into fa / fb by join().
  constexpr int NRD_A = 2 * kSFM, NRD_B = 2 * kSFN, NRD_S = (kSFM + kSFN) * S;
  // reads of the stage in ring slot SLOT: the packed path reads scales only
  // for a group's first stage (half 0 of its bytes) and, fp4, its third (half 1)
  auto nrd_of = [](auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    return NRD_A + NRD_B + (!PK ? NRD_S : (SLOT == 0 || (BITS == 4 && SLOT == 2)) ? kSFM + kSFN : 0);
  };
  i32x4 ta[kSFM][2], tb[kSFN][2];
  auto read_one = [&](int kt, int q, auto p_tag, auto slot_tag) {
    constexpr int P = decltype(p_tag)::value;
    constexpr int SLOT = decltype(slot_tag)::value;
    const char* as = smem + SLOT * kSlot;
    const char* bs = as + kAStage;
    if (q < NRD_A) {
      const int i = q >> 1, h = q & 1;
      ta[i][h] = *(const i32x4*)(as + (h ? a_l1 : a_l0) + i * 32 * kRowB);
    } else if (q < NRD_A + NRD_B) {
      const int j = (q - NRD_A) >> 1, h = q & 1;
      tb[j][h] = *(const i32x4*)(bs + (h ? b_l1 : b_l0) + j * 32 * kRowB);
    } else if constexpr (PK) {
      // 8 bytes, half H of the row's window bytes of group kt / 4 (window
      // position (kbg & 15) + 8 H, 8-byte aligned, chunks swapped as written)
      constexpr int H = SLOT == 2 ? 1 : 0;
      const char* sas = smem + kSNS * kSlot + ((kt / kSG) & 1) * kScBuf;
      const int kbg = first_block(kt & ~(kSG - 1));
      const int w = q - NRD_A - NRD_B;
      const int row = w < kSFM ? ra0 + w * 32 : kASc / kSWin + rb0 + (w - kSFM) * 32;
      scr[w] = *(const uint64_t*)(sas + row * kSWin + (((kbg & 15) + 8 * H) ^ s_swz));
    } else {
      const unsigned char* sas = (const unsigned char*)(smem + kSNS * kSlot + ((kt / kSG) & 1) * kScBuf);
      const unsigned char* sbs = sas + kASc;
      const int u = q - NRD_A - NRD_B, s = u / (kSFM + kSFN), w = u % (kSFM + kSFN);
      const int kbg = first_block(kt & ~(kSG - 1));
      const int kb = (int)(((uint32_t)kt * (KS / 32) + 2 * s + half) >> p.lg_bq);
      if (w < kSFM)
        sca[P][w][s] = sas[(ra0 + w * 32) * kSWin + ((((a_ph[w] + kbg) & 15) + (kb - kbg)) ^ s_swz)];
      else
        scb[P][w - kSFM][s] = sbs[(rb0 + (w - kSFM) * 32) * kSWin + ((((b_ph[w - kSFM] + kbg) & 15) + (kb - kbg)) ^ s_swz)];
    }
  };
  auto join = [&](auto p_tag) {
    constexpr int P = decltype(p_tag)::value;
#pragma unroll
    for (int i = 0; i < kSFM; ++i) fa[P][i] = __builtin_shufflevector(ta[i][0], ta[i][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < kSFN; ++j) fb[P][j] = __builtin_shufflevector(tb[j][0], tb[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // packed path, after the scale reads of stage kt (ring slot SLOT): gather
  // each lane's four bytes; bytes of blocks at or past K get a finite scale
  // (127), since the window may hold anything there (NaN included) and their
  // data is zero
  auto pack_scales = [&](int kt, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    if constexpr (PK && (SLOT == 0 || (BITS == 4 && SLOT == 2))) {
      constexpr int H = SLOT == 2 ? 1 : 0;
      const int kb0 = first_block(kt & ~(kSG - 1)) + 8 * H + half;
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) m |= kb0 + 2 * i >= p.nkb ? 0xFFu << (8 * i) : 0u;
#pragma unroll
      for (int w = 0; w < kSFM + kSFN; ++w) {
        const uint32_t v = __builtin_amdgcn_perm((uint32_t)(scr[w] >> 32), (uint32_t)scr[w], s_sel);
        scp[w][H] = (v & ~m) | (0x7F7F7F7Fu & m);
      }
    }
  };
  auto read_stage = [&](int kt, auto p_tag, auto slot_tag) {
#pragma unroll
    for (int q = 0; q < nrd_of(slot_tag); ++q) read_one(kt, q, p_tag, slot_tag);
    join(p_tag);
    pack_scales(kt, slot_tag);
  };

  // one K step on stage kt (kt % 4 == PH), whose operands are in buffer P:
  // stage kt + 1 (published) is read into buffer 1 - P and stage kt + 4's DMA
  // goes to ring slot kt % 4 (stage kt, read before the last barrier), both
  // alongside the MFMAs; when PH == 3 the window of group g = (kt + 5) / 4
  // goes first, into window buffer g % 2 (last read for stage 4g - 5, before
  // the last barrier).  At the end stage kt + 2 has landed once only what was
  // issued after it is in flight (operations complete in order): stages kt +
  // 3 and kt + 4, and the window of the step with PH == 3 among the last two;
  // the barrier publishes it, and its fence waits for the reads of kt + 1.
  auto step = [&](int kt, auto p_tag, auto ph_tag) {
    constexpr int P = decltype(p_tag)::value;
    constexpr int PH = decltype(ph_tag)::value;
    constexpr int NM = kSFM * kSFN * S;
    constexpr int NW = PH == 3 ? kWDma : 0;  // window instructions this step
    constexpr int NRD = nrd_of(std::integral_constant<int, (PH + 1) % kSNS>());
    constexpr int ND = NW + kDma;
    // this step's bookkeeping (descriptors and K bound of stage kt + 4's
    // DMA, the window's group) is issued after the first MFMA, which needs
    // only the previous step's registers: with one wave per SIMD,
    // instructions issued while an MFMA runs cost the matrix core nothing
    u32x4_s rsa, rsb;
    int g = 0, kbw = 0, kl_d = 0;
    auto cap_of = [&](int s) {
      return (int)(((uint32_t)kt * (KS / 32) + 2 * s + half) >> p.lg_bq) < p.nkb ? 255 : 127;
    };
    auto bookkeeping = [&]() {
      stage_rsrc(kt + kSNS, rsa, rsb);
      g = (kt + 5) / kSG;
      kbw = NW ? first_block(g * kSG) : 0;
      kl_d = k_left(kt + kSNS);
    };
    // stage kt + 1 is in ring slot (PH + 1) % 4; its reads go between the
    // MFMAs (fp8: two after each of the first ones; fp4: spread over all but
    // the last two, which leave the last reads time to land before the
    // barrier -- the faster placement for each, measured): issued in a burst,
    // they would fill the LDS queue and hold back the MFMAs behind them
    using PN = std::integral_constant<int, 1 - P>;
    using SN = std::integral_constant<int, (PH + 1) % kSNS>;
    // scale bytes of K blocks past K may be anything (NaN included): they
    // are capped to a finite value, their data being zero; applied a step
    // after the bytes were read (so that no wait holds the MFMAs), in place,
    // just before each value's first MFMA
    int cap = 0;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < kSFM; ++i)
#pragma unroll
        for (int j = 0; j < kSFN; ++j) {
          i32x8 av, bv;
          if (BITS == 8) {
            av = fa[P][i];
            bv = fb[P][j];
          } else if (s == 0) {  // fp4 reads only the first four registers
            av = __builtin_shufflevector(fa[P][i], fa[P][i], 0, 1, 2, 3, -1, -1, -1, -1);
            bv = __builtin_shufflevector(fb[P][j], fb[P][j], 0, 1, 2, 3, -1, -1, -1, -1);
          } else {
            av = __builtin_shufflevector(fa[P][i], fa[P][i], 4, 5, 6, 7, -1, -1, -1, -1);
            bv = __builtin_shufflevector(fb[P][j], fb[P][j], 4, 5, 6, 7, -1, -1, -1, -1);
          }
          if constexpr (PK) {
            // byte of the packed scales: fp8, stage PH of the group; fp4,
            // MFMA step s of stage PH, in word PH / 2
            constexpr int H = BITS == 8 ? 0 : PH >> 1;
            constexpr int SEL0 = BITS == 8 ? PH : 2 * (PH & 1), SEL1 = SEL0 + 1;
            const int sa_w = (int)scp[i][H], sb_w = (int)scp[kSFM + j][H];
            acc[i][j] = s == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], FA, FB, SEL0,
                                                                                 sa_w, SEL0, sb_w)
                               : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], FA, FB, SEL1,
                                                                                 sa_w, SEL1, sb_w);
          } else {
            if (i == 0 && j == 0) cap = cap_of(s);
            if (j == 0) sca[P][i][s] = min(sca[P][i][s], cap);
            if (i == 0) scb[P][j][s] = min(scb[P][j][s], cap);
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av, bv, acc[i][j], FA, FB, 0, sca[P][i][s], 0, scb[P][j][s]);
          }
          const int m = (s * kSFM + i) * kSFN + j;
          if (m == 0) {
            __builtin_amdgcn_sched_barrier(0);
            bookkeeping();
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int q = 0; q < NRD; ++q) {
            if ((BITS == 8 ? q / 2 : (q * (NM - 2)) / NRD) == m) {
              __builtin_amdgcn_sched_barrier(0);
              read_one(kt + 1, q, PN(), SN());
              __builtin_amdgcn_sched_barrier(0);
            }
          }
#pragma unroll
          for (int d = 0; d < ND; ++d) {
            const int after = ((d + 1) * NM) / ND - 1;
            if ((after < 0 ? 0 : after) == m) {
              __builtin_amdgcn_sched_barrier(0);
              if (d < NW)
                wdma_one(g, kbw, d);
              else
                dma_one(PH, kt + kSNS, kl_d, d - NW, rsa, rsb);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
    __builtin_amdgcn_sched_barrier(0);  // every MFMA is issued before the wait
    join(PN());
    pack_scales(kt + 1, SN());
    wait_vmcnt(2 * kDma + (PH == 0 || PH == 3 ? kWDma : 0));
    __syncthreads();
  };

  // (K = 0 has no stage: the epilogue writes acc or zeros)
  if (nk > 0) {
    // prologue, in the steady state's issue order: window 0, stages 0 .. 2,
    // window 1, stage 3; then wait for window 0 and stages 0 and 1
    for (int q = 0; q < kWDma; ++q) wdma_one(0, 0, q);
    for (int s = 0; s < kSNS; ++s) {
      if (s == kSNS - 1) {
        const int kbw = first_block(kSG);
        for (int q = 0; q < kWDma; ++q) wdma_one(1, kbw, q);
      }
      u32x4_s rsa, rsb;
      stage_rsrc(s, rsa, rsb);
#pragma unroll
      for (int q = 0; q < kDma; ++q) dma_one(s, s, k_left(s), q, rsa, rsb);
    }
    wait_vmcnt(2 * kDma + kWDma);
    __syncthreads();
    read_stage(0, std::integral_constant<int, 0>(), std::integral_constant<int, 0>());
    // step 0 sends stage 4 into stage 0's slot: every wave's reads of it
    // must be done (the barrier's fence waits for them)
    __syncthreads();
    // a multiple of 4 steps (whole window groups); the ones past nk run on
    // stages whose data is all zeros and add nothing
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (int kt = 0; kt < nk; kt += kSG) {
      step(kt, I0(), I0());
      step(kt + 1, I1(), I1());
      step(kt + 2, I0(), I2());
      step(kt + 3, I1(), I3());
    }
  }
  // no LDS DMA may still be in flight when the workgroup ends
  wait_vmcnt(0);

  // clipped fp32 epilogue: lane l, accumulator r of block (i, j) is row
  // 8(r/4) + 4(l/32) + r%4, column l%32 of that block
#pragma unroll
  for (int i = 0; i < kSFM; ++i)
#pragma unroll
    for (int j = 0; j < kSFN; ++j) {
      const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < p.M) {
          float v = acc[i][j][r];
          if (p.acc) v += p.acc[row * p.ldacc + col];
          p.C[row * p.ldc + col] = v;
        }
      }
    }
}

// The last N mod 256 <= 8 columns, when the big tiles' last column would
// hold only those: a tile column of 256 for a handful of columns costs a whole
// extra round of workgroups (at N = 8193 the grid is 1056 tiles where 1024
// fill the chip exactly four times).  This kernel reads A once and the R
// remainder rows of Bt: four rows per wave, lanes across K in 16-byte chunks
// (16 fp8 or 32 fp4 values, always within one scale block), values decoded
// to fp32 with their block scale by the gfx950 scaled conversions, fp32 FMAs,
// and one cross-lane sum per output.
constexpr int kSkRows = 4, kSkWaves = 4, kSkMaxR = 8;

__device__ __forceinline__ float e8m0_value(int e) {
  // 2^(e - 127): the bit pattern of a normal float, except e = 0 (2^-127, a
  // subnormal) and e = 255 (NaN)
  return e == 0 ? __uint_as_float(0x00400000u) : e == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float((uint32_t)e << 23);
}

// two values of word half / byte `sel` of dword w, times scale
template <int F>
__device__ __forceinline__ f32x2_s decode2(uint32_t w, float scale, int sel) {
  if constexpr (F == 0)
    return sel ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, false);
  else if constexpr (F == 1)
    return sel ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, true)
               : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, false);
  else
    return sel == 0   ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0)
           : sel == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1)
           : sel == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2)
                      : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3);
}

template <int FA, int FB, int BITS>
__global__ __launch_bounds__(kSkWaves * 64) void gemm_scaled_skinny_kernel(ScaledParams p, int64_t n0, int R) {
  constexpr int VALS = 16 * 8 / BITS;  // values per 16-byte chunk
  constexpr int PAIRS = VALS / 2;      // decode steps per chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = ((int64_t)blockIdx.x * kSkWaves + wave) * kSkRows;
  const uint8_t* sa = (const uint8_t*)p.sa + p.sa_delta;
  const uint8_t* sb = (const uint8_t*)p.sb + p.sb_delta;
  float acc[kSkRows][kSkMaxR];
#pragma unroll
  for (int r = 0; r < kSkRows; ++r)
#pragma unroll
    for (int c = 0; c < kSkMaxR; ++c) acc[r][c] = 0.f;
  bool row_ok[kSkRows];
#pragma unroll
  for (int r = 0; r < kSkRows; ++r) row_ok[r] = m0 + r < p.M;

  for (int64_t k0 = (int64_t)lane * VALS; k0 < p.K; k0 += 64 * VALS) {
    const int64_t kb = k0 >> (5 + p.lg_bq);
    const int64_t byte0 = k0 * BITS / 8;
    u32x4 a[kSkRows];
    float as[kSkRows];
#pragma unroll
    for (int r = 0; r < kSkRows; ++r) {
      const int64_t m = row_ok[r] ? m0 + r : 0;  // rows past M read row 0 and are not written
      a[r] = *(const u32x4*)(p.A + m * p.lda + byte0);
      as[r] = e8m0_value(sa[m * p.lds_a + kb]);
    }
#pragma unroll
    for (int c = 0; c < kSkMaxR; ++c) {
      if (c >= R) break;
      const u32x4 b = *(const u32x4*)(p.B + (n0 + c) * p.ldb + byte0);
      const float bs = e8m0_value(sb[(n0 + c) * p.lds_b + kb]);
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        const int w = BITS == 8 ? q / 2 : q / 4, sel = BITS == 8 ? q % 2 : q % 4;
        const f32x2_s bv = decode2<FB>(b[w], bs, sel);
#pragma unroll
        for (int r = 0; r < kSkRows; ++r) {
          const f32x2_s av = decode2<FA>(a[r][w], as[r], sel);
          acc[r][c] = fmaf(av[0], bv[0], acc[r][c]);
          acc[r][c] = fmaf(av[1], bv[1], acc[r][c]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kSkRows; ++r)
#pragma unroll
    for (int c = 0; c < kSkMaxR; ++c) {
      if (c >= R) break;
      float v = acc[r][c];
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0 && row_ok[r]) {
        const int64_t m = m0 + r, n = n0 + c;
        if (p.acc) v += p.acc[m * p.ldacc + n];
        p.C[m * p.ldc + n] = v;
      }
    }
}


// main kernel on the first p.N columns; the skinny kernel on columns
// n_skinny .. n_skinny + r_skinny - 1 (r_skinny = 0: none)
template <int FA, int FB, int BITS>
int launch_scaled(const ScaledParams& p, bool packed, int64_t n_wg, int64_t n_skinny, int r_skinny, hipStream_t s) {
  if (n_wg > 0) {
    if (packed)
      launch_kernel("gemm_scaled/main", gemm_scaled_kernel<FA, FB, BITS, true>, dim3((unsigned)n_wg), dim3(kSNT),
                    (uint32_t)kScaledLds, s, p);
    else
      launch_kernel("gemm_scaled/main", gemm_scaled_kernel<FA, FB, BITS, false>, dim3((unsigned)n_wg), dim3(kSNT),
                    (uint32_t)kScaledLds, s, p);
    if (int rc = check_launch("gemm_scaled/main")) return rc;
  }
  if (r_skinny > 0) {
    const int64_t wg = (p.M + kSkRows * kSkWaves - 1) / (kSkRows * kSkWaves);
    launch_kernel("gemm_scaled/skinny", gemm_scaled_skinny_kernel<FA, FB, BITS>, dim3((unsigned)wg),
                  dim3(kSkWaves * 64), 0u, s, p, n_skinny, r_skinny);
    return check_launch("gemm_scaled/skinny");
  }
  return STG_OK;
}

template <int FA, int FB, int BITS>
bool set_lds() {
  return hipFuncSetAttribute((const void*)gemm_scaled_kernel<FA, FB, BITS, false>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, kScaledLds) == hipSuccess &&
         hipFuncSetAttribute((const void*)gemm_scaled_kernel<FA, FB, BITS, true>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, kScaledLds) == hipSuccess;
}

}  // namespace
}  // namespace stg

using namespace stg;

namespace {

// the scaled MFMA takes e8m0 scales per 32 K values of two operands of one
// width; every other case goes to the general path
bool scaled_mfma_path(int32_t a_fmt, int32_t b_fmt, int32_t scale_fmt, int64_t block) {
  const int bits = a_fmt == STG_LP_E2M1 ? 4 : 8, bits_b = b_fmt == STG_LP_E2M1 ? 4 : 8;
  return scale_fmt == STG_SC_E8M0 && block >= 32 && (block & (block - 1)) == 0 && bits == bits_b;
}

int scaled_impl(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a, const void* Bt,
                int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b, int32_t scale_fmt, int64_t block,
                const float* acc, int64_t ldacc, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                void* workspace, int64_t workspace_bytes, void* stream) {
  const char* name = "gemm_scaled";
  auto known = [](int32_t f) { return f == STG_LP_E4M3 || f == STG_LP_E5M2 || f == STG_LP_E2M1; };
  if (!known(a_fmt) || !known(b_fmt)) return fail(STG_ERR_UNSUPPORTED, "%s: unknown operand format", name);
  if (scale_fmt != STG_SC_E8M0 && scale_fmt != STG_SC_E4M3)
    return fail(STG_ERR_UNSUPPORTED, "%s: unknown scale format", name);
  if (M < 0 || N < 0 || K < 0) return fail(STG_ERR_INVALID, "%s: negative size", name);
  if (block < 1) return fail(STG_ERR_INVALID, "%s: block must be >= 1", name);
  if (K % block) return fail(STG_ERR_INVALID, "%s: K %lld is not a multiple of the block %lld", name, (long long)K,
                             (long long)block);
  const int bits = a_fmt == STG_LP_E2M1 ? 4 : 8, bits_b = b_fmt == STG_LP_E2M1 ? 4 : 8;
  if (lda < (K * bits + 7) / 8 || ldb < (K * bits_b + 7) / 8 || lds_a < K / block || lds_b < K / block || ldc < N ||
      (acc && ldacc < N))
    return fail(STG_ERR_INVALID, "%s: row strides must cover the rows", name);
  if (M == 0 || N == 0) return STG_OK;
  if (!C || (K > 0 && (!A || !Bt || !a_scale || !b_scale))) return fail(STG_ERR_INVALID, "%s: null operand", name);
  if (!scaled_mfma_path(a_fmt, b_fmt, scale_fmt, block))
    return gemm_scaled_general(A, a_fmt, lda, a_scale, lds_a, Bt, b_fmt, ldb, b_scale, lds_b, scale_fmt, block, acc,
                               ldacc, C, ldc, M, N, K, workspace, workspace_bytes, as_stream(stream));
  if ((int64_t)kSBM * lda + 256 >= kMaxOffset32 || (int64_t)kSBN * ldb + 256 >= kMaxOffset32 ||
      M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2 ||
      (M - 1) * lds_a + K / block + 64 >= kMaxOffset32 || (N - 1) * lds_b + K / block + 64 >= kMaxOffset32)
    return fail(STG_ERR_RANGE, "%s: a stage or a scale matrix spans more than 2^31 bytes, or a size is too large",
                name);
  // once on each device
  static OncePerDevice once;
  const bool lds_ok = once.run([] {
    return set_lds<0, 0, 8>() && set_lds<0, 1, 8>() && set_lds<1, 0, 8>() && set_lds<1, 1, 8>() &&
           set_lds<4, 4, 4>();
  });
  if (!lds_ok) return fail(STG_ERR_LAUNCH, "%s: cannot reserve LDS for the scaled GEMM kernels", name);
  ScaledParams p{};
  p.A = (const char*)A;
  p.B = (const char*)Bt;
  // scale windows are read as aligned 16-byte chunks from 16-byte aligned
  // bases; the readable extent is rounded up to whole chunks (an aligned
  // chunk never crosses a page, so the bytes beyond the matrix it holds are
  // mapped)
  const uintptr_t ua = (uintptr_t)a_scale, ub = (uintptr_t)b_scale;
  p.sa = (const char*)(ua & ~(uintptr_t)15);
  p.sb = (const char*)(ub & ~(uintptr_t)15);
  p.sa_delta = (int32_t)(ua & 15);
  p.sb_delta = (int32_t)(ub & 15);
  p.sa_bytes = K > 0 ? (p.sa_delta + (M - 1) * lds_a + K / block + 15) & ~(int64_t)15 : 0;
  p.sb_bytes = K > 0 ? (p.sb_delta + (N - 1) * lds_b + K / block + 15) & ~(int64_t)15 : 0;
  p.acc = acc;
  p.C = C;
  p.lda = lda, p.ldb = ldb, p.lds_a = lds_a, p.lds_b = lds_b, p.ldacc = ldacc, p.ldc = ldc;
  p.M = M, p.N = N, p.K = K;
  p.lg_bq = 0;
  while ((int64_t)32 << p.lg_bq < block) ++p.lg_bq;
  p.nkb = (int32_t)(K / block);
  // a remainder of at most 8 columns past the last whole tile column goes to
  // the skinny kernel; the main kernel then sees N rounded down
  const int r_skinny = N % kSBN <= kSkMaxR ? (int)(N % kSBN) : 0;
  p.N = N - r_skinny;
  p.tiles_m = (int32_t)((M + kSBM - 1) / kSBM);
  p.tiles_n = (int32_t)((p.N + kSBN - 1) / kSBN);
  const int64_t n_wg = (int64_t)p.tiles_m * p.tiles_n;
  const hipStream_t s = as_stream(stream);
  const int code_a = a_fmt == STG_LP_E4M3 ? 0 : a_fmt == STG_LP_E5M2 ? 1 : 4;
  const int code_b = b_fmt == STG_LP_E4M3 ? 0 : b_fmt == STG_LP_E5M2 ? 1 : 4;
  const int64_t n_sk = p.N;
  // packed-scale path: 32-value blocks, every scale row starting 16-byte aligned
  const bool packed = p.lg_bq == 0 && p.sa_delta == 0 && p.sb_delta == 0 && lds_a % 16 == 0 && lds_b % 16 == 0;
  if (bits == 4) return launch_scaled<4, 4, 4>(p, packed, n_wg, n_sk, r_skinny, s);
  if (code_a == 0 && code_b == 0) return launch_scaled<0, 0, 8>(p, packed, n_wg, n_sk, r_skinny, s);
  if (code_a == 0) return launch_scaled<0, 1, 8>(p, packed, n_wg, n_sk, r_skinny, s);
  if (code_b == 0) return launch_scaled<1, 0, 8>(p, packed, n_wg, n_sk, r_skinny, s);
  return launch_scaled<1, 1, 8>(p, packed, n_wg, n_sk, r_skinny, s);
}

}  // namespace

extern "C" int gemm_scaled(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                           const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                           int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  clear_error();
  return scaled_impl(A, a_fmt, lda, a_scale, lds_a, Bt, b_fmt, ldb, b_scale, lds_b, scale_fmt, block, acc, ldacc, C,
                     ldc, M, N, K, nullptr, 0, stream);
}

extern "C" int gemm_scaled_ws(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                              const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                              int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  clear_error();
  if (workspace_bytes < 0) return fail(STG_ERR_INVALID, "gemm_scaled_ws: negative workspace_bytes");
  return scaled_impl(A, a_fmt, lda, a_scale, lds_a, Bt, b_fmt, ldb, b_scale, lds_b, scale_fmt, block, acc, ldacc, C,
                     ldc, M, N, K, workspace, workspace ? workspace_bytes : 0, stream);
}

extern "C" int64_t gemm_scaled_workspace(int32_t a_fmt, int32_t b_fmt, int32_t scale_fmt, int64_t block, int64_t M,
                                         int64_t N, int64_t K) {
  clear_error();
  const char* name = "gemm_scaled_workspace";
  auto known = [](int32_t f) { return f == STG_LP_E4M3 || f == STG_LP_E5M2 || f == STG_LP_E2M1; };
  if (!known(a_fmt) || !known(b_fmt) || (scale_fmt != STG_SC_E8M0 && scale_fmt != STG_SC_E4M3))
    return -fail(STG_ERR_UNSUPPORTED, "%s: unknown operand or scale format", name);
  if (M < 0 || N < 0 || K < 0 || block < 1 || K % block)
    return -fail(STG_ERR_INVALID, "%s: negative size, or K not a multiple of the block", name);
  if (scaled_mfma_path(a_fmt, b_fmt, scale_fmt, block)) return 0;
  return gemm_scaled_general_workspace(M, N, K);
}
