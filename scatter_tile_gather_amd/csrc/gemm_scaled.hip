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
// the 16-byte chunks 2p + l / 32 (p = 0, 1) of the step's 64-byte K run: K
// values 32 p + 16 (l / 32) .. +15 of fp8, 32 p + 16 (l / 32) .. of fp4 at
// twice the density.  The accumulator layout is the 32x32 MFMA layout.
//  * Tiles 256 x 256, 8 waves of 128 x 64 accumulators (two waves per SIMD).
//  * Both operands are staged by LDS DMA into 64-byte rows -- 64 fp8 or 128
//    fp4 K values per stage -- with the conflict-free chunk swizzle of the bf16
//    GEMM, out-of-range rows and K chunks landing as zeros; a 4-stage ring,
//    the DMA of stage k+3 spread among stage k's MFMAs.
//  * Each lane loads its scale bytes LA stages ahead (fp8: 2, fp4: 1 -- an fp4
//    step has twice the MFMAs, and twice the scale bytes) into one of LA + 1
//    register sets (the K loop is unrolled by LA + 1 so the set is known at
//    compile time).  Vector-memory operations complete in issue order, so the
//    compiler's own wait before a set's first use only forces DMA issued LA
//    steps earlier, and the explicit wait at the end of step k (allowing the
//    operations issued after stage k+1's scales to stay in flight) covers
//    stage k+1's data and scales.  Every step issues its DMA; past the end of K the
//    offsets fall outside the descriptor and the DMA writes zeros into ring
//    slots nothing reads any more.
//  * Clipped fp32 epilogue adding the optional accumulator input.
#include "gemm_common.h"

#include <type_traits>

namespace stg {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16_s __attribute__((ext_vector_type(16)));

struct ScaledParams {
  const char* A;  // (M, K), row stride lda bytes
  const char* B;  // Bt (N, K), row stride ldb bytes
  const uint8_t* sa;  // e8m0 (M, K / block), row stride lds_a
  const uint8_t* sb;  // e8m0 (N, K / block), row stride lds_b
  const float* acc;   // (M, N) f32, row stride ldacc, or null
  float* C;           // (M, N) f32, row stride ldc
  int64_t lda, ldb, lds_a, lds_b, ldacc, ldc;
  int64_t M, N, K;
  int32_t bq;   // block / 32
  int32_t nkb;  // K / block
  int32_t tiles_m, tiles_n;
};

constexpr int kSBM = 256, kSBN = 256, kSWN = 4, kSNW = 8, kSNT = kSNW * 64;
constexpr int kSFM = 4, kSFN = 2;  // 32x32 blocks per wave: 128 x 64
constexpr int kSNS = 4;            // ring depth
constexpr int kRowB = 64;          // bytes per operand row per stage
constexpr int kAStage = kSBM * kRowB, kBStage = kSBN * kRowB, kStage = kAStage + kBStage;
constexpr int kADma = kAStage / 1024 / kSNW, kBDma = kBStage / 1024 / kSNW, kDma = kADma + kBDma;
constexpr int kScaledLds = kSNS * kStage;  // 128 KiB

// FA / FB: operand format codes of the scaled MFMA (0 e4m3, 1 e5m2, 4 e2m1);
// BITS: 8 for fp8 operands, 4 for fp4 (both operands of one width)
template <int FA, int FB, int BITS>
__global__ __launch_bounds__(kSNT) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_scaled_kernel(
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

  // DMA chunks of this lane (row r of the stage, logical chunk c): offsets are
  // the same for every stage (the descriptors move with K)
  uint32_t a_off[kADma], b_off[kBDma];
  int a_kc[kADma], b_kc[kBDma];
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
  const uint32_t smem_lds =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem);

  auto stage_rsrc = [&](int kt, u32x4_s& rsa, u32x4_s& rsb) {
    const int64_t kb = (int64_t)kt * kRowB;  // byte offset of the stage in a row
    rsa = rsrc_words(p.A + m0 * p.lda + kb, (p.M - 1 - m0) * p.lda + (row_bytes - kb));
    rsb = rsrc_words(p.B + n0 * p.ldb + kb, (p.N - 1 - n0) * p.ldb + (row_bytes - kb));
  };
  // DMA instruction q (A first, then B) of stage kt; chunks at or past K land as zeros
  auto dma_one = [&](int kt, int q, const u32x4_s& rsa, const u32x4_s& rsb) {
    const uint32_t st = smem_lds + (kt % kSNS) * kStage;
    const int64_t kleft = p.K - (int64_t)kt * KS;
    if (q < kADma) {
      dma16(rsa, a_kc[q] < kleft ? a_off[q] : kOOB, st + (wave * kADma + q) * 1024);
    } else {
      const int qb = q - kADma;
      dma16(rsb, b_kc[qb] < kleft ? b_off[qb] : kOOB, st + kAStage + (wave * kBDma + qb) * 1024);
    }
  };

  // scale bytes of stage kt for this lane's rows (A) and columns (B), into
  // register set SLOT (a compile-time constant); indices past the matrix or
  // past K are clamped (their data is zero)
  constexpr int NSL = (kSFM + kSFN) * S;  // scale loads per stage
  constexpr int LA = BITS == 8 ? 2 : 1;   // scales are loaded LA stages ahead
  constexpr int NSET = LA + 1;            // register sets of scales
  // operations issued after stage k+1's scales by the end of step k, in order:
  // LA = 2: DMA(k+2), scales(k+2), DMA(k+3); LA = 1: DMA(k+3)
  constexpr int IN_FLIGHT = LA == 2 ? 2 * kDma + NSL : kDma;
  int sc_a[NSET][kSFM][S], sc_b[NSET][kSFN][S];
  auto load_scales = [&](int kt, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t k32 = (uint32_t)kt * (KS / 32) + 2 * s + half;  // 32-value block of K
      int64_t kb = k32 / (uint32_t)p.bq;
      kb = kb < p.nkb ? kb : p.nkb - 1;
#pragma unroll
      for (int i = 0; i < kSFM; ++i) {
        int64_t r = m0 + wm * 128 + i * 32 + (lane & 31);
        r = r < p.M ? r : p.M - 1;
        sc_a[SLOT][i][s] = p.sa[r * p.lds_a + kb];
      }
#pragma unroll
      for (int j = 0; j < kSFN; ++j) {
        int64_t r = n0 + wn * 64 + j * 32 + (lane & 31);
        r = r < p.N ? r : p.N - 1;
        sc_b[SLOT][j][s] = p.sb[r * p.lds_b + kb];
      }
    }
  };

  // operand chunks 2h + half (h = 0, 1) of stage kt: fp8 -- the lane's two
  // 16-byte pieces of the one MFMA step (scale blocks 0 and 1 of the step);
  // fp4 -- the lane's 16 bytes of MFMA step h
  u32x4 fa[kSFM][2], fb[kSFN][2];
  auto read_frags = [&](int kt) {
    const char* as = smem + (kt % kSNS) * kStage;
    const char* bs = as + kAStage;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * h + half;
#pragma unroll
      for (int i = 0; i < kSFM; ++i) {
        const int r = (wave / kSWN) * 128 + i * 32 + (lane & 31);
        fa[i][h] = *(const u32x4*)(as + r * kRowB + (a_phys(r, c) << 4));
      }
#pragma unroll
      for (int j = 0; j < kSFN; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        fb[j][h] = *(const u32x4*)(bs + r * kRowB + (a_phys(r, c) << 4));
      }
    }
  };

  // the MFMAs of one stage (scales from buffer SLOT) with the DMA
  // instructions of stage kd spread among them
  auto mfmas_dma = [&](auto slot_tag, int kd, int nq, const u32x4_s& rsa, const u32x4_s& rsb) {
    constexpr int slot = decltype(slot_tag)::value;
    constexpr int NM = kSFM * kSFN * S;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < kSFM; ++i)
#pragma unroll
        for (int j = 0; j < kSFN; ++j) {
          i32x8 av, bv;
          if (BITS == 8) {
            av = (i32x8){(int)fa[i][0][0], (int)fa[i][0][1], (int)fa[i][0][2], (int)fa[i][0][3],
                         (int)fa[i][1][0], (int)fa[i][1][1], (int)fa[i][1][2], (int)fa[i][1][3]};
            bv = (i32x8){(int)fb[j][0][0], (int)fb[j][0][1], (int)fb[j][0][2], (int)fb[j][0][3],
                         (int)fb[j][1][0], (int)fb[j][1][1], (int)fb[j][1][2], (int)fb[j][1][3]};
          } else {
            av = (i32x8){(int)fa[i][s][0], (int)fa[i][s][1], (int)fa[i][s][2], (int)fa[i][s][3], 0, 0, 0, 0};
            bv = (i32x8){(int)fb[j][s][0], (int)fb[j][s][1], (int)fb[j][s][2], (int)fb[j][s][3], 0, 0, 0, 0};
          }
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], FA, FB, 0, sc_a[slot][i][s],
                                                                      0, sc_b[slot][j][s]);
          const int m = (s * kSFM + i) * kSFN + j;
#pragma unroll
          for (int d = 0; d < nq; ++d) {
            const int after = ((d + 1) * NM) / nq - 1;
            if ((after < 0 ? 0 : after) == m) {
              __builtin_amdgcn_sched_barrier(0);
              dma_one(kd, d, rsa, rsb);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
  };

  // one K step on stage kt, whose scales are in register set SLOT = kt % 3:
  // issue stage kt+2's scales and stage kt+3's DMA (zeros past K) while stage
  // kt feeds the MFMAs
  auto step = [&](int kt, auto slot_tag) {
    constexpr int SLOT = decltype(slot_tag)::value;
    u32x4_s rsa, rsb;
    load_scales(kt + LA, std::integral_constant<int, (SLOT + LA) % NSET>());
    stage_rsrc(kt + kSNS - 1, rsa, rsb);
    read_frags(kt);
    mfmas_dma(slot_tag, kt + kSNS - 1, kDma, rsa, rsb);
    // stage kt+1 and its scales have landed once only what was issued after
    // those scales is still in flight (operations complete in order)
    wait_vmcnt(IN_FLIGHT);
    // publishes stage kt + 1; ring slot kt % NS is free after this
    __syncthreads();
  };

  // prologue, in the steady state's issue order (a step issues the scales
  // LA stages ahead, then the DMA three stages ahead):
  //   LA = 2: DMA(0), scales(0), DMA(1), scales(1), DMA(2)
  //   LA = 1: DMA(0), DMA(1), scales(0), DMA(2)
  // (K = 0 has no stage and no scale: the epilogue writes acc or zeros)
  if (nk > 0) {
    for (int s = 0; s < kSNS - 1; ++s) {
      u32x4_s rsa, rsb;
      if (LA == 1 && s == 2) load_scales(0, std::integral_constant<int, 0>());
      stage_rsrc(s, rsa, rsb);
#pragma unroll
      for (int q = 0; q < kDma; ++q) dma_one(s, q, rsa, rsb);
      if (LA == 2 && s == 0) load_scales(0, std::integral_constant<int, 0>());
      if (LA == 2 && s == 1) load_scales(1, std::integral_constant<int, 1 % NSET>());
    }
    wait_vmcnt(IN_FLIGHT);
    __syncthreads();
    int kt = 0;
    if constexpr (NSET == 3) {
      for (; kt + 2 < nk; kt += 3) {
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
        step(kt + 2, std::integral_constant<int, 2>());
      }
      if (kt < nk) step(kt, std::integral_constant<int, 0>());
      if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>());
    } else {
      for (; kt + 1 < nk; kt += 2) {
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
      }
      if (kt < nk) step(kt, std::integral_constant<int, 0>());
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
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
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

bool scaled_lds_configured = false;

template <int FA, int FB, int BITS>
int launch_scaled(const ScaledParams& p, int64_t n_wg, hipStream_t s) {
  auto k = gemm_scaled_kernel<FA, FB, BITS>;
  launch_kernel("gemm_scaled", k, dim3((unsigned)n_wg), dim3(kSNT), (uint32_t)kScaledLds, s, p);
  return check_launch("gemm_scaled");
}

template <int FA, int FB, int BITS>
bool set_lds() {
  return hipFuncSetAttribute((const void*)gemm_scaled_kernel<FA, FB, BITS>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, kScaledLds) == hipSuccess;
}

}  // namespace
}  // namespace stg

using namespace stg;

extern "C" int gemm_scaled(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                           const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                           int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, void* stream) {
  clear_error();
  const char* name = "gemm_scaled";
  auto known = [](int32_t f) { return f == STG_LP_E4M3 || f == STG_LP_E5M2 || f == STG_LP_E2M1; };
  if (!known(a_fmt) || !known(b_fmt)) return fail(STG_ERR_UNSUPPORTED, "%s: unknown operand format", name);
  if ((a_fmt == STG_LP_E2M1) != (b_fmt == STG_LP_E2M1))
    return fail(STG_ERR_UNSUPPORTED, "%s: fp4 operands pair only with fp4 operands here", name);
  if (scale_fmt != STG_SC_E8M0 && scale_fmt != STG_SC_E4M3)
    return fail(STG_ERR_UNSUPPORTED, "%s: unknown scale format", name);
  if (scale_fmt == STG_SC_E4M3)
    return fail(STG_ERR_UNSUPPORTED, "%s: e4m3 scales are not powers of two; the scaled MFMA takes e8m0 only", name);
  if (M < 0 || N < 0 || K < 0) return fail(STG_ERR_INVALID, "%s: negative size", name);
  if (block < 32 || block % 32) return fail(STG_ERR_UNSUPPORTED, "%s: block must be a positive multiple of 32", name);
  if (K % block) return fail(STG_ERR_INVALID, "%s: K %lld is not a multiple of the block %lld", name, (long long)K,
                             (long long)block);
  const int bits = a_fmt == STG_LP_E2M1 ? 4 : 8;
  const int64_t row_bytes = K * bits / 8;
  if (lda < row_bytes || ldb < row_bytes || lds_a < K / block || lds_b < K / block || ldc < N ||
      (acc && ldacc < N))
    return fail(STG_ERR_INVALID, "%s: row strides must cover the rows", name);
  if (M == 0 || N == 0) return STG_OK;
  if (!C || (K > 0 && (!A || !Bt || !a_scale || !b_scale))) return fail(STG_ERR_INVALID, "%s: null operand", name);
  if ((int64_t)kSBM * lda + 256 >= kMaxOffset32 || (int64_t)kSBN * ldb + 256 >= kMaxOffset32 ||
      M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2)
    return fail(STG_ERR_RANGE, "%s: a stage spans more than 2^31 bytes or a size is too large", name);
  if (!scaled_lds_configured) {
    if (!set_lds<0, 0, 8>() || !set_lds<0, 1, 8>() || !set_lds<1, 0, 8>() || !set_lds<1, 1, 8>() ||
        !set_lds<4, 4, 4>())
      return fail(STG_ERR_LAUNCH, "%s: cannot reserve LDS: %s", name, hipGetErrorString(hipGetLastError()));
    scaled_lds_configured = true;
  }
  ScaledParams p{};
  p.A = (const char*)A;
  p.B = (const char*)Bt;
  p.sa = (const uint8_t*)a_scale;
  p.sb = (const uint8_t*)b_scale;
  p.acc = acc;
  p.C = C;
  p.lda = lda, p.ldb = ldb, p.lds_a = lds_a, p.lds_b = lds_b, p.ldacc = ldacc, p.ldc = ldc;
  p.M = M, p.N = N, p.K = K;
  p.bq = (int32_t)(block / 32);
  p.nkb = (int32_t)(K / block);
  p.tiles_m = (int32_t)((M + kSBM - 1) / kSBM);
  p.tiles_n = (int32_t)((N + kSBN - 1) / kSBN);
  const int64_t n_wg = (int64_t)p.tiles_m * p.tiles_n;
  const hipStream_t s = as_stream(stream);
  const int code_a = a_fmt == STG_LP_E4M3 ? 0 : a_fmt == STG_LP_E5M2 ? 1 : 4;
  const int code_b = b_fmt == STG_LP_E4M3 ? 0 : b_fmt == STG_LP_E5M2 ? 1 : 4;
  if (bits == 4) return launch_scaled<4, 4, 4>(p, n_wg, s);
  if (code_a == 0 && code_b == 0) return launch_scaled<0, 0, 8>(p, n_wg, s);
  if (code_a == 0) return launch_scaled<0, 1, 8>(p, n_wg, s);
  if (code_b == 0) return launch_scaled<1, 0, 8>(p, n_wg, s);
  return launch_scaled<1, 1, 8>(p, n_wg, s);
}
