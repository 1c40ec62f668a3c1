// Block-scaled GEMM, general path: any operand pair, e8m0 or e4m3 scales,
// any scale block that divides K.
//
// Semantics (cuTile.jl Operations, muladd_scaled: (a . a_scale)(b . b_scale)
// + acc, each scale element multiplying a contiguous block of K / K_s values
// along K of its operand; a and b in f8e4m3fn, f8e5m2 or f4e2m1fn, scales in
// f8e8m0fnu or f8e4m3fn, an f32 accumulator; reinterpret: FP4 travels two
// values per byte).  Layout as on the scaled-MFMA path: A (M, K) and B given
// K-major as Bt (N, K), element k of an FP4 row at byte k / 2, the even
// element in the low nibble; scales (M, K / block) and (N, K / block).
//
// gfx950's scaled MFMA applies one e8m0 scale per 32 K values of both
// operands of one width, so it computes this product only for e8m0 scales,
// blocks of 32 times a power of two and fp8 x fp8 or fp4 x fp4.  Everything
// else runs here: each value is multiplied by its scale while the operands
// are staged, and the scaled values go through the bf16 MFMA with fp32
// accumulation.  The scaling is exact: an operand value has at most 4
// significant bits (e4m3: 4, e5m2: 3, e2m1: 2) and a scale at most 4 (e4m3)
// or 1 (e8m0), so value x scale has at most 8 and is a bf16 number whenever
// its exponent lies in bf16's range -- always with e4m3 scales (the products
// lie in [2^-18, 2^25]); with e8m0 scales whenever 2^(e-127) times the
// operand value neither overflows nor falls below 2^-133.  The bf16 products
// of two such values are exact in fp32, so the result differs from the exact
// sum only by fp32 accumulation rounding.
//
//  * Tiles 256 x 256 on 8 waves (2 x 4), each wave 128 x 64 accumulators of
//    v_mfma_f32_32x32x16_bf16; K steps of 32.
//  * Staging: each lane owns 16 consecutive K values of one row of A and of
//    one row of Bt per step.  It loads their codes with one buffer load (16
//    bytes of fp8, 8 of fp4) through a range-checked buffer resource (rows
//    past M or N and bytes past the matrix read as zero codes), finds each
//    value's scale byte, decodes code and scale from their bit fields,
//    multiplies, rounds to bf16 (exact, above) and writes the 16 bf16 values
//    to an LDS stage of 64-byte rows with the bf16 GEMM's conflict-free chunk
//    swizzle; values at K and beyond are written as zero.  Both operands are
//    K-contiguous rows, so both MFMA operands are plain ds_read_b128 reads.
//  * Two LDS stages: the codes of step k+1 are loaded before step k's MFMAs
//    and decoded into the other stage after them; one barrier per step.
//  * Clipped fp32 epilogue adding the optional accumulator input.
#include "gemm_common.h"

namespace stg {
namespace {

typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef float f32x16_g __attribute__((ext_vector_type(16)));

constexpr int kGBM = 256, kGBN = 256, kGBK = 32;
constexpr int kGWM = 2, kGWN = 4, kGNT = kGWM * kGWN * 64;
constexpr int kGFM = kGBM / kGWM / 32, kGFN = kGBN / kGWN / 32;  // 4 x 2 blocks of 32 x 32 per wave
constexpr int kGStage = (kGBM + kGBN) * kGBK * 2;                 // 32 KiB: A rows then B rows, 64 bytes each

struct GeneralParams {
  const char* A;
  const char* B;
  const char* sa;
  const char* sb;
  const float* acc;
  float* C;
  int64_t lda, ldb, lds_a, lds_b, ldacc, ldc;
  int64_t M, N, K;
  int32_t fa, fb, sf;  // operand formats (stg_lowp_format), scale format (stg_scale_format)
  int32_t block;
  int32_t tiles_m, tiles_n;
};

// Value of an operand code (cuTile.jl Operations: the f8e4m3fn, f8e5m2 and
// f4e2m1fn formats; e4m3fn has no infinities and S.1111.111 is NaN; e5m2 is
// the top byte of an IEEE binary16; e2m1 has values {0, 0.5, 1, 1.5, 2, 3, 4,
// 6} and a sign), built from its bit fields.
__device__ __forceinline__ float decode_code(uint32_t c, int fmt) {
  if (fmt == STG_LP_E2M1) {
    const uint32_t e = (c >> 1) & 3, m = c & 1;
    const float mag = e == 0 ? 0.5f * (float)m : (float)(2 + m) * (float)(1 << e) * 0.25f;
    return (c & 8) ? -mag : mag;
  }
  if (fmt == STG_LP_E5M2) {
    const uint32_t e = (c >> 2) & 31, m = c & 3, s = (c >> 7) << 31;
    if (e == 31) return __uint_as_float(s | 0x7F800000u | (m << 21));  // infinities and NaNs
    if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0x1p-16f));
    return __uint_as_float(s | ((e + 112) << 23) | (m << 21));
  }
  // e4m3fn
  const uint32_t e = (c >> 3) & 15, m = c & 7, s = (c >> 7) << 31;
  if (e == 15 && m == 7) return __uint_as_float(0x7FC00000u);
  if (e == 0) return __uint_as_float(s | __float_as_uint((float)m * 0x1p-9f));
  return __uint_as_float(s | ((e + 120) << 23) | (m << 20));
}

// Value of a scale byte: e8m0 is 2^(b - 127) (0xFF is NaN; b = 0 is the fp32
// subnormal 2^-127); e4m3 as an operand code.
__device__ __forceinline__ float decode_scale(uint32_t b, int sf) {
  if (sf == STG_SC_E4M3) return decode_code(b, STG_LP_E4M3);
  if (b == 0xFF) return __uint_as_float(0x7FC00000u);
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Codes of one lane's 16 K values of one row: 16 bytes (fp8) or 8 (fp4).
struct Codes {
  u32x4 w;
  uint32_t s0, s1;  // scale bytes of the first and the last of the 16 values (blocks of 16 or more)
};

__global__ __launch_bounds__(kGNT) void gemm_scaled_general_kernel(GeneralParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kGWN, wn = wave % kGWN;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kGBM, n0 = (int64_t)tn * kGBN;
  const int nk = (int)((p.K + kGBK - 1) / kGBK);

  // this lane's staging rows: row r of the A tile and of the Bt tile, K
  // values 16h .. 16h+15 of each step
  const int r = tid >> 1, h = tid & 1;
  const int bits_a = p.fa == STG_LP_E2M1 ? 4 : 8, bits_b = p.fb == STG_LP_E2M1 ? 4 : 8;
  const int64_t ra = m0 + r, rb = n0 + r;
  // buffer resources over each operand's rows of this tile (zero past the
  // matrix) and over the scale matrices
  auto rsrc_rows = [](const char* base, int64_t row0, int64_t rows, int64_t ld, int64_t row_bytes) {
    const int64_t avail = rows > row0 ? (rows - 1 - row0) * ld + row_bytes : 0;
    return make_rsrc(base + (rows > row0 ? row0 * ld : 0), (uint32_t)(avail < (int64_t)kOOB ? avail : kOOB - 1));
  };
  const int64_t rba = (p.K * bits_a + 7) / 8, rbb = (p.K * bits_b + 7) / 8;
  const int64_t nkb = p.K / p.block;
  const __amdgpu_buffer_rsrc_t rs_a = rsrc_rows(p.A, m0, p.M, p.lda, rba);
  const __amdgpu_buffer_rsrc_t rs_b = rsrc_rows(p.B, n0, p.N, p.ldb, rbb);
  const __amdgpu_buffer_rsrc_t rs_sa = rsrc_rows(p.sa, m0, p.M, p.lds_a, nkb);
  const __amdgpu_buffer_rsrc_t rs_sb = rsrc_rows(p.sb, n0, p.N, p.lds_b, nkb);
  const bool in_a = ra < p.M, in_b = rb < p.N;
  const uint32_t row_a = in_a ? (uint32_t)(r * p.lda) : kOOB, row_b = in_b ? (uint32_t)(r * p.ldb) : kOOB;
  const uint32_t srow_a = in_a ? (uint32_t)(r * p.lds_a) : kOOB, srow_b = in_b ? (uint32_t)(r * p.lds_b) : kOOB;
  const bool blk16 = p.block % 16 == 0;  // the 16 values of a lane share one scale

  auto load_codes = [&](int kt, const __amdgpu_buffer_rsrc_t& rs, uint32_t row_off, int bits,
                        const __amdgpu_buffer_rsrc_t& rss, uint32_t srow) {
    Codes c;
    const int64_t k = (int64_t)kt * kGBK + 16 * h;
    const uint32_t off = row_off == kOOB ? kOOB : row_off + (uint32_t)(k * bits / 8);
    c.w = (u32x4){0, 0, 0, 0};
    if (k + 16 <= p.K) {
      if (bits == 8) {
        c.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
        c.w = (u32x4){v[0], v[1], 0, 0};
      }
    } else if (k < p.K && row_off != kOOB) {
      // the row ends inside these 16 values: byte loads up to the row's last
      // byte, so no load reaches past the matrix
      const int nb = (int)(((p.K - k) * bits + 7) / 8);
#pragma unroll
      for (int b = 0; b < 16; ++b)
        if (b < nb) c.w[b >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, off + b, 0, 0) << (8 * (b & 3));
    }
    c.s0 = c.s1 = 0;
    if (blk16 && k < p.K && srow != kOOB)
      c.s0 = c.s1 = __builtin_amdgcn_raw_buffer_load_b8(rss, srow + (uint32_t)k / (uint32_t)p.block, 0, 0);
    return c;
  };
  // scaled bf16 values of one lane's 16 K values into LDS row `row` of the
  // operand region at `region` (zero at K and beyond)
  auto decode_store = [&](int kt, const Codes& c, int fmt, int bits, const __amdgpu_buffer_rsrc_t& rss,
                          uint32_t srow, char* region) {
    const int64_t k0 = (int64_t)kt * kGBK + 16 * h;
    u32x4 out[2];
    float sc = decode_scale(c.s0, p.sf);
    int64_t sidx = -1, next = 0;  // general blocks: scale index of the current value, first K of the next block
    if (!blk16 && k0 < p.K) {
      sidx = (uint32_t)k0 / (uint32_t)p.block;
      next = (sidx + 1) * p.block;
      sc = decode_scale(srow == kOOB ? 0u : __builtin_amdgcn_raw_buffer_load_b8(rss, srow + (uint32_t)sidx, 0, 0),
                        p.sf);
    }
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      float v[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ee = e + u;
        const uint32_t code = bits == 8 ? (c.w[ee >> 2] >> (8 * (ee & 3))) & 0xFF : (c.w[ee >> 3] >> (4 * (ee & 7))) & 0xF;
        const int64_t k = k0 + ee;
        if (!blk16 && k < p.K && k >= next) {  // k == next: the next block starts here
          sidx += 1;
          next += p.block;
          sc = decode_scale(srow == kOOB ? 0u : __builtin_amdgcn_raw_buffer_load_b8(rss, srow + (uint32_t)sidx, 0, 0),
                            p.sf);
        }
        v[u] = k < p.K ? decode_code(code, fmt) * sc : 0.f;
      }
      const __bf16 b0 = (__bf16)v[0], b1 = (__bf16)v[1];
      out[e >> 3][(e >> 1) & 3] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
    }
    *(u32x4*)(region + r * 64 + (a_phys(r, 2 * h) << 4)) = out[0];
    *(u32x4*)(region + r * 64 + (a_phys(r, 2 * h + 1) << 4)) = out[1];
  };

  f32x16_g acc[kGFM][kGFN];
#pragma unroll
  for (int i = 0; i < kGFM; ++i)
#pragma unroll
    for (int j = 0; j < kGFN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  auto stage_a = [&](int kt) { return smem + (kt & 1) * kGStage; };
  auto stage_b = [&](int kt) { return smem + (kt & 1) * kGStage + kGBM * 64; };

  if (nk > 0) {
    const Codes ca = load_codes(0, rs_a, row_a, bits_a, rs_sa, srow_a);
    const Codes cb = load_codes(0, rs_b, row_b, bits_b, rs_sb, srow_b);
    decode_store(0, ca, p.fa, bits_a, rs_sa, srow_a, stage_a(0));
    decode_store(0, cb, p.fb, bits_b, rs_sb, srow_b, stage_b(0));
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    Codes ca, cb;
    const bool more = kt + 1 < nk;
    if (more) {
      ca = load_codes(kt + 1, rs_a, row_a, bits_a, rs_sa, srow_a);
      cb = load_codes(kt + 1, rs_b, row_b, bits_b, rs_sb, srow_b);
    }
    const char* as = stage_a(kt);
    const char* bs = stage_b(kt);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_g fa[kGFM], fb[kGFN];
#pragma unroll
      for (int i = 0; i < kGFM; ++i) {
        const int rr = wm * (kGBM / kGWM) + i * 32 + (lane & 31);
        fa[i] = *(const bf16x8_g*)(as + rr * 64 + (a_phys(rr, 2 * ks + (lane >> 5)) << 4));
      }
#pragma unroll
      for (int j = 0; j < kGFN; ++j) {
        const int rr = wn * (kGBN / kGWN) + j * 32 + (lane & 31);
        fb[j] = *(const bf16x8_g*)(bs + rr * 64 + (a_phys(rr, 2 * ks + (lane >> 5)) << 4));
      }
#pragma unroll
      for (int i = 0; i < kGFM; ++i)
#pragma unroll
        for (int j = 0; j < kGFN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      // stage (kt + 1) & 1 was last read in step kt - 1, before its barrier
      decode_store(kt + 1, ca, p.fa, bits_a, rs_sa, srow_a, stage_a(kt + 1));
      decode_store(kt + 1, cb, p.fb, bits_b, rs_sb, srow_b, stage_b(kt + 1));
    }
    __syncthreads();
  }

  // clipped epilogue: lane l, accumulator q of block (i, j) is row
  // 8(q/4) + 4(l/32) + q%4, column l%32 of that 32 x 32 block
#pragma unroll
  for (int i = 0; i < kGFM; ++i)
#pragma unroll
    for (int j = 0; j < kGFN; ++j) {
      const int64_t col = n0 + wn * (kGBN / kGWN) + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm * (kGBM / kGWM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (row >= p.M) continue;
        const float a = p.acc ? p.acc[row * p.ldacc + col] : 0.f;
        p.C[row * p.ldc + col] = a + acc[i][j][q];
      }
    }
}

}  // namespace

int gemm_scaled_general(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                        const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                        int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const char* name = "gemm_scaled";
  // 32-bit buffer offsets within one tile's rows (codes and scale bytes)
  if ((int64_t)kGBM * lda + 64 >= kMaxOffset32 || (int64_t)kGBN * ldb + 64 >= kMaxOffset32 ||
      (int64_t)kGBM * lds_a + 64 >= kMaxOffset32 || (int64_t)kGBN * lds_b + 64 >= kMaxOffset32 ||
      M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2 || block > INT32_MAX)
    return fail(STG_ERR_RANGE, "%s: a tile's rows span more than 2^31 bytes, or a size is too large", name);
  static const bool lds_ok = hipFuncSetAttribute((const void*)gemm_scaled_general_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 2 * kGStage) == hipSuccess;
  if (!lds_ok) return fail(STG_ERR_LAUNCH, "%s: cannot reserve LDS for the general scaled GEMM kernel", name);
  GeneralParams p{};
  p.A = (const char*)A;
  p.B = (const char*)Bt;
  p.sa = (const char*)a_scale;
  p.sb = (const char*)b_scale;
  p.acc = acc;
  p.C = C;
  p.lda = lda, p.ldb = ldb, p.lds_a = lds_a, p.lds_b = lds_b, p.ldacc = ldacc, p.ldc = ldc;
  p.M = M, p.N = N, p.K = K;
  p.fa = a_fmt, p.fb = b_fmt, p.sf = scale_fmt;
  p.block = (int32_t)block;
  p.tiles_m = (int32_t)((M + kGBM - 1) / kGBM);
  p.tiles_n = (int32_t)((N + kGBN - 1) / kGBN);
  const int64_t n_wg = (int64_t)p.tiles_m * p.tiles_n;
  if (n_wg == 0) return STG_OK;
  launch_kernel("gemm_scaled/general", gemm_scaled_general_kernel, dim3((unsigned)n_wg), dim3(kGNT),
                (uint32_t)(2 * kGStage), s, p);
  return check_launch(name);
}

}  // namespace stg
