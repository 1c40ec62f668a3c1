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
// it is a multiple of 2^-133 (bf16's subnormal step) below 2^128 -- always
// with e4m3 scales (the products lie in [2^-25, 2^25]); with e8m0 scale
// bytes 3..246 for e4m3 operands, 10..239 for e5m2 and 0..252 for e2m1.  The
// bf16 MFMA keeps subnormal inputs, and the bf16 products of two such values
// are exact in fp32, so the result differs from the exact sum only by fp32
// accumulation rounding.
//
//  * Tiles 256 x 256 on 8 waves (2 x 4), each wave 128 x 64 accumulators of
//    v_mfma_f32_32x32x16_bf16; K steps of 64.
//  * Staging: four lanes share a row, each owning 16 consecutive K values of
//    two rows of A and of two rows of Bt per step.  A lane loads their codes
//    with one buffer load per row (16 bytes of fp8, 8 of fp4) through a
//    range-checked buffer resource (rows past M or N and bytes past the
//    matrix read as zero codes), finds the values' scale byte, decodes code
//    and scale from their bit fields, multiplies, rounds to bf16 (exact,
//    above) and writes the 16 bf16 values to an LDS stage of 128-byte rows
//    under a conflict-free chunk swizzle; values at K and beyond are written
//    as zero.  Both operands are K-contiguous rows, so both MFMA operands are
//    plain ds_read_b128 reads.
//  * Codes are loaded two steps ahead into two register sets; two LDS
//    stages: step k's MFMAs, then the decode of step k+1 into the other
//    stage, interleaved by the scheduler; one barrier per step.
//  * Clipped fp32 epilogue adding the optional accumulator input.
#include "gemm_common.h"

#include <type_traits>

namespace stg {
namespace {

typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef float f32x16_g __attribute__((ext_vector_type(16)));
typedef float f32x2_g __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_g __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even) and packed, element 0 in the
// low half: one v_cvt_pk_bf16_f32 (converting each value on its own left two
// conversions plus a shift and an or per pair).
__device__ __forceinline__ uint32_t pack_bf16x2(f32x2_g v) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_g));
}

constexpr int kGBM = 256, kGBN = 256, kGBK = 64;
constexpr int kGWM = 2, kGWN = 4, kGNT = kGWM * kGWN * 64;
constexpr int kGFM = kGBM / kGWM / 32, kGFN = kGBN / kGWN / 32;  // 4 x 2 blocks of 32 x 32 per wave
constexpr int kGRowB = kGBK * 2;                                   // bytes per staged bf16 row
constexpr int kGStage = (kGBM + kGBN) * kGRowB;                    // 64 KiB: A rows then B rows, 128 bytes each

// Physical 16-byte chunk of logical chunk c (0..7) in staged row r: the 16
// consecutive rows one ds_read_b128 phase reads (one logical chunk each) fall
// on 16 distinct 16-byte bank groups of the 256-byte bank sweep -- rows of
// one parity share a half of the sweep and (r >> 1) & 7 spreads them over it.
__device__ __forceinline__ int g_phys(int r, int c) { return c ^ ((r >> 1) & 7); }

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

// 16 codes of one format times one scale, as 16 bf16 values.  The gfx950
// conversions (v_cvt_scalef32_pk_f32_fp8 / _bf8 / _fp4) decode two codes
// exactly and multiply them by 2^(exponent of their f32 scale operand) --
// only the exponent is used -- so `pow2` carries the scale's power of two
// and `mult` the rest (an e4m3 scale's significand and sign, a zero or NaN
// scale), applied by an exact fp32 multiply before the bf16 rounding.
template <int FMT, int E>
__device__ __forceinline__ uint32_t decode2(const u32x4& w, float pow2, float mult) {
  f32x2_g f;
  if constexpr (FMT == STG_LP_E4M3)
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[E >> 2], pow2, ((E >> 1) & 1) != 0);
  else if constexpr (FMT == STG_LP_E5M2)
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w[E >> 2], pow2, ((E >> 1) & 1) != 0);
  else
    f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[E >> 3], pow2, (E >> 1) & 3);
  return pack_bf16x2(f * mult);
}
template <int FMT>
__device__ __forceinline__ void decode16(const u32x4& w, float pow2, float mult, u32x4 out[2]) {
  out[0] = (u32x4){decode2<FMT, 0>(w, pow2, mult), decode2<FMT, 2>(w, pow2, mult), decode2<FMT, 4>(w, pow2, mult),
                   decode2<FMT, 6>(w, pow2, mult)};
  out[1] = (u32x4){decode2<FMT, 8>(w, pow2, mult), decode2<FMT, 10>(w, pow2, mult), decode2<FMT, 12>(w, pow2, mult),
                   decode2<FMT, 14>(w, pow2, mult)};
}

// A block scale byte as decode16's pow2 and mult, selected without a branch
// (a branch in the GEMM's K loop would cut a step into blocks the scheduler
// cannot interleave): e8m0, 2^(b-127), b = 0 as 2^-126 * 0.5 (an exponent
// field of 0 is not a power of two for the conversion), 0xFF NaN; e4m3, its
// value (normal f32, zero or NaN) decoded by the hardware conversion with a
// unit scale, split into its power of two and the rest.
__device__ __forceinline__ void split_scale(uint32_t b, int32_t sf, float& pow2, float& mult) {
  const float p8 = b ? __uint_as_float(b << 23) : 0x1p-126f;
  const float m8 = b == 0xFF ? __uint_as_float(0x7FC00000u) : b ? 1.f : 0.5f;
  const float sc = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b, 1.0f, false)[0];
  const bool zero = sc == 0.f, nan = sc != sc;
  const float p4 = zero || nan ? 1.f : __uint_as_float(__float_as_uint(sc) & 0x7F800000u);
  const float m4 = zero ? 0.f : nan ? sc : __uint_as_float((__float_as_uint(sc) & 0x807FFFFFu) | 0x3F800000u);
  const bool e8 = sf == STG_SC_E8M0;
  pow2 = e8 ? p8 : p4;
  mult = e8 ? m8 : m4;
}

// Codes of one lane's 16 K values of one row (16 bytes of fp8 or 8 of fp4)
// and the scale byte they share (blocks that are multiples of 16).
struct Codes {
  u32x4 w;
  uint32_t s;
};

template <int FA, int FB, bool BLK16>
__global__ __launch_bounds__(kGNT) void gemm_scaled_general_kernel(GeneralParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int BA = FA == STG_LP_E2M1 ? 4 : 8, BB = FB == STG_LP_E2M1 ? 4 : 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kGWN, wn = wave % kGWN;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * kGBM, n0 = (int64_t)tn * kGBN;
  const int nk = (int)((p.K + kGBK - 1) / kGBK);

  // this lane's staging: K values 16q .. 16q+15 of each step in rows r and
  // r + 128 of the A tile and of the Bt tile.  Four lanes cover a row's 64
  // K values, so one load instruction reads 16 rows x 64 contiguous bytes of
  // codes (fp8): 16 cache lines per KiB where two lanes per row, 32 K values
  // a step, touched 32 (and the kernel spent about a third of its time on
  // those requests)
  const int r = tid >> 2, q = tid & 3;
  constexpr int kRP = kGBM / (kGNT / 4);  // row passes: 2
  // buffer resources over each operand's rows of this tile and over the
  // scale matrices: offsets past the matrix read as zero
  auto rsrc_rows = [](const char* base, int64_t row0, int64_t rows, int64_t ld, int64_t row_bytes) {
    const int64_t avail = rows > row0 ? (rows - 1 - row0) * ld + row_bytes : 0;
    return make_rsrc(base + (rows > row0 ? row0 * ld : 0), (uint32_t)(avail < (int64_t)kOOB ? avail : kOOB - 1));
  };
  const int64_t nkb = p.K / p.block;
  const __amdgpu_buffer_rsrc_t rs_a = rsrc_rows(p.A, m0, p.M, p.lda, (p.K * BA + 7) / 8);
  const __amdgpu_buffer_rsrc_t rs_b = rsrc_rows(p.B, n0, p.N, p.ldb, (p.K * BB + 7) / 8);
  const __amdgpu_buffer_rsrc_t rs_sa = rsrc_rows(p.sa, m0, p.M, p.lds_a, nkb);
  const __amdgpu_buffer_rsrc_t rs_sb = rsrc_rows(p.sb, n0, p.N, p.lds_b, nkb);
  uint32_t row_a[kRP], row_b[kRP], srow_a[kRP], srow_b[kRP];
#pragma unroll
  for (int t = 0; t < kRP; ++t) {
    const int rt = r + t * (kGNT / 4);
    const bool in_a = m0 + rt < p.M, in_b = n0 + rt < p.N;
    row_a[t] = in_a ? (uint32_t)(rt * p.lda) : kOOB;
    row_b[t] = in_b ? (uint32_t)(rt * p.ldb) : kOOB;
    srow_a[t] = in_a ? (uint32_t)(rt * p.lds_a) : kOOB;
    srow_b[t] = in_b ? (uint32_t)(rt * p.lds_b) : kOOB;
  }

  // codes of step kt.  All but the last step lie inside K: one vector load
  // each.  In the last step the row may end inside a lane's 16 values, and a
  // vector load there could reach past the matrix's last byte: byte loads up
  // to the row's end instead (bytes past it read as zero).
  auto load_codes = [&](auto bits_c, int kt, const __amdgpu_buffer_rsrc_t& rs, uint32_t row_off,
                        const __amdgpu_buffer_rsrc_t& rss, uint32_t srow, bool last, uint32_t sq) {
    constexpr int bits = decltype(bits_c)::value;
    Codes c;
    const uint32_t k = (uint32_t)kt * kGBK + 16 * q;
    const uint32_t off = row_off == kOOB ? kOOB : row_off + k * bits / 8;
    c.w = (u32x4){0, 0, 0, 0};
    if (!last || (int64_t)k + 16 <= p.K) {
      if constexpr (bits == 8) {
        c.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
        c.w = (u32x4){v[0], v[1], 0, 0};
      }
    } else if ((int64_t)k < p.K && row_off != kOOB) {
      const int nb = (int)(((p.K - k) * bits + 7) / 8);
      uint32_t by[16];
#pragma unroll
      for (int b = 0; b < 16; ++b) by[b] = __builtin_amdgcn_raw_buffer_load_b8(rs, b < nb ? off + b : kOOB, 0, 0);
#pragma unroll
      for (int b = 0; b < 16; ++b) c.w[b >> 2] |= by[b] << (8 * (b & 3));
      // fp4 with an odd number of values left: the last byte's high nibble
      // is past K
      if (bits == 4 && ((p.K - k) & 1)) c.w[(nb - 1) >> 2] &= ~(0xF0u << (8 * ((nb - 1) & 3)));
    }
    c.s = 0;
    if constexpr (BLK16)
      c.s = __builtin_amdgcn_raw_buffer_load_b8(
          rss, (srow == kOOB || (int64_t)k >= p.K) ? kOOB : srow + sq, 0, 0);
    return c;
  };

  // scaled bf16 values of one lane's 16 K values into LDS row rw of the
  // operand region (zero at K and beyond)
  auto decode_store = [&](auto fmt_c, int kt, const Codes& c, const __amdgpu_buffer_rsrc_t& rss, uint32_t srow,
                          char* region, int rw) {
    constexpr int fmt = decltype(fmt_c)::value;
    u32x4 out[2];
    if constexpr (BLK16) {
      // one scale for the 16 values; codes past K were loaded as zero
      float pow2, mult;
      split_scale(c.s, p.sf, pow2, mult);
      decode16<fmt>(c.w, pow2, mult, out);
    } else {
      // blocks that do not hold whole 16-value runs: each value finds its
      // scale (the block boundaries inside the run, at most 16)
      constexpr int bits = fmt == STG_LP_E2M1 ? 4 : 8;
      const int64_t k0 = (int64_t)kt * kGBK + 16 * q;
      float sc = 0.f;
      int64_t sidx = -1, next = 0;  // scale index of the current value, first K of the next block
      if (k0 < p.K) {
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
          const uint32_t code =
              bits == 8 ? (c.w[ee >> 2] >> (8 * (ee & 3))) & 0xFF : (c.w[ee >> 3] >> (4 * (ee & 7))) & 0xF;
          const int64_t k = k0 + ee;
          if (k < p.K && k >= next) {  // k == next: the next block starts here
            sidx += 1;
            next += p.block;
            sc = decode_scale(
                srow == kOOB ? 0u : __builtin_amdgcn_raw_buffer_load_b8(rss, srow + (uint32_t)sidx, 0, 0), p.sf);
          }
          v[u] = k < p.K ? decode_code(code, fmt) * sc : 0.f;
        }
        out[e >> 3][(e >> 1) & 3] = pack_bf16x2((f32x2_g){v[0], v[1]});
      }
    }
    *(u32x4*)(region + rw * kGRowB + (g_phys(rw, 2 * q) << 4)) = out[0];
    *(u32x4*)(region + rw * kGRowB + (g_phys(rw, 2 * q + 1) << 4)) = out[1];
  };

  f32x16_g acc[kGFM][kGFN];
#pragma unroll
  for (int i = 0; i < kGFM; ++i)
#pragma unroll
    for (int j = 0; j < kGFN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto stage_a = [&](int kt) { return smem + (kt & 1) * kGStage; };
  auto stage_b = [&](int kt) { return smem + (kt & 1) * kGStage + kGBM * kGRowB; };
  using IA = std::integral_constant<int, FA>;
  using IB = std::integral_constant<int, FB>;
  using BitsA = std::integral_constant<int, BA>;
  using BitsB = std::integral_constant<int, BB>;

  // codes are loaded two steps ahead (one global round trip is longer than
  // a step), into two register sets used alternately, each holding this
  // lane's 16 values in each of its rows of A and of Bt
  struct CodeSet {
    Codes a[kRP], b[kRP];
  };
  CodeSet set0, set1;
  // scale block of this lane's 16 values in the next step loaded, as a
  // running quotient and remainder of 64 kt + 16 q by the block (loads go
  // step by step, 0, 1, 2, ...; a block of 16 or more advances at most four
  // times per step), instead of a division per load
  uint32_t s_q = 0, s_r = 0;
  if constexpr (BLK16) {
    s_q = 16u * q / (uint32_t)p.block;
    s_r = 16u * q % (uint32_t)p.block;
  }
  auto next_scale = [&]() {
    const uint32_t sq = s_q;
    if constexpr (BLK16) {
      const uint32_t blk = (uint32_t)p.block;
      s_r += kGBK;
#pragma unroll
      for (int u = 0; u < kGBK / 16; ++u)
        if (s_r >= blk) s_r -= blk, ++s_q;
    }
    return sq;
  };
  auto load_set = [&](int kt, CodeSet& cs, bool last) {
    const uint32_t sq = next_scale();
#pragma unroll
    for (int t = 0; t < kRP; ++t) {
      cs.a[t] = load_codes(BitsA{}, kt, rs_a, row_a[t], rs_sa, srow_a[t], last, sq);
      cs.b[t] = load_codes(BitsB{}, kt, rs_b, row_b[t], rs_sb, srow_b[t], last, sq);
    }
  };
  auto decode_set = [&](int kt, const CodeSet& cs) {
#pragma unroll
    for (int t = 0; t < kRP; ++t) {
      decode_store(IA{}, kt, cs.a[t], rs_sa, srow_a[t], stage_a(kt), r + t * (kGNT / 4));
      decode_store(IB{}, kt, cs.b[t], rs_sb, srow_b[t], stage_b(kt), r + t * (kGNT / 4));
    }
  };
  auto mfma_step = [&](int kt) {
    const char* as = stage_a(kt);
    const char* bs = stage_b(kt);
#pragma unroll
    for (int ks = 0; ks < kGBK / 16; ++ks) {
      bf16x8_g fa[kGFM], fb[kGFN];
#pragma unroll
      for (int i = 0; i < kGFM; ++i) {
        const int rr = wm * (kGBM / kGWM) + i * 32 + (lane & 31);
        fa[i] = *(const bf16x8_g*)(as + rr * kGRowB + (g_phys(rr, 2 * ks + (lane >> 5)) << 4));
      }
#pragma unroll
      for (int j = 0; j < kGFN; ++j) {
        const int rr = wn * (kGBN / kGWN) + j * 32 + (lane & 31);
        fb[j] = *(const bf16x8_g*)(bs + rr * kGRowB + (g_phys(rr, 2 * ks + (lane >> 5)) << 4));
      }
#pragma unroll
      for (int i = 0; i < kGFM; ++i)
#pragma unroll
        for (int j = 0; j < kGFN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };
  // step kt: load the codes of step kt + 2 into `later` -- that set's codes,
  // of step kt, were decoded in step kt - 1 -- then the MFMAs of stage kt,
  // then the decode of step kt + 1 from `next` into the other stage, last
  // read in step kt - 1 before its barrier
  auto step = [&](int kt, CodeSet& next, CodeSet& later) {
    if (kt + 2 < nk) load_set(kt + 2, later, kt + 2 == nk - 1);
    mfma_step(kt);
    if (kt + 1 < nk) decode_set(kt + 1, next);
    __syncthreads();
  };
  // the same with only whole-vector loads and no end tests, for the steps
  // whose loads and decodes all lie before the last step
  constexpr int kMfmas = kGFM * kGFN * (kGBK / 16);  // per wave and step
  auto inner_step = [&](int kt, CodeSet& next, CodeSet& later) {
    load_set(kt + 2, later, false);
    mfma_step(kt);
    decode_set(kt + 1, next);
    // the decode's VALU work between the MFMAs of the same wave: left to
    // itself the scheduler issues all the MFMAs and then the decode, and the
    // per-step barrier keeps a SIMD's two waves in that same phase, so the
    // matrix core idled through both waves' decodes
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // the first operand reads
#pragma unroll
    for (int i = 0; i < kMfmas; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // five VALU
    }
    __syncthreads();
  };

  if (nk > 0) {
    load_set(0, set0, nk == 1);
    if (nk > 1) load_set(1, set1, nk == 2);
    decode_set(0, set0);
  }
  __syncthreads();
  int kt = 0;
  // inner steps while kt + 2 < nk - 1, two at a time (the register sets swap)
  for (; kt + 4 < nk; kt += 2) {
    inner_step(kt, set1, set0);
    inner_step(kt + 1, set0, set1);
  }
  for (; kt + 1 < nk; kt += 2) {
    step(kt, set1, set0);
    step(kt + 1, set0, set1);
  }
  if (kt < nk) step(kt, set1, set0);

  // clipped epilogue: lane l, accumulator v of block (i, j) is row
  // 8(v/4) + 4(l/32) + v%4, column l%32 of that 32 x 32 block
#pragma unroll
  for (int i = 0; i < kGFM; ++i)
#pragma unroll
    for (int j = 0; j < kGFN; ++j) {
      const int64_t col = n0 + wn * (kGBN / kGWN) + j * 32 + (lane & 31);
      if (col >= p.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * (kGBM / kGWM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (row >= p.M) continue;
        const float a = p.acc ? p.acc[row * p.ldacc + col] : 0.f;
        p.C[row * p.ldc + col] = a + acc[i][j][v];
      }
    }
}

// ---- decoded operands: each value scaled and rounded to bf16 once ---------
//
// The kernel above decodes an operand row in every tile that uses it: at
// (8191, 8193, 4096) each A row 33 times and each Bt row 32 times, so its
// decode work is as large as its MFMA work.  With a workspace, the operands
// are instead decoded once, exactly as above (the same conversions, the same
// bf16 values), into bf16 matrices A' (M, K) and B' (K, N) -- B transposed,
// the layout the bf16 GEMM stages -- and the bf16 GEMM multiplies them with
// the same fp32 accumulation: the results differ only by its summation order.

struct DecodeParams {
  const char* codes;     // (rows, K) operand codes, row stride ld bytes
  const uint8_t* scale;  // (rows, K / block) scale bytes, row stride lds
  __bf16* out;           // A': (rows, ldo); B' (transposed): (K, ldo)
  int64_t ld, lds, ldo, rows, K;
  int32_t block, sf;
};

// The 16 codes of run k0 .. k0+15 of row r (k0 < K), values past K as code 0.
template <int BITS>
__device__ __forceinline__ u32x4 run_codes(const DecodeParams& d, int64_t r, int64_t k0) {
  const char* row = d.codes + r * d.ld + k0 * BITS / 8;
  u32x4 w = {0, 0, 0, 0};
  if (k0 + 16 <= d.K) {
    if constexpr (BITS == 8) {
      w = ld16(row);
    } else {
      uint32_t h[2];
      __builtin_memcpy(h, row, 8);
      w[0] = h[0], w[1] = h[1];
    }
    return w;
  }
  const int nv = (int)(d.K - k0);                 // values left in the row, 1..15
  const int nb = (nv * BITS + 7) / 8;             // their bytes
  for (int b = 0; b < nb; ++b) w[b >> 2] |= (uint32_t)(uint8_t)row[b] << (8 * (b & 3));
  if (BITS == 4 && (nv & 1)) w[(nb - 1) >> 2] &= ~(0xF0u << (8 * ((nb - 1) & 3)));  // nibble past K
  return w;
}

// 16 bf16 values of run k0 of row r, as the GEMM kernel above decodes them.
template <int FMT, bool BLK16>
__device__ __forceinline__ void run_decode(const DecodeParams& d, int64_t r, int64_t k0, u32x4 out[2]) {
  constexpr int BITS = FMT == STG_LP_E2M1 ? 4 : 8;
  const u32x4 w = run_codes<BITS>(d, r, k0);
  const uint8_t* srow = d.scale + r * d.lds;
  if constexpr (BLK16) {
    float pow2, mult;
    split_scale(srow[k0 / d.block], d.sf, pow2, mult);
    decode16<FMT>(w, pow2, mult, out);
  } else {
    for (int e = 0; e < 16; e += 2) {
      float v[2];
      for (int u = 0; u < 2; ++u) {
        const int ee = e + u;
        const int64_t k = k0 + ee;
        const uint32_t code = BITS == 8 ? (w[ee >> 2] >> (8 * (ee & 3))) & 0xFF : (w[ee >> 3] >> (4 * (ee & 7))) & 0xF;
        v[u] = k < d.K ? decode_code(code, FMT) * decode_scale(srow[k / d.block], d.sf) : 0.f;
      }
      out[e >> 3][(e >> 1) & 3] = pack_bf16x2((f32x2_g){v[0], v[1]});
    }
  }
}

// A': one thread per run of 16 values; ldo is a multiple of 16, so a row's
// last run (zero past K) stays inside the row.
template <int FMT, bool BLK16>
__global__ __launch_bounds__(256) void decode_rows_kernel(DecodeParams d, int64_t runs_per_row) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= d.rows * runs_per_row) return;
  const int64_t r = t / runs_per_row, k0 = (t - r * runs_per_row) * 16;
  u32x4 out[2];
  run_decode<FMT, BLK16>(d, r, k0, out);
  char* dst = (char*)(d.out + r * d.ldo + k0);
  st16(dst, out[0]);
  st16(dst + 16, out[1]);
}

// B': a workgroup decodes 64 rows x 64 K values of Bt (four threads per row,
// one run each) into LDS, then writes them transposed: 64 rows of B', each 64
// columns as eight 16-byte chunks.  ldo is a multiple of 8, so a chunk that
// starts before N stays inside its row.
constexpr int kDecT = 64;
template <int FMT, bool BLK16>
__global__ __launch_bounds__(256) void decode_cols_kernel(DecodeParams d, int64_t n_tiles) {
  constexpr int kPitch = kDecT + 8;  // bf16 per LDS row: 144 bytes, 16-byte aligned, reads spread over banks
  __shared__ __attribute__((aligned(16))) __bf16 tile[kDecT * kPitch];
  const int tid = threadIdx.x;
  // workgroup (row tile, K tile), row tiles fastest
  const int64_t bt = (int64_t)blockIdx.x / n_tiles;
  const int64_t n0 = ((int64_t)blockIdx.x - bt * n_tiles) * kDecT, kb = bt * kDecT;
  {
    const int n = tid >> 2, q = tid & 3;
    const int64_t k0 = kb + 16 * q;
    u32x4 out[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    if (n0 + n < d.rows && k0 < d.K) run_decode<FMT, BLK16>(d, n0 + n, k0, out);
    *(u32x4*)(tile + n * kPitch + 16 * q) = out[0];
    *(u32x4*)(tile + n * kPitch + 16 * q + 8) = out[1];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i, kk = c >> 3, nc = c & 7;
    const int64_t k = kb + kk, n = n0 + 8 * nc;
    if (k >= d.K || n >= d.rows) continue;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t lo = __builtin_bit_cast(uint16_t, tile[(8 * nc + e) * kPitch + kk]);
      const uint32_t hi = __builtin_bit_cast(uint16_t, tile[(8 * nc + e + 1) * kPitch + kk]);
      v[e >> 1] = lo | hi << 16;
    }
    st16((char*)(d.out + k * d.ldo + n), v);
  }
}

constexpr int64_t kDecAlign = 256;
inline int64_t dec_up(int64_t x) { return (x + kDecAlign - 1) / kDecAlign * kDecAlign; }
// leading dimensions of A' and B' (elements): whole runs of 16 in A' rows;
// B' rows a multiple of 128 bytes, so the transposed 128-byte chunks are whole
// cache lines (with rows 16-byte aligned only: decode B 3 us slower, the bf16
// GEMM 3-6 us)
inline int64_t dec_lda(int64_t K) { return (K + 15) / 16 * 16; }
inline int64_t dec_ldb(int64_t N) { return (N + 63) / 64 * 64; }

template <int FMT>
int launch_decode(bool rows, bool blk16, const DecodeParams& d, hipStream_t s) {
  if (rows) {
    const int64_t runs = (d.K + 15) / 16;
    const int64_t grid = (d.rows * runs + 255) / 256;
    if (grid > INT32_MAX) return fail(STG_ERR_RANGE, "gemm_scaled: too many values to decode");
    if (blk16)
      launch_kernel("gemm_scaled/decode_a", decode_rows_kernel<FMT, true>, dim3((unsigned)grid), dim3(256), 0, s, d,
                    runs);
    else
      launch_kernel("gemm_scaled/decode_a", decode_rows_kernel<FMT, false>, dim3((unsigned)grid), dim3(256), 0, s, d,
                    runs);
  } else {
    const int64_t n_tiles = (d.rows + kDecT - 1) / kDecT, grid = n_tiles * ((d.K + kDecT - 1) / kDecT);
    if (grid > INT32_MAX) return fail(STG_ERR_RANGE, "gemm_scaled: too many values to decode");
    if (blk16)
      launch_kernel("gemm_scaled/decode_b", decode_cols_kernel<FMT, true>, dim3((unsigned)grid), dim3(256), 0, s, d,
                    n_tiles);
    else
      launch_kernel("gemm_scaled/decode_b", decode_cols_kernel<FMT, false>, dim3((unsigned)grid), dim3(256), 0, s, d,
                    n_tiles);
  }
  return check_launch("gemm_scaled");
}

int decode_operand(int32_t fmt, bool rows, bool blk16, const DecodeParams& d, hipStream_t s) {
  switch (fmt) {
    case STG_LP_E4M3: return launch_decode<STG_LP_E4M3>(rows, blk16, d, s);
    case STG_LP_E5M2: return launch_decode<STG_LP_E5M2>(rows, blk16, d, s);
    default: return launch_decode<STG_LP_E2M1>(rows, blk16, d, s);
  }
}

template <int FA, int FB>
int launch_general(const GeneralParams& p, int64_t n_wg, hipStream_t s) {
  static OncePerDevice once;  // the kernels' dynamic LDS limit, once on each device
  const bool lds_ok = once.run([] {
    return hipFuncSetAttribute((const void*)gemm_scaled_general_kernel<FA, FB, true>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kGStage) == hipSuccess &&
           hipFuncSetAttribute((const void*)gemm_scaled_general_kernel<FA, FB, false>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kGStage) == hipSuccess;
  });
  if (!lds_ok) return fail(STG_ERR_LAUNCH, "gemm_scaled: cannot reserve LDS for the general scaled GEMM kernel");
  if (p.block % 16 == 0)
    launch_kernel("gemm_scaled/general", gemm_scaled_general_kernel<FA, FB, true>, dim3((unsigned)n_wg), dim3(kGNT),
                  (uint32_t)(2 * kGStage), s, p);
  else
    launch_kernel("gemm_scaled/general", gemm_scaled_general_kernel<FA, FB, false>, dim3((unsigned)n_wg), dim3(kGNT),
                  (uint32_t)(2 * kGStage), s, p);
  return check_launch("gemm_scaled");
}

template <int FA>
int launch_general_a(const GeneralParams& p, int64_t n_wg, hipStream_t s) {
  switch (p.fb) {
    case STG_LP_E4M3: return launch_general<FA, STG_LP_E4M3>(p, n_wg, s);
    case STG_LP_E5M2: return launch_general<FA, STG_LP_E5M2>(p, n_wg, s);
    default: return launch_general<FA, STG_LP_E2M1>(p, n_wg, s);
  }
}

}  // namespace

int64_t gemm_scaled_general_workspace(int64_t M, int64_t N, int64_t K) {
  // decoding first pays once each operand row would be decoded by more than
  // one tile of the kernel above; the bf16 GEMM takes sizes up to 2^30 and a
  // stage (256 rows of A', 32 of B') within 2^31 bytes
  if (M <= kGBM || N <= kGBN || K == 0 || M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return 0;
  if (256 * dec_lda(K) * 2 + 256 >= kMaxOffset32 || 32 * dec_ldb(N) * 2 + 512 >= kMaxOffset32) return 0;
  return dec_up(M * dec_lda(K) * 2) + dec_up(K * dec_ldb(N) * 2);
}

int gemm_scaled_general(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                        const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                        int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t s) {
  const char* name = "gemm_scaled";
  const int64_t need = gemm_scaled_general_workspace(M, N, K);
  if (workspace && need > 0) {
    if (workspace_bytes < need)
      return fail(STG_ERR_INVALID, "%s: workspace of %lld bytes, %lld needed", name, (long long)workspace_bytes,
                  (long long)need);
    if ((uintptr_t)workspace % kDecAlign) return fail(STG_ERR_INVALID, "%s: workspace must be 256-byte aligned", name);
    __bf16* ad = (__bf16*)workspace;
    __bf16* bd = (__bf16*)((char*)workspace + dec_up(M * dec_lda(K) * 2));
    DecodeParams d{};
    d.block = (int32_t)block;
    d.sf = scale_fmt;
    d.K = K;
    const bool blk16 = block % 16 == 0;
    d.codes = (const char*)A, d.scale = (const uint8_t*)a_scale, d.out = ad;
    d.ld = lda, d.lds = lds_a, d.ldo = dec_lda(K), d.rows = M;
    int rc = decode_operand(a_fmt, true, blk16, d, s);
    if (rc) return rc;
    d.codes = (const char*)Bt, d.scale = (const uint8_t*)b_scale, d.out = bd;
    d.ld = ldb, d.lds = lds_b, d.ldo = dec_ldb(N), d.rows = N;
    if ((rc = decode_operand(b_fmt, false, blk16, d, s))) return rc;
    static const GemmNames names{"gemm_scaled", "gemm_scaled/bf16_main", "gemm_scaled/bf16_edge",
                                 "gemm_scaled/bf16_skinny"};
    return gemm_bf16(names, ad, dec_lda(K), bd, dec_ldb(N), acc, ldacc, C, ldc, M, N, K, STG_F32, s);
  }
  // 32-bit buffer offsets within one tile's rows (codes and scale bytes)
  if ((int64_t)kGBM * lda + 64 >= kMaxOffset32 || (int64_t)kGBN * ldb + 64 >= kMaxOffset32 ||
      (int64_t)kGBM * lds_a + 64 >= kMaxOffset32 || (int64_t)kGBN * lds_b + 64 >= kMaxOffset32 ||
      M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2 || block > INT32_MAX)
    return fail(STG_ERR_RANGE, "%s: a tile's rows span more than 2^31 bytes, or a size is too large", name);
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
  switch (a_fmt) {
    case STG_LP_E4M3: return launch_general_a<STG_LP_E4M3>(p, n_wg, s);
    case STG_LP_E5M2: return launch_general_a<STG_LP_E5M2>(p, n_wg, s);
    default: return launch_general_a<STG_LP_E2M1>(p, n_wg, s);
  }
}

}  // namespace stg
