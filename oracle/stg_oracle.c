/*
 * stg_oracle.c -- plain single-threaded CPU oracle.  TEST INFRASTRUCTURE
 * ONLY: never linked into, included by or called from the product library.
 * Definitions and citations are in stg_oracle.h; each function below is the
 * definition written out as loops, with no blocking or reordering.
 */
#include "stg_oracle.h"

#include <math.h>
#include <string.h>

/* ---- grid sizing ------------------------------------------------------ */

int64_t orc_tile_grid(int64_t extent, int64_t origin, int64_t tile) {
  int64_t span = extent - origin; /* elements from the first origin to the end */
  if (span <= 0 || tile <= 0) return 0;
  return (span + tile - 1) / tile; /* ceiling division of a positive span */
}

/* ---- rounding to a binary interchange format -------------------------- */

uint64_t orc_round_to_format(double v, int ebits, int mbits) {
  const int bias = (1 << (ebits - 1)) - 1;
  const int emin = 1 - bias;
  const int emax = bias;
  const uint64_t sign = signbit(v) ? (uint64_t)1 << (ebits + mbits) : 0;
  const uint64_t exp_all = ((uint64_t)1 << ebits) - 1;
  if (isnan(v)) return sign | (exp_all << mbits) | ((uint64_t)1 << (mbits - 1));
  double a = fabs(v);
  if (isinf(a)) return sign | (exp_all << mbits);
  if (a == 0.0) return sign;
  int x;
  frexp(a, &x); /* a = f * 2^x, f in [0.5, 1) */
  int e = x - 1; /* a in [2^e, 2^(e+1)) */
  if (e < emin) {
    /* subnormal range: fixed quantum 2^(emin - mbits); a carry to 2^mbits
     * lands exactly on the smallest normal's bit pattern */
    double n = rint(ldexp(a, mbits - emin));
    return sign | (uint64_t)n;
  }
  double n = rint(ldexp(a, mbits - e)); /* in [2^mbits, 2^(mbits+1)] */
  if (n == ldexp(1.0, mbits + 1)) {
    e += 1;
    n = ldexp(1.0, mbits);
  }
  if (e > emax) return sign | (exp_all << mbits);
  return sign | ((uint64_t)(e + bias) << mbits) | ((uint64_t)n - ((uint64_t)1 << mbits));
}

int orc_padding_bits(double v, int dtype, void* out) {
  switch (dtype) {
    case ORC_F32: {
      uint32_t b = (uint32_t)orc_round_to_format(v, 8, 23);
      memcpy(out, &b, 4);
      return 0;
    }
    case ORC_BF16: {
      uint16_t b = (uint16_t)orc_round_to_format(v, 8, 7);
      memcpy(out, &b, 2);
      return 0;
    }
    case ORC_F16: {
      uint16_t b = (uint16_t)orc_round_to_format(v, 5, 10);
      memcpy(out, &b, 2);
      return 0;
    }
    case ORC_F64:
      memcpy(out, &v, 8);
      return 0;
    case ORC_I32: {
      if (!(v > -2147483649.0 && v < 2147483648.0)) return -1;
      int32_t b = (int32_t)v;
      memcpy(out, &b, 4);
      return 0;
    }
    case ORC_I64: {
      if (!(v >= -9223372036854775808.0 && v < 9223372036854775808.0)) return -1;
      int64_t b = (int64_t)v;
      memcpy(out, &b, 8);
      return 0;
    }
    case ORC_U8: {
      if (!(v > -1.0 && v < 256.0)) return -1;
      uint8_t b = (uint8_t)v;
      memcpy(out, &b, 1);
      return 0;
    }
    default:
      return -1;
  }
}

/* ---- helpers ---------------------------------------------------------- */

static char* elem_ptr(const orc_array* x, const int64_t* coord) {
  int64_t off = 0;
  for (int d = 0; d < x->rank; ++d) off += coord[d] * x->stride[d];
  return (char*)x->data + off * (int64_t)x->esize;
}

/* Shape padded to 4 dims with trailing 1s, for uniform nested loops. */
static void shape4(const int64_t* shape, int rank, int64_t* s4) {
  for (int d = 0; d < 4; ++d) s4[d] = d < rank ? shape[d] : 1;
}

/* Shared body of the plain and masked gather: fill is the bits written for a
 * masked-out or out-of-range element. */
static void gather_body(const orc_array* a, const int32_t* indices, const uint8_t* mask,
                        int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                        int32_t axis, const void* fill, orc_array* out) {
  const int rank = a->rank;
  const int64_t T = tile_shape[axis];
  const int64_t n_tiles = T > 0 ? n_indices / T : 0;
  int64_t ts[4];
  shape4(tile_shape, rank, ts);
  int64_t c[4];
  for (int64_t t = 0; t < n_tiles; ++t)
    for (c[0] = 0; c[0] < ts[0]; ++c[0])
      for (c[1] = 0; c[1] < ts[1]; ++c[1])
        for (c[2] = 0; c[2] < ts[2]; ++c[2])
          for (c[3] = 0; c[3] < ts[3]; ++c[3]) {
            int64_t o[4], s[4];
            for (int d = 0; d < 4; ++d) o[d] = c[d];
            o[axis] += t * T;
            int valid = 1;
            for (int d = 0; d < rank; ++d) {
              s[d] = d == axis ? offset[axis] + (int64_t)indices[o[axis]] : offset[d] + o[d];
              if (s[d] < 0 || s[d] >= a->shape[d]) valid = 0;
            }
            if (mask && mask[o[axis]] == 0) valid = 0;
            char* dst = elem_ptr(out, o);
            if (valid)
              memcpy(dst, elem_ptr(a, s), (size_t)a->esize);
            else
              memcpy(dst, fill, (size_t)a->esize);
          }
}

/* ---- gather / scatter ------------------------------------------------- */

void orc_tile_gather(const orc_array* a, const int32_t* indices, int64_t n_indices,
                     const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                     orc_array* out) {
  const uint64_t zero = 0;
  gather_body(a, indices, NULL, n_indices, tile_shape, offset, axis, &zero, out);
}

void orc_tile_gather_masked(const orc_array* a, const int32_t* indices, const uint8_t* mask,
                            int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                            int32_t axis, const void* pad, orc_array* out) {
  gather_body(a, indices, mask, n_indices, tile_shape, offset, axis, pad, out);
}

void orc_tile_scatter_masked(orc_array* a, const int32_t* indices, const uint8_t* mask,
                             int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                             int32_t axis, const orc_array* tile) {
  const int rank = a->rank;
  const int64_t T = tile_shape[axis];
  const int64_t n_tiles = T > 0 ? n_indices / T : 0;
  int64_t ts[4];
  shape4(tile_shape, rank, ts);
  int64_t c[4];
  for (int64_t t = 0; t < n_tiles; ++t)
    for (c[0] = 0; c[0] < ts[0]; ++c[0])
      for (c[1] = 0; c[1] < ts[1]; ++c[1])
        for (c[2] = 0; c[2] < ts[2]; ++c[2])
          for (c[3] = 0; c[3] < ts[3]; ++c[3]) {
            int64_t o[4], s[4];
            for (int d = 0; d < 4; ++d) o[d] = c[d];
            o[axis] += t * T;
            if (mask && mask[o[axis]] == 0) continue;
            int valid = 1;
            for (int d = 0; d < rank; ++d) {
              s[d] = d == axis ? offset[axis] + (int64_t)indices[o[axis]] : offset[d] + o[d];
              if (s[d] < 0 || s[d] >= a->shape[d]) valid = 0;
            }
            if (valid) memcpy(elem_ptr(a, s), elem_ptr(tile, o), (size_t)a->esize);
          }
}

/* ---- boundary-tile copy and clipped store ----------------------------- */

void orc_tile_copy_bounded(const orc_array* src, int64_t tm, int64_t tn, int64_t origin_row,
                           int64_t origin_col, void* tiles_out) {
  const int64_t M = src->shape[0], N = src->shape[1];
  const int64_t gr_n = orc_tile_grid(M, origin_row, tm);
  const int64_t gc_n = orc_tile_grid(N, origin_col, tn);
  const size_t es = (size_t)src->esize;
  char* out = (char*)tiles_out;
  for (int64_t gr = 0; gr < gr_n; ++gr)
    for (int64_t gc = 0; gc < gc_n; ++gc) {
      const int64_t R = origin_row + gr * tm, C = origin_col + gc * tn;
      for (int64_t i = 0; i < tm; ++i)
        for (int64_t j = 0; j < tn; ++j) {
          char* dst = out + (((gr * gc_n + gc) * tm + i) * tn + j) * (int64_t)es;
          const int64_t r = R + i, col = C + j;
          if (r >= 0 && r < M && col >= 0 && col < N) {
            const int64_t coord[2] = {r, col};
            memcpy(dst, elem_ptr(src, coord), es);
          } else {
            memset(dst, 0, es);
          }
        }
    }
}

void orc_tile_store_clipped(const void* tiles_in, int32_t esize, int64_t tm, int64_t tn,
                            int64_t origin_row, int64_t origin_col, orc_array* dst) {
  const int64_t M = dst->shape[0], N = dst->shape[1];
  const int64_t gr_n = orc_tile_grid(M, origin_row, tm);
  const int64_t gc_n = orc_tile_grid(N, origin_col, tn);
  const char* in = (const char*)tiles_in;
  for (int64_t gr = 0; gr < gr_n; ++gr)
    for (int64_t gc = 0; gc < gc_n; ++gc) {
      const int64_t R = origin_row + gr * tm, C = origin_col + gc * tn;
      for (int64_t i = 0; i < tm; ++i)
        for (int64_t j = 0; j < tn; ++j) {
          const int64_t r = R + i, col = C + j;
          if (r < 0 || r >= M || col < 0 || col >= N) continue;
          const int64_t coord[2] = {r, col};
          memcpy(elem_ptr(dst, coord), in + (((gr * gc_n + gc) * tm + i) * tn + j) * (int64_t)esize,
                 (size_t)esize);
        }
    }
}

/* ---- gather backward (adjoint of the gather) -------------------------- */

void orc_tile_gather_backward(const orc_array* grad_out, const int32_t* indices, int64_t n_indices,
                              const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                              const int64_t* a_shape, double* acc, double* abs_sum, int64_t* count) {
  const int rank = grad_out->rank;
  const int64_t T = tile_shape[axis];
  const int64_t n_tiles = T > 0 ? n_indices / T : 0;
  int64_t ts[4], as4[4];
  shape4(tile_shape, rank, ts);
  shape4(a_shape, rank, as4);
  int64_t c[4];
  for (int64_t t = 0; t < n_tiles; ++t)
    for (c[0] = 0; c[0] < ts[0]; ++c[0])
      for (c[1] = 0; c[1] < ts[1]; ++c[1])
        for (c[2] = 0; c[2] < ts[2]; ++c[2])
          for (c[3] = 0; c[3] < ts[3]; ++c[3]) {
            int64_t o[4], s[4] = {0, 0, 0, 0};
            for (int d = 0; d < 4; ++d) o[d] = c[d];
            o[axis] += t * T;
            int valid = 1;
            for (int d = 0; d < rank; ++d) {
              s[d] = d == axis ? offset[axis] + (int64_t)indices[o[axis]] : offset[d] + o[d];
              if (s[d] < 0 || s[d] >= a_shape[d]) valid = 0;
            }
            if (!valid) continue;
            const char* gp = elem_ptr(grad_out, o);
            double g;
            if (grad_out->esize == 4) {
              float f;
              memcpy(&f, gp, 4);
              g = (double)f;
            } else {
              memcpy(&g, gp, 8);
            }
            int64_t lin = 0; /* row-major position of s in a's shape */
            for (int d = 0; d < 4; ++d) lin = lin * as4[d] + s[d];
            acc[lin] += g;
            abs_sum[lin] += g < 0 ? -g : g;
            count[lin] += 1;
          }
}

/* ---- tile windows with a step ----------------------------------------- */

void orc_tile_copy_windows(const orc_array* src, int64_t tm, int64_t tn, int64_t step_rows,
                           int64_t step_cols, int64_t origin_row, int64_t origin_col, void* tiles_out) {
  const int64_t M = src->shape[0], N = src->shape[1];
  const int64_t gr_n = orc_tile_grid(M, origin_row, step_rows);
  const int64_t gc_n = orc_tile_grid(N, origin_col, step_cols);
  const size_t es = (size_t)src->esize;
  char* out = (char*)tiles_out;
  for (int64_t gr = 0; gr < gr_n; ++gr)
    for (int64_t gc = 0; gc < gc_n; ++gc) {
      const int64_t R = origin_row + gr * step_rows, C = origin_col + gc * step_cols;
      for (int64_t i = 0; i < tm; ++i)
        for (int64_t j = 0; j < tn; ++j) {
          char* dst = out + (((gr * gc_n + gc) * tm + i) * tn + j) * (int64_t)es;
          const int64_t r = R + i, col = C + j;
          if (r >= 0 && r < M && col >= 0 && col < N) {
            const int64_t coord[2] = {r, col};
            memcpy(dst, elem_ptr(src, coord), es);
          } else {
            memset(dst, 0, es);
          }
        }
    }
}

void orc_tile_store_windows(const void* tiles_in, int32_t esize, int64_t tm, int64_t tn,
                            int64_t step_rows, int64_t step_cols, int64_t origin_row,
                            int64_t origin_col, orc_array* dst) {
  const int64_t M = dst->shape[0], N = dst->shape[1];
  const int64_t gr_n = orc_tile_grid(M, origin_row, step_rows);
  const int64_t gc_n = orc_tile_grid(N, origin_col, step_cols);
  const char* in = (const char*)tiles_in;
  for (int64_t gr = 0; gr < gr_n; ++gr)
    for (int64_t gc = 0; gc < gc_n; ++gc) {
      const int64_t R = origin_row + gr * step_rows, C = origin_col + gc * step_cols;
      for (int64_t i = 0; i < tm; ++i)
        for (int64_t j = 0; j < tn; ++j) {
          const int64_t r = R + i, col = C + j;
          if (r < 0 || r >= M || col < 0 || col >= N) continue;
          const int64_t coord[2] = {r, col};
          memcpy(elem_ptr(dst, coord), in + (((gr * gc_n + gc) * tm + i) * tn + j) * (int64_t)esize,
                 (size_t)esize);
        }
    }
}

/* ---- ragged varlen 3-D tiles ------------------------------------------ */

int64_t orc_ragged_schedule(const int64_t* seq_lens, int64_t n_seqs, int32_t bm_seq,
                            int32_t middle_dim, uint32_t* ragged_idx, uint32_t* dynamic_dim,
                            uint32_t* middle_idx) {
  int64_t k = 0, start = 0;
  for (int64_t s = 0; s < n_seqs; ++s) {
    const int64_t L = seq_lens[s];
    const int64_t n_u = (L + bm_seq - 1) / bm_seq;
    for (int64_t u = 0; u < n_u; ++u)
      for (int32_t m = 0; m < middle_dim; ++m) {
        if (ragged_idx) {
          const int64_t rem = L - u * bm_seq;
          ragged_idx[k] = (uint32_t)(start + u * bm_seq);
          dynamic_dim[k] = (uint32_t)(rem < bm_seq ? rem : bm_seq);
          middle_idx[k] = (uint32_t)m;
        }
        ++k;
      }
    start += L;
  }
  return k;
}

void orc_ragged_tile_load(const void* X, int32_t esize, int64_t total_rows, int32_t middle_dim,
                          int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                          const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                          const uint32_t* middle_idx, int64_t n_tiles, void* tiles_out) {
  const int32_t bm_seq = BM / group;
  const int64_t heads = (int64_t)middle_dim * group; /* X viewed as (rows, heads, depth) */
  const char* x = (const char*)X;
  char* out = (char*)tiles_out;
  for (int64_t k = 0; k < n_tiles; ++k) {
    const int64_t ri = ragged_idx[k], dyn = dynamic_dim[k], mi = middle_idx[k];
    for (int32_t s = 0; s < bm_seq; ++s)
      for (int32_t g = 0; g < group; ++g)
        for (int32_t c = 0; c < BN; ++c) {
          char* dst = out + ((k * BM + (int64_t)s * group + g) * BN + c) * (int64_t)esize;
          const int64_t row = ri + s, head = mi * group + g, col = (int64_t)col0 + c;
          if (s < dyn && row < total_rows && col < depth && mi < middle_dim)
            memcpy(dst, x + ((row * heads + head) * depth + col) * (int64_t)esize, (size_t)esize);
          else
            memset(dst, 0, (size_t)esize);
        }
  }
}

/* ---- ragged varlen 3-D store ------------------------------------------ */

void orc_ragged_tile_store(const void* tiles_in, int32_t esize, int64_t total_rows, int32_t middle_dim,
                           int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                           const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                           const uint32_t* middle_idx, int64_t n_tiles, void* X) {
  const int32_t bm_seq = BM / group;
  const int64_t heads = (int64_t)middle_dim * group; /* X viewed as (rows, heads, depth) */
  const char* in = (const char*)tiles_in;
  char* x = (char*)X;
  for (int64_t k = 0; k < n_tiles; ++k) {
    const int64_t ri = ragged_idx[k], dyn = dynamic_dim[k], mi = middle_idx[k];
    for (int32_t s = 0; s < bm_seq; ++s)
      for (int32_t g = 0; g < group; ++g)
        for (int32_t c = 0; c < BN; ++c) {
          const int64_t row = ri + s, head = mi * group + g, col = (int64_t)col0 + c;
          if (s < dyn && row < total_rows && col < depth && mi < middle_dim)
            memcpy(x + ((row * heads + head) * depth + col) * (int64_t)esize,
                   in + ((k * BM + (int64_t)s * group + g) * BN + c) * (int64_t)esize, (size_t)esize);
        }
  }
}

/* ---- block-scaled GEMM reference -------------------------------------- */

double orc_decode_lowp(uint8_t code, int32_t fmt) {
  int s, e, m, ebits, mbits, bias;
  if (fmt == ORC_LP_E4M3) {
    ebits = 4, mbits = 3, bias = 7;
  } else if (fmt == ORC_LP_E5M2) {
    ebits = 5, mbits = 2, bias = 15;
  } else {
    ebits = 2, mbits = 1, bias = 1;
    code &= 0xF;
  }
  s = (code >> (ebits + mbits)) & 1;
  e = (code >> mbits) & ((1 << ebits) - 1);
  m = code & ((1 << mbits) - 1);
  const double sign = s ? -1.0 : 1.0;
  if (fmt == ORC_LP_E4M3 && e == 15 && m == 7) return NAN;
  if (fmt == ORC_LP_E5M2 && e == 31) return m == 0 ? sign * INFINITY : NAN;
  if (e == 0) return sign * ldexp((double)m, 1 - bias - mbits); /* subnormal: m / 2^mbits * 2^(1 - bias) */
  return sign * ldexp((double)((1 << mbits) + m), e - bias - mbits);
}

double orc_decode_scale(uint8_t code, int32_t fmt) {
  if (fmt == ORC_SC_E8M0) return code == 0xFF ? NAN : ldexp(1.0, (int)code - 127);
  return orc_decode_lowp(code, ORC_LP_E4M3);
}

/* element k of a row of low-precision values */
static double lowp_at(const uint8_t* row, int64_t k, int32_t fmt) {
  if (fmt == ORC_LP_E2M1) {
    const uint8_t byte = row[k / 2];
    return orc_decode_lowp((uint8_t)(k % 2 == 0 ? byte & 0xF : byte >> 4), fmt);
  }
  return orc_decode_lowp(row[k], fmt);
}

void orc_gemm_scaled(const uint8_t* A, int32_t a_fmt, int64_t lda_bytes, const uint8_t* a_scale,
                     int64_t lds_a, const uint8_t* Bt, int32_t b_fmt, int64_t ldb_bytes,
                     const uint8_t* b_scale, int64_t lds_b, int32_t s_fmt, const float* acc,
                     int64_t ldacc, int64_t M, int64_t N, int64_t K, int64_t block, double* C) {
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double sum = acc ? (double)acc[m * ldacc + n] : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double a = lowp_at(A + m * lda_bytes, k, a_fmt) * orc_decode_scale(a_scale[m * lds_a + k / block], s_fmt);
        const double b = lowp_at(Bt + n * ldb_bytes, k, b_fmt) * orc_decode_scale(b_scale[n * lds_b + k / block], s_fmt);
        sum += a * b;
      }
      C[m * N + n] = sum;
    }
}

/* ---- bounded GEMM reference ------------------------------------------- */

double orc_bf16_to_f64(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

void orc_gemm_f64(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, double* C64,
                  int64_t ldc, int64_t M, int64_t N, int64_t K) {
  for (int64_t r = 0; r < M; ++r)
    for (int64_t c = 0; c < N; ++c) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k)
        acc += orc_bf16_to_f64(A[r * lda + k]) * orc_bf16_to_f64(B[k * ldb + c]);
      C64[r * ldc + c] = acc;
    }
}

void orc_gemm_sample_f64(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                         int64_t K, const int64_t* rows, const int64_t* cols, int64_t n,
                         double* out) {
  for (int64_t i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
      acc += orc_bf16_to_f64(A[rows[i] * lda + k]) * orc_bf16_to_f64(B[k * ldb + cols[i]]);
    out[i] = acc;
  }
}
