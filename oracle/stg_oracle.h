/*
 * stg_oracle.h -- plain, single-threaded CPU oracle for bounds-checked tile
 * movement and the bounded-edge GEMM that consumes the tiles.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no source with the HIP
 * path: its own header, its own types, its own conversions.
 *
 * Every function is a direct transcription of the definition it cites, with
 * no blocking, fusion or reordering.  Coordinates are int64; element data is
 * moved as raw bytes (memcpy of the element size) and never passes through a
 * floating-point register, so NaN payloads and -0.0 survive.  The GEMM sums
 * in fp64, where each bf16 product is exact.
 *
 * All indices are 0-based (the Warp, Tylo and Mojo pages are 0-based; the
 * cuTile.jl pages are 1-based and are read with 1 subtracted).
 *
 * Pins: every function here is checked by CPU tests against values the pages
 * print, closed forms, special cases that reduce to a library routine, and
 * brute force on tiny inputs written in a second, independent formulation.
 */
#ifndef STG_ORACLE_H
#define STG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A strided array of rank 1..4; strides and shape are in elements. */
typedef struct {
  void* data;
  int32_t esize; /* bytes per element: 1, 2, 4 or 8 */
  int32_t rank;
  int64_t shape[4];
  int64_t stride[4];
} orc_array;

/* Element types known to the padding conversion. */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2, ORC_I32 = 3, ORC_U8 = 4, ORC_F64 = 5, ORC_I64 = 6 };

/* Number of tile origins origin, origin+tile, ... that start before
 * `extent` (cuTile.jl Memory, "Tile windows": host-side count is a ceiling
 * division; Tylo.jl Boundary tiles, "Accumulator stores and GEMM": ceiling
 * division for the output grid and K loop).  0 when origin >= extent. */
int64_t orc_tile_grid(int64_t extent, int64_t origin, int64_t tile);

/* Round a double to the binary interchange format with `ebits` exponent bits
 * and `mbits` stored mantissa bits, to nearest with ties to even; returns the
 * bit pattern (sign bit at position ebits+mbits).  Overflow gives infinity,
 * NaN gives the canonical quiet NaN of that sign. */
uint64_t orc_round_to_format(double v, int ebits, int mbits);

/* Convert the padding value to the element type `dtype` and write its bits
 * to `out` (element-size bytes).  Integer types take the value truncated
 * toward zero.  Returns 0, or -1 when the value is not representable. */
int orc_padding_bits(double v, int dtype, void* out);

/* Indexed tile gather (Warp tile_load_indexed page, description and
 * parameters).  Tiles are stacked along `axis`: tile t uses
 * indices[t*T .. t*T+T) with T = tile_shape[axis].  For out element with
 * coordinate o (o[axis] = t*T + c[axis]):
 *   s[d]    = offset[d] + o[d]                      for d != axis
 *   s[axis] = offset[axis] + indices[o[axis]]
 *   out[o]  = all s[d] in [0, a.shape[d]) ? a[s] : 0 bits.
 * out has shape tile_shape with out.shape[axis] = n_indices. */
void orc_tile_gather(const orc_array* a, const int32_t* indices, int64_t n_indices,
                     const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                     orc_array* out);

/* Masked gather (cuTile.jl Memory, the gather call with mask and
 * padding_value).  Like orc_tile_gather, except an element is filled with
 * the padding bits `pad` when mask[o[axis]] == 0 or any coordinate is out
 * of range; one mask byte per index. */
void orc_tile_gather_masked(const orc_array* a, const int32_t* indices, const uint8_t* mask,
                            int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                            int32_t axis, const void* pad, orc_array* out);

/* Masked scatter (cuTile.jl Memory, the scatter call with mask; "Sparse
 * views": stores clip, conflicting stores are undefined).  For every tile
 * element o with mask[o[axis]] != 0 and all s[d] in range: a[s] = tile[o].
 * Nothing else is written.  Duplicate active destinations are undefined by
 * the pages; this oracle applies them in index order (last writer wins). */
void orc_tile_scatter_masked(orc_array* a, const int32_t* indices, const uint8_t* mask,
                             int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                             int32_t axis, const orc_array* tile);

/* Boundary-tile copy with zero fill (Tylo.jl Boundary tiles, opening
 * section and "A concrete edge"; cuTile.jl Memory, "Bounds checking").
 * src is rank 2 (M, N) with arbitrary strides.  For grid tile (gr, gc),
 * origin (R, C) = (origin_row + gr*TM, origin_col + gc*TN):
 *   out[gr][gc][i][j] = (0 <= R+i < M and 0 <= C+j < N) ? src[R+i][C+j] : 0 bits
 * out is dense (G_r, G_c, TM, TN) row-major, G = orc_tile_grid(...). */
void orc_tile_copy_bounded(const orc_array* src, int64_t tm, int64_t tn, int64_t origin_row,
                           int64_t origin_col, void* tiles_out);

/* Clipped tile store (Tylo.jl Boundary tiles, "Accumulator stores and
 * GEMM": invalid coordinates are suppressed and padding is left unchanged;
 * cuTile.jl Memory, "Bounds checking": stores clip).  Same grid as the copy;
 * only valid (i, j) write dst[R+i][C+j] = tiles[gr][gc][i][j]. */
void orc_tile_store_clipped(const void* tiles_in, int32_t esize, int64_t tm, int64_t tn,
                            int64_t origin_row, int64_t origin_col, orc_array* dst);

/* Backward of the indexed gather (Warp, warp.tile_load_indexed,
 * description: the load is differentiable; its backward adds the output
 * gradient into a.grad at each location the forward read, atomically).  For every coordinate o of grad_out (the gather's output
 * shape) whose source coordinate s -- as in orc_tile_gather -- is in range:
 *   acc[s] += grad_out[o];  abs_sum[s] += |grad_out[o]|;  count[s] += 1
 * Out-of-range sources contribute nothing; repeated indices add up.
 * grad_out holds float (esize 4) or double (esize 8) values; acc, abs_sum
 * and count are dense row-major arrays of a's shape a_shape[0..rank-1]
 * (rank = grad_out's), initialised by the caller (acc with a.grad's initial
 * values, abs_sum with their magnitudes, count with zeros).  The sums are in
 * fp64, in coordinate order. */
void orc_tile_gather_backward(const orc_array* grad_out, const int32_t* indices, int64_t n_indices,
                              const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                              const int64_t* a_shape, double* acc, double* abs_sum, int64_t* count);

/* Tile windows with a step (cuTile.jl Memory, "Tile windows": eachtile with
 * step per dimension controlling the tile origins, not the element stride
 * inside a tile; neighbouring windows overlap when step < shape and leave
 * gaps when step > shape; the window count is cld(extent, step)).  Window
 * (gr, gc) has origin (origin_row + gr*step_rows, origin_col + gc*step_cols);
 * G_r = orc_tile_grid(M, origin_row, step_rows), G_c likewise.  The copy is
 * the bounded copy of each window (zero outside the logical extent); with
 * step equal to the shape this is orc_tile_copy_bounded. */
void orc_tile_copy_windows(const orc_array* src, int64_t tm, int64_t tn, int64_t step_rows,
                           int64_t step_cols, int64_t origin_row, int64_t origin_col, void* tiles_out);

/* The clipped store of every window, windows taken in row-major grid order
 * (where windows overlap the later one wins here; the product leaves
 * conflicting stores undefined, as the page does for sparse views). */
void orc_tile_store_windows(const void* tiles_in, int32_t esize, int64_t tm, int64_t tn,
                            int64_t step_rows, int64_t step_cols, int64_t origin_row,
                            int64_t origin_col, orc_array* dst);

/* Ragged schedule: the tiles that cover a packed varlen batch.  Sequence s
 * of length L_s starts at row cu[s] = L_0 + ... + L_{s-1}; for u in
 * [0, ceil(L_s/bm_seq)) and m in [0, middle_dim), in lexicographic order
 * (s, u, m):  (ragged_idx, dynamic_dim, middle_idx) =
 *   (cu[s] + u*bm_seq, min(bm_seq, L_s - u*bm_seq), m).
 * Writes the triples when the output pointers are non-NULL; returns the
 * number of tiles. */
int64_t orc_ragged_schedule(const int64_t* seq_lens, int64_t n_seqs, int32_t bm_seq,
                            int32_t middle_dim, uint32_t* ragged_idx, uint32_t* dynamic_dim,
                            uint32_t* middle_idx);

/* Ragged varlen 3-D tile load (Mojo RaggedTMA3DTile page: description,
 * parameters BM/BN/middle_dim/group, comptime BM_seq, and the copy
 * arguments ragged_idx/dynamic_dim/middle_idx).  X is contiguous
 * (total_rows, middle_dim*group, depth).  With BM_seq = BM/group, for tile
 * k, s < BM_seq, g < group, c < BN:
 *   out[k][s*group + g][c] = (s < dyn and ri+s < total_rows and col0+c < depth
 *                             and mi < middle_dim)
 *                            ? X[ri+s][mi*group + g][col0+c] : 0 bits
 * out is dense (n_tiles, BM, BN). */
void orc_ragged_tile_load(const void* X, int32_t esize, int64_t total_rows, int32_t middle_dim,
                          int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                          const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                          const uint32_t* middle_idx, int64_t n_tiles, void* tiles_out);

/* Ragged varlen 3-D tile store, the store direction of the same descriptor
 * (Mojo RaggedTMA3DTile page: async_copy_from_col and async_copy_batched --
 * a copy from the shared-memory tile to global memory of dynamic_dim rows
 * (sequence positions when group > 1) at ragged_idx for head middle_idx,
 * with the part of the box that overhangs the array masked off).  tiles is
 * dense (n_tiles, BM, BN); X is contiguous (total_rows, middle_dim*group,
 * depth).  For tile k, s < BM_seq, g < group, c < BN, in tile order:
 *   if s < dyn and ri+s < total_rows and col0+c < depth and mi < middle_dim:
 *     X[ri+s][mi*group + g][col0+c] = tiles[k][s*group + g][c]
 * Every other element of X is left as it was (tiles that write the same
 * element: the later tile wins here; the product leaves that undefined). */
void orc_ragged_tile_store(const void* tiles_in, int32_t esize, int64_t total_rows, int32_t middle_dim,
                           int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                           const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                           const uint32_t* middle_idx, int64_t n_tiles, void* X);

/* Low-precision element and scale formats of block-scaled GEMM (cuTile.jl
 * Operations, muladd_scaled: a / b are f8e4m3fn, f8e5m2 or f4e2m1fn; a_scale /
 * b_scale are f8e8m0fnu or f8e4m3fn).  Decoded exactly to double from the
 * format definitions:
 *   e4m3fn  sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
 *           subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities.
 *   e5m2    sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE rules
 *           (exponent 31: infinity when m = 0, else NaN).
 *   e2m1    sign, 2 exponent bits (bias 1), 1 mantissa bit, no NaN or
 *           infinity: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   e8m0    unsigned exponent byte e: 2^(e - 127); 0xFF is NaN. */
enum { ORC_LP_E4M3 = 0, ORC_LP_E5M2 = 1, ORC_LP_E2M1 = 2 };
enum { ORC_SC_E8M0 = 0, ORC_SC_E4M3 = 1 };
double orc_decode_lowp(uint8_t code, int32_t fmt); /* fmt ORC_LP_*; e2m1 uses the low 4 bits */
double orc_decode_scale(uint8_t code, int32_t fmt); /* fmt ORC_SC_* */

/* Block-scaled GEMM (cuTile.jl Operations, muladd_scaled: (a . a_scale) *
 * (b . b_scale) + acc, each scale element multiplying a contiguous block of
 * `block` = K / K_s values along K of its operand, f32 accumulation).
 * A is (M, K) with K contiguous, row stride lda_bytes; B is given K-major as
 * Bt (N, K) = B transposed, row stride ldb_bytes.  e2m1 operands hold two
 * values per byte, element k at byte k/2, the even element in the low nibble
 * (cuTile.jl Operations, reinterpret: a UInt8 tile of N bytes is an FP4 tile
 * of 2N values).  a_scale is (M, K/block) bytes with row stride lds_a,
 * b_scale (N, K/block) with row stride lds_b.  acc is (M, N) f32 with row
 * stride ldacc, or NULL for zero.  C (M, N) dense row-major, in fp64:
 *   C[m][n] = acc[m][n] + sum_k A(m,k) sa(m, k/block) B(k,n) sb(n, k/block) */
void orc_gemm_scaled(const uint8_t* A, int32_t a_fmt, int64_t lda_bytes, const uint8_t* a_scale,
                     int64_t lds_a, const uint8_t* Bt, int32_t b_fmt, int64_t ldb_bytes,
                     const uint8_t* b_scale, int64_t lds_b, int32_t s_fmt, const float* acc,
                     int64_t ldacc, int64_t M, int64_t N, int64_t K, int64_t block, double* C);

/* Decode one bf16 bit pattern to double (exact: bf16 is the top half of
 * an IEEE binary32). */
double orc_bf16_to_f64(uint16_t h);

/* Bounded GEMM reference (cuTile.jl Operations, muladd: bf16 inputs
 * accumulate in f32 -- here in f64, where each product is exact; Tylo.jl
 * Boundary tiles, "Accumulator stores and GEMM").  A is (M, K) bf16 with row
 * stride lda, B is (K, N) bf16 with row stride ldb.  Writes
 * C64[r*ldc + c] = sum_k A[r][k] * B[k][c] in double, for r < M, c < N. */
void orc_gemm_f64(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, double* C64,
                  int64_t ldc, int64_t M, int64_t N, int64_t K);

/* Same sum for n selected output coordinates (rows[i], cols[i]). */
void orc_gemm_sample_f64(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                         int64_t K, const int64_t* rows, const int64_t* cols, int64_t n,
                         double* out);

#ifdef __cplusplus
}
#endif
#endif /* STG_ORACLE_H */
