/*
 * stg.h -- C ABI of libstg, bounds-checked tile movement between global memory
 * and tiles on AMD Instinct MI355X (gfx950), plus the bounded-edge GEMM that
 * consumes such tiles.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Indices and coordinates are 0-based (as on the Warp, Tylo.jl and Mojo
 *   pages; the cuTile.jl pages count from 1).  Strides are in elements.
 * - Every data pointer (tensor data, indices, masks, tile buffers, ragged
 *   triples) is a DEVICE pointer on the current HIP device.  Small parameter
 *   arrays (tile_shape, offset, sequence lengths) are HOST pointers.
 * - The caller owns every buffer.  The library never allocates or frees
 *   memory and never synchronises (kernel tracing, when switched on, keeps a
 *   pool of HIP events): work is enqueued on `stream` (a hipStream_t passed as
 *   void*, NULL = the default stream) and the caller synchronises, just as the
 *   caller of an asynchronous tile copy synchronises producers and consumers
 *   (Tylo.jl Boundary tiles, "Copy completion and buffer reuse").
 * - Return value: STG_OK (0) on success, otherwise an stg_status code; the
 *   message of the last failure on the calling thread is stg_last_error().
 *   Nothing is enqueued when an argument check fails.  No C++ exception
 *   crosses this boundary.
 * - Out-of-range indices and coordinates are DEFINED behaviour: loads read
 *   zero (or the padding value), stores skip the element.  They never form an
 *   address outside the logical extent.  Undefined, and not checked: two
 *   active scatter lanes with the same destination, and output storage that
 *   overlaps an input or itself.
 * - Data movement copies element bits; no floating-point arithmetic touches
 *   them, so NaN payloads and -0.0 are preserved bit-exactly.
 */
#ifndef STG_H
#define STG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STG_F32 = 0,
  STG_BF16 = 1,
  STG_F16 = 2,
  STG_I32 = 3,
  STG_U8 = 4,
  STG_F64 = 5,
  STG_I64 = 6
} stg_dtype;

typedef enum {
  STG_OK = 0,
  STG_ERR_INVALID = 1,     /* null pointer, negative size, length mismatch, bad rank/axis ... */
  STG_ERR_UNSUPPORTED = 2, /* dtype or layout the entry point does not handle */
  STG_ERR_RANGE = 3,       /* a size or byte range exceeds what the kernels address */
  STG_ERR_LAUNCH = 4       /* the HIP launch itself failed */
} stg_status;

/* A strided device array: the logical extent `shape` of a (possibly larger)
 * allocation.  rank is 1..4; entries past rank are ignored.  Strides are in
 * elements and must be >= 0.  Every entry point rejects with STG_ERR_RANGE a
 * descriptor with an extent or stride above 2^40 or more than 2^48 elements. */
typedef struct {
  void* data;
  int32_t dtype; /* stg_dtype */
  int32_t rank;
  int64_t shape[4];
  int64_t stride[4];
} stg_tensor;

/* Library version (major*10000 + minor*100 + patch). */
int stg_version(void);

/* Message for the last failing call on this thread ("" if none). */
const char* stg_last_error(void);

/* Number of tiles of size `tile` whose origins origin, origin+tile, ... start
 * before `extent`: ceil((extent - origin) / tile), or 0 when origin >= extent
 * (cuTile.jl Memory, "Tile windows": the host-side window count is a ceiling
 * division; Tylo.jl Boundary tiles, "Accumulator stores and GEMM": ceiling
 * division for the output grid and the K loop).  Returns -1 if tile <= 0. */
int64_t stg_tile_grid(int64_t extent, int64_t origin, int64_t tile);

/* Indexed tile gather along one axis (Warp, warp.tile_load_indexed:
 * description, parameters `indices`, `shape`, `offset`, `axis`).
 *
 * Tiles of shape tile_shape[0..rank) are stacked along `axis` in `out`: tile t
 * uses indices[t*T .. t*T+T), T = tile_shape[axis], so n_indices must be a
 * multiple of T and out->shape must equal tile_shape except
 * out->shape[axis] == n_indices.  For every out coordinate o:
 *   s[d]    = offset[d] + o[d]                  (d != axis)
 *   s[axis] = offset[axis] + indices[o[axis]]
 *   out[o]  = (0 <= s[d] < a->shape[d] for all d) ? a[s] : 0
 * so -1 works as a padding sentinel.  Every coordinate is checked against
 * both bounds before an address is formed.
 *   a, out      rank 1..4, same dtype; out must not overlap a.
 *   indices     device int32[n_indices].
 *   tile_shape  host int64[rank], entries >= 1.
 *   offset      host int64[rank] (may be NULL = all zero); any sign.
 * Each workgroup stages its slice of the index tile in LDS (the page keeps the
 * index tile in shared memory). */
int tile_gather(const stg_tensor* a, const int32_t* indices, int64_t n_indices,
                const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                const stg_tensor* out, void* stream);

/* Masked gather with a padding value (cuTile.jl Memory: gather with a
 * per-element mask and padding_value for masked-out elements).
 * As tile_gather, except out[o] = padding when mask[o[axis]] == 0 or any
 * coordinate is out of range; one mask byte per index (nonzero = true), so a
 * mask entry applies to the whole slice gathered by that index.  mask may be
 * NULL (all true).  padding_value is converted to the element type by rounding
 * to nearest even (floats; infinities on overflow) or by truncation toward zero
 * (integers; STG_ERR_INVALID if not representable). */
int tile_gather_masked(const stg_tensor* a, const int32_t* indices, const uint8_t* mask,
                       int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                       int32_t axis, double padding_value, const stg_tensor* out,
                       void* stream);

/* Masked scatter (cuTile.jl Memory: scatter writes only where the mask is
 * true; "Sparse views": partially out-of-bounds stores clip and conflicting
 * stores are undefined).  The inverse of tile_gather_masked: for every
 * coordinate o of `tile` (shape as `out` of the gather) with
 * mask[o[axis]] != 0 and s fully in range, a[s] = tile[o].  Nothing else in
 * `a` is written.  Two active elements with the same destination: undefined
 * (not checked; with the environment variable STG_DEBUG set to anything but
 * "0", the call first synchronizes `stream`, checks on the host that no two
 * active indices in range along `axis` are equal, and fails with
 * STG_ERR_INVALID if they are; that synchronization rules the debug mode out
 * under stream capture).
 * Active rows of each workgroup are compacted with wavefront ballots before
 * the copy, so inactive rows cost neither reads nor writes. */
int tile_scatter_masked(const stg_tensor* a, const int32_t* indices, const uint8_t* mask,
                        int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                        int32_t axis, const stg_tensor* tile, void* stream);

/* Backward of tile_gather (Warp, warp.tile_load_indexed, description: the
 * load is differentiable, and its backward adds the output gradient into
 * a.grad at each location the forward read, with atomic adds).
 * grad_out has the shape of tile_gather's `out` for the same indices,
 * tile_shape, offset and axis; for every coordinate o of grad_out whose source
 * coordinate s (as in tile_gather) is in range:
 *   a_grad[s] += grad_out[o]
 * Out-of-range sources contribute nothing; repeated indices add up, in an
 * unspecified order (the sum is exact up to fp rounding of that order).
 * a_grad and grad_out are STG_F32 or STG_F64 (else STG_ERR_UNSUPPORTED) of one
 * dtype.  Other arguments, checks and errors as for tile_gather.
 *
 * Two executions, same result up to summation order:
 *  - workspace == NULL: every term is a hardware float atomic add into a_grad
 *    (a_grad must be device memory from hipMalloc, coarse-grained; the
 *    hardware add may flush subnormal values).
 *  - workspace != NULL: a device buffer of at least
 *    tile_gather_backward_workspace(...) bytes, 256-byte aligned, owned by the
 *    caller and not used by anything else until the work completes; for the
 *    row layout (gather axis not the last, unit last-dimension strides) the
 *    terms are grouped by destination row and each row of a_grad is summed and
 *    written once, without float atomics -- except for rows that take more
 *    than 64 terms, whose segment is split into pieces summed in parallel
 *    and added with the same hardware float atomics (STG_ERR_INVALID if the buffer is
 *    too small; STG_ERR_RANGE with 2^31 - 2^20 or more destination rows or terms, or
 *    when the per-4096-term bucket-count table would reach 2^31 entries).  The
 *    buffer holds about 8 bytes per destination row and 12 per term.  For
 *    any other layout the workspace is not used. */
int tile_gather_backward(const stg_tensor* a_grad, const int32_t* indices, int64_t n_indices,
                         const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                         const stg_tensor* grad_out, void* workspace, int64_t workspace_bytes,
                         void* stream);

/* Workspace bytes tile_gather_backward's grouped execution needs for a_grad's
 * layout, n_indices indices and tile_shape along axis (0 when the layout is
 * not the row layout, which always runs on atomics); a negative status code on
 * invalid arguments.  Host only. */
int64_t tile_gather_backward_workspace(const stg_tensor* a_grad, int64_t n_indices,
                                       const int64_t* tile_shape, int32_t axis);

/* tile_gather_backward without a caller workspace, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, semantics and errors as
 * tile_gather_backward with a workspace, except that the grouped execution's
 * scratch lives in a static device array of the library holding
 * STG_STATIC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, kept until the
 * process ends; a call needing more (tile_gather_backward_workspace(...) >
 * STG_STATIC_SCRATCH_BYTES, about 4M terms onto 1M rows) returns
 * STG_ERR_RANGE and enqueues nothing.  Layouts that take no workspace run on
 * float atomics as in tile_gather_backward.  The call allocates and frees
 * nothing.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (two streams, or two host threads without ordering) race and
 * give undefined results.  `stream` must belong to the current device
 * (STG_ERR_INVALID otherwise, before anything is enqueued). */
#define STG_STATIC_SCRATCH_BYTES (64ll << 20)
int tile_gather_backward_static(const stg_tensor* a_grad, const int32_t* indices, int64_t n_indices,
                                const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                                const stg_tensor* grad_out, void* stream);

/* Boundary-tile copy with zero fill (Tylo.jl Boundary tiles: opening section,
 * "A concrete edge"; cuTile.jl Memory, "Bounds checking": loads pad).
 * src is rank 2, logical (M, N), any strides (leading stride need not be
 * aligned).  The tiles of a grid based at (origin_row, origin_col) -- either may
 * be negative -- with step equal to the tile shape, G_r = stg_tile_grid(M,
 * origin_row, tile_rows) by G_c = stg_tile_grid(N, origin_col, tile_cols),
 * are written densely to tiles_out, row-major (G_r, G_c, tile_rows, tile_cols):
 *   tiles_out[gr][gc][i][j] = (0 <= R+i < M and 0 <= C+j < N) ? src[R+i][C+j] : 0
 * with (R, C) = (origin_row + gr*tile_rows, origin_col + gc*tile_cols).
 * tiles_out is a device buffer of G_r*G_c*tile_rows*tile_cols elements of
 * src's dtype, not overlapping src. */
int tile_copy_bounded(const stg_tensor* src, int64_t tile_rows, int64_t tile_cols,
                      int64_t origin_row, int64_t origin_col, void* tiles_out, void* stream);

/* Clipped tile store (Tylo.jl Boundary tiles, "Accumulator stores and GEMM":
 * invalid coordinates are suppressed and padding outside the logical extent
 * is left unchanged; cuTile.jl Memory, "Bounds checking": stores clip).
 * The inverse of tile_copy_bounded over the same grid: for valid (i, j) only,
 * dst[R+i][C+j] = tiles_in[gr][gc][i][j].  Elements outside the logical
 * extent of dst (for example the columns between N and the row stride) are
 * never written. */
int tile_store_clipped(const void* tiles_in, int64_t tile_rows, int64_t tile_cols,
                       int64_t origin_row, int64_t origin_col, const stg_tensor* dst,
                       void* stream);

/* Tile windows with a step, and the unchecked full-tile path.
 * (cuTile.jl Memory, "Tile windows": eachtile's step sets the tile origins,
 * not the element stride inside a tile -- windows overlap when step < shape
 * and leave gaps when step > shape -- and there are cld(extent, step) of them;
 * cuTile.jl Memory, "Bounds checking": check_bounds=false promises that every
 * element of the tile is in the array and drops load padding; Tylo.jl Boundary
 * tiles, "Accumulator stores and GEMM": bounds=false keeps the full-tile path.)
 * Window (gr, gc) has origin (R, C) = (origin_row + gr*step_rows, origin_col +
 * gc*step_cols) for gr < G_r = stg_tile_grid(M, origin_row, step_rows) and
 * gc < G_c = stg_tile_grid(N, origin_col, step_cols); tiles are (G_r, G_c,
 * tile_rows, tile_cols) row-major as for tile_copy_bounded, which is the case
 * step = shape.
 *   tile_copy_windows:  tiles_out[gr][gc][i][j] = in range ? src[R+i][C+j] : 0
 *   tile_store_windows: dst[R+i][C+j] = tiles_in[gr][gc][i][j] for in-range
 *                       (R+i, C+j) only; where windows overlap, conflicting
 *                       stores are undefined (equal values are fine).
 * check_bounds != 0: bounded semantics as above.  check_bounds == 0: the
 * caller promises that every window lies inside the logical extent; the
 * promise is verified on the host from the dimensions and a broken promise
 * returns STG_ERR_INVALID (nothing is launched).  Whenever every window lies
 * inside -- promised or not, and for tile_copy_bounded / tile_store_clipped
 * too -- the launch uses the unchecked kernel instance, whose vectors need no
 * validity test.  step_rows, step_cols >= 1 (else STG_ERR_INVALID); other
 * arguments, ownership and errors as for tile_copy_bounded / tile_store_clipped. */
int tile_copy_windows(const stg_tensor* src, int64_t tile_rows, int64_t tile_cols, int64_t step_rows,
                      int64_t step_cols, int64_t origin_row, int64_t origin_col, int32_t check_bounds,
                      void* tiles_out, void* stream);
int tile_store_windows(const void* tiles_in, int64_t tile_rows, int64_t tile_cols, int64_t step_rows,
                       int64_t step_cols, int64_t origin_row, int64_t origin_col, int32_t check_bounds,
                       const stg_tensor* dst, void* stream);

/* Host helper: the tiles that cover a packed varlen batch for ragged_tile_load.
 * Sequence s (length seq_lens[s] >= 0) starts at row cu[s] = sum of the earlier
 * lengths; for u in [0, ceil(L_s/bm_seq)) and m in [0, middle_dim), in that
 * nesting order, one tile (ragged_idx, dynamic_dim, middle_idx) =
 * (cu[s] + u*bm_seq, min(bm_seq, L_s - u*bm_seq), m).
 * All pointers are HOST pointers; the three outputs may be NULL to only count.
 * *n_tiles receives the count.  STG_ERR_RANGE if a row index exceeds 2^32-1. */
int ragged_tile_schedule(const int64_t* seq_lens, int64_t n_seqs, int32_t bm_seq,
                         int32_t middle_dim, uint32_t* ragged_idx, uint32_t* dynamic_dim,
                         uint32_t* middle_idx, int64_t* n_tiles);

/* Ragged varlen 3-D tile load (Mojo, layout.tma_async.RaggedTMA3DTile:
 * description, parameters BM, BN, middle_dim, group, comptime BM_seq, and the
 * per-copy arguments ragged_idx, dynamic_dim, middle_idx).
 * src is contiguous (total_rows, middle_dim*group, depth) of `dtype`; with
 * group > 1 it is the 4-D view (rows, middle_dim, group, depth).  The page's
 * merged selector coordinate (ragged_idx + dynamic_dim)*middle_dim + middle_idx
 * addresses, relative to a descriptor based BM_seq rows in front of the data,
 * exactly the rows ragged_idx .. ragged_idx+dynamic_dim-1 of head middle_idx;
 * this entry point reads those rows directly, so nothing needs to be
 * allocated in front of src.  With BM_seq = BM / group, for tile k,
 * s < BM_seq, g < group, c < BN:
 *   tiles_out[k][s*group + g][c] =
 *       (s < dynamic_dim[k] and ragged_idx[k]+s < total_rows and col0+c < depth)
 *       ? src[ragged_idx[k]+s][middle_idx[k]*group + g][col0+c] : 0
 * Host-checked requirements (else STG_ERR_INVALID): group >= 1, BM % group == 0,
 * BN >= 1, 0 <= col0 < depth, middle_dim >= 1.  The triples live on the device
 * and are not checked on the host; instead the kernel guards them: a
 * dynamic_dim above BM_seq simply makes every row valid, and a middle_idx >=
 * middle_dim yields an all-zero tile without reading src.  Rows that fail the
 * predicate are written as zero and never read.  The three triple arrays are
 * device uint32[n_tiles]; tiles_out is a device buffer (n_tiles, BM, BN). */
int ragged_tile_load(const void* src, int32_t dtype, int64_t total_rows, int32_t middle_dim,
                     int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                     const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                     const uint32_t* middle_idx, int64_t n_tiles, void* tiles_out,
                     void* stream);

/* Ragged varlen 3-D tile store, the store direction of the same descriptor
 * (Mojo, layout.tma_async.RaggedTMA3DTile: async_copy_from_col and
 * async_copy_batched copy a tile from shared memory to global memory -- only
 * dynamic_dim rows (sequence positions when group > 1) at ragged_idx for head
 * middle_idx, with the part of the box that overhangs the array masked off).
 * tiles_in is a device buffer (n_tiles, BM, BN) of `dtype`; dst is contiguous
 * (total_rows, middle_dim*group, depth).  With BM_seq = BM / group, for tile
 * k, s < BM_seq, g < group, c < BN:
 *   if s < dynamic_dim[k] and ragged_idx[k]+s < total_rows and col0+c < depth
 *      and middle_idx[k] < middle_dim:
 *     dst[ragged_idx[k]+s][middle_idx[k]*group + g][col0+c] = tiles_in[k][s*group + g][c]
 * No other element of dst is written (tile rows at or past dynamic_dim, columns
 * past depth, rows past total_rows, a middle_idx >= middle_dim).  Two tiles
 * that write the same element: undefined (the schedule of
 * ragged_tile_schedule never does).  Host checks, triples and error codes as
 * for ragged_tile_load; tiles_in must not overlap dst. */
int ragged_tile_store(const void* tiles_in, int32_t dtype, int64_t total_rows, int32_t middle_dim,
                      int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                      const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                      const uint32_t* middle_idx, int64_t n_tiles, void* dst, void* stream);

/* Block-scaled GEMM (cuTile.jl Operations, muladd_scaled: (a . a_scale) *
 * (b . b_scale) + acc, each scale element multiplying a contiguous block of
 * `block` = K / K_s values along K of its operand; operands f8e4m3fn, f8e5m2
 * or f4e2m1fn, scales f8e8m0fnu or f8e4m3fn, f32 accumulator; reinterpret:
 * FP4 values travel two per byte).
 *   A        (M, K) operand codes, K contiguous, row stride lda BYTES.
 *   Bt       B given K-major: (N, K), K contiguous, row stride ldb BYTES.
 *            e2m1 packs two values per byte, element k at byte k/2, the even
 *            element in the low nibble.
 *   a_scale  (M, K/block) scale bytes, row stride lds_a; b_scale (N, K/block),
 *            row stride lds_b; scale_fmt STG_SC_E8M0 (2^(e-127)) or STG_SC_E4M3.
 *   acc      (M, N) f32, row stride ldacc, or NULL for zero; C (M, N) f32, row
 *            stride ldc (C may be acc: the sum is written in place).
 *   C[m][n] = acc[m][n] + sum_k A(m,k) sa(m,k/block) B(k,n) sb(n,k/block)
 * in fp32 accumulation.  Only C[m][n] with m < M, n < N is written.
 * Requirements: block >= 1 and K a multiple of block; fp4 rows hold
 * ceil(K/2) bytes.  Errors as for gemm_bounded.
 * Two executions, chosen from the arguments:
 *  - e8m0 scales, block 32 times a power of two, and fp8 x fp8 or fp4 x fp4
 *    operands run on the gfx950 scaled MFMA, which applies one e8m0 scale per
 *    32 K values itself.  Its sums are not fp32-exact: within each group of
 *    8 consecutive K values, products smaller than 2^-13 of the group's
 *    largest are cut toward zero to that grid before the group is added
 *    (error below 7 * 2^-13 of the group's largest product, at most
 *    7 * 2^-13 * sum |terms| overall, plus fp32 accumulation of the group
 *    sums); fp4 products never span that range inside a group.  With 32-value
 *    blocks, both scale matrices 16-byte aligned and lds_a, lds_b multiples of
 *    16, a faster scale path is taken (fp4 about 6% faster).
 *  - every other case (e4m3 scales, blocks such as 16 or 48, fp4 x fp8 pairs)
 *    multiplies each value by its scale while staging -- exact in bf16 for
 *    e4m3 scales, and for e8m0 scales while value x 2^(e-127) is a multiple
 *    of 2^-133 (bf16's subnormal step) below 2^128: scale bytes 3..246 with
 *    e4m3 operands, 10..239 with e5m2, 0..252 with e2m1 -- and sums with the
 *    bf16 MFMA (which keeps subnormal inputs) in fp32: the result is within
 *    fp32 accumulation rounding of the exact sum.
 */
typedef enum { STG_LP_E4M3 = 0, STG_LP_E5M2 = 1, STG_LP_E2M1 = 2 } stg_lowp_format;
typedef enum { STG_SC_E8M0 = 0, STG_SC_E4M3 = 1 } stg_scale_format;
int gemm_scaled(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C,
                int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/* gemm_scaled with a caller-owned workspace (the same product, cuTile.jl
 * Operations, muladd_scaled).  Where the second execution above applies and
 * gemm_scaled_workspace returns n > 0 bytes, a workspace of at least n bytes
 * (device memory, 256-byte aligned, owned by the caller, unused once the
 * stream has run the call) makes the call decode each operand once into
 * bf16 matrices there -- the same exact scaled values -- and multiply them
 * with the bf16 GEMM of gemm_bounded in fp32: the result is again within fp32
 * accumulation rounding of the exact sum (the summation order differs).
 * Without a workspace (NULL, or where the query returns 0) this is
 * gemm_scaled.  STG_ERR_INVALID for a workspace smaller than the query's
 * bytes or not 256-byte aligned; otherwise errors as for gemm_scaled.  Calls
 * that share a workspace and overlap in time race on it. */
int gemm_scaled_ws(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                   const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                   int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                   int64_t workspace_bytes, void* stream);

/* Workspace bytes for gemm_scaled_ws: 0 where the call takes the scaled MFMA
 * or decoding first does not pay (M or N at most 256, K = 0, or sizes past
 * the bf16 GEMM's limits); otherwise the bytes of the decoded operands, bf16
 * (M, ceil(K/16)*16) and (K, ceil(N/64)*64), each rounded up to 256.  A
 * negative value is minus an error code (unknown formats: STG_ERR_UNSUPPORTED;
 * negative sizes, block < 1, K not a multiple of block: STG_ERR_INVALID). */
int64_t gemm_scaled_workspace(int32_t a_fmt, int32_t b_fmt, int32_t scale_fmt, int64_t block, int64_t M,
                              int64_t N, int64_t K);

/* Bounded-edge GEMM C = A . B (cuTile.jl Operations, muladd: bf16 operands
 * accumulate in f32; Tylo.jl Boundary tiles, "Accumulator stores and GEMM":
 * ceiling-division output grid and K loop, zero-filled edge stages, and an
 * epilogue that converts the f32 accumulator to the destination type and
 * suppresses invalid coordinates).
 *   A  bf16 (M, K) row-major, row stride lda >= K (any alignment).
 *   B  bf16 (K, N) row-major, row stride ldb >= N (any alignment).
 *   C  (M, N) row-major, row stride ldc >= N, c_dtype STG_BF16 (f32 rounded to
 *      nearest even) or STG_F32.  Only C[r][c] with r < M, c < N is written.
 * M, N, K >= 0; K == 0 writes zeros.  Summation order is unspecified (results
 * match an exact reference to accumulation rounding); it does not depend on
 * the strides: rows that start 16-byte aligned (lda, ldb multiples of 8, A
 * and B 16-byte aligned) take a faster kernel that gives the same bits. */
int gemm_bounded(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, int32_t c_dtype, void* stream);

/* Kernel tracing, for measurement.  While enabled (on != 0) on the calling
 * thread, every kernel the library launches from that thread records a
 * start/stop hipEvent pair that is part of its own dispatch
 * (hipExtLaunchKernel), so the pair times the kernel alone, without the queue
 * gaps between dependent launches.  Returns the previous setting.  Tracing
 * creates events lazily and keeps them for reuse until the process ends. */
int stg_trace_enable(int on);

/* After the caller has synchronised the streams the traced kernels ran on:
 * writes up to `cap` records, oldest first -- names[i] (a static string naming
 * the entry point and, where it launches more than one kernel, the kernel) and
 * ms[i] (milliseconds, -1 if that kernel had not completed) -- then clears the
 * log (records beyond `cap` are dropped).  Returns the number written, or a
 * negative stg_status on bad arguments. */
int stg_trace_read(int cap, const char** names, float* ms);

#ifdef __cplusplus
}
#endif
#endif /* STG_H */
