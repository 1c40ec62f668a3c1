// Boundary-tile copy with zero fill, and the clipped store back.
//
// Semantics (Tylo.jl Boundary tiles: opening section, "A concrete edge",
// "Accumulator stores and GEMM"; cuTile.jl Memory, "Bounds checking"): a tile
// of static capacity (tile_rows, tile_cols) at origin (R, C) of a matrix with
// logical extent (M, N) -- R and C may be negative, the row stride need not be
// aligned -- reads src[R+i][C+j] where valid and zero elsewhere; the store
// writes only the valid elements and never touches padding.
//
// Vector classification follows the page's copy plan, recast for gfx950: each
// lane owns fixed 16-byte vectors of the dense tile buffer.  A vector whose
// source elements are all valid is one dwordx4 buffer load at its (often
// unaligned) byte offset -- gfx950 services unaligned dwordx4 accesses, so a
// leading dimension that is not a multiple of eight bf16 values does not force
// a slower path.  A vector with no valid element is given an offset past the
// buffer's num_records, so the same load instruction returns zeros (and the
// same store instruction is dropped) without forming an address outside the
// logical extent.  Only vectors that straddle the right or left edge take a
// per-element path.
//
// Tile windows (cuTile.jl Memory, "Tile windows"): window (gr, gc) starts at
// (r0 + gr*step_rows, c0 + gc*step_cols); the step sets only the origins, so
// windows overlap when it is below the tile shape and leave gaps above it.
// With step = shape these are the plain tile grids.
//
// Unchecked instance (cuTile.jl Memory, "Bounds checking": check_bounds=false
// is a promise that every element of the tile is in the array; Tylo.jl
// Boundary tiles: bounds=false keeps the full-tile path): when every window
// of the grid lies inside the logical extent, the host launches the CHECK =
// false instance, whose lanes load and store their vectors with no validity
// test.  The bounded entry points choose it by themselves from the
// dimensions; the window entry points take an explicit check_bounds = 0,
// whose promise is verified on the host (a broken promise is an error here,
// not an out-of-bounds access).
//
// Work mapping: a workgroup covers `rows_per_wg` rows of one tile row band and
// `tiles_per_wg` adjacent tiles along the columns, so a wavefront reads one
// contiguous source row segment (64 lanes x 16 bytes when tiles_per_wg *
// chunks_per_tile_row == 64) and writes whole 64-byte tile rows.  The buffer
// resource is rebased at the workgroup's first source row so 32-bit offsets
// cover any matrix size.
#include "stg_internal.h"

namespace stg {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;  // vectors per lane per pass (measured best with 8-row workgroups)

struct CopyParams {
  const char* m;  // element (0, 0) of the matrix (source of the copy, destination of the store)
  char* tiles;    // dense (G_r, G_c, tm, tn) buffer
  int64_t M, N;
  int64_t ld_b;  // matrix row stride in bytes
  int64_t r0, c0;
  int64_t sr, sc;  // window step (origin of window (gr, gc) = (r0 + gr*sr, c0 + gc*sc))
  int64_t G_c;
  int32_t tm, tn;
  int32_t cpt;            // 16-byte chunks per tile row
  int32_t rows_per_wg;    // rows of a tile handled by one workgroup
  int32_t tiles_per_wg;   // tiles along the column grid per workgroup
  int32_t row_blocks;     // ceil(tm / rows_per_wg)
  uint32_t n_cb;          // workgroups along the tile-column grid
  uint32_t span_magic;    // division by tiles_per_wg * cpt
  uint32_t cpt_magic;     // division by cpt
  int32_t esize;
};

// Location of item `it` of this workgroup.
struct Item {
  int64_t r, c;     // source row / first source column of the vector
  int64_t t_off;    // byte offset in the tile buffer
  bool in_tile;     // row < tm and tile column < G_c
};

__device__ __forceinline__ Item locate(const CopyParams& p, int it, int64_t gr, int rblk, int64_t gc0) {
  const int span = p.tiles_per_wg * p.cpt;
  const int rl = (int)div_small((uint32_t)it, p.span_magic);
  const int k = it - rl * span;
  const int tcol = (int)div_small((uint32_t)k, p.cpt_magic);
  const int v = k - tcol * p.cpt;
  const int i = rblk * p.rows_per_wg + rl;
  const int64_t gc = gc0 + tcol;
  Item x;
  x.in_tile = i < p.tm && gc < p.G_c;
  x.r = p.r0 + gr * p.sr + i;
  x.c = p.c0 + gc * p.sc + (int64_t)v * (16 / p.esize);
  x.t_off = (((gr * p.G_c + gc) * p.tm + i) * p.tn) * p.esize + (int64_t)v * 16;
  return x;
}

template <int ESIZE, bool CHECK>
__global__ __launch_bounds__(kThreads) void copy_bounded_kernel(CopyParams p) {
  constexpr int V = 16 / ESIZE;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t band = wg / p.n_cb;
  const int64_t gc0 = (int64_t)(wg - band * p.n_cb) * p.tiles_per_wg;
  const int64_t gr = band / p.row_blocks;
  const int rblk = (int)(band - gr * p.row_blocks);
  // rebase the buffer resource at the first valid source row of this workgroup
  int64_t base_row = p.r0 + gr * p.sr + (int64_t)rblk * p.rows_per_wg;
  base_row = base_row < 0 ? 0 : base_row >= p.M ? p.M - 1 : base_row;
  int64_t avail = (p.M - 1 - base_row) * p.ld_b + p.N * ESIZE;
  if (p.M <= 0 || p.N <= 0) base_row = 0, avail = 0;
  const char* base = p.m + base_row * p.ld_b;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(avail < (int64_t)kOOB ? avail : (int64_t)kOOB - 1));
  const int items = p.rows_per_wg * p.tiles_per_wg * p.cpt;
  for (int b0 = 0; b0 < items; b0 += kThreads * kUnroll) {
    u32x4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = b0 + u * kThreads + threadIdx.x;
      dst[u] = -1;
      v[u] = (u32x4){0, 0, 0, 0};
      if (it < items) {
        const Item x = locate(p, it, gr, rblk, gc0);
        if (!CHECK && x.in_tile) {
          dst[u] = x.t_off;
          v[u] = ld16(p.m + x.r * p.ld_b + x.c * ESIZE);
        } else if (x.in_tile) {
          dst[u] = x.t_off;
          const bool row_ok = x.r >= 0 && x.r < p.M;
          const bool full = row_ok && x.c >= 0 && x.c + V <= p.N;
          const uint32_t off = full ? (uint32_t)((x.r - base_row) * p.ld_b + x.c * ESIZE) : kOOB;
          v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          if (row_ok && !full && x.c + V > 0 && x.c < p.N) {
            const char* rowp = p.m + x.r * p.ld_b;
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const int64_t c = x.c + e;
              if (c >= 0 && c < p.N) vec_set<ESIZE>(v[u], e, load_elem<ESIZE>(rowp + c * ESIZE));
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (dst[u] >= 0) *(u32x4*)(p.tiles + dst[u]) = v[u];
  }
}

template <int ESIZE, bool CHECK>
__global__ __launch_bounds__(kThreads) void store_clipped_kernel(CopyParams p) {
  constexpr int V = 16 / ESIZE;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t band = wg / p.n_cb;
  const int64_t gc0 = (int64_t)(wg - band * p.n_cb) * p.tiles_per_wg;
  const int64_t gr = band / p.row_blocks;
  const int rblk = (int)(band - gr * p.row_blocks);
  int64_t base_row = p.r0 + gr * p.sr + (int64_t)rblk * p.rows_per_wg;
  base_row = base_row < 0 ? 0 : base_row >= p.M ? p.M - 1 : base_row;
  int64_t avail = (p.M - 1 - base_row) * p.ld_b + p.N * ESIZE;
  if (p.M <= 0 || p.N <= 0) base_row = 0, avail = 0;
  char* base = const_cast<char*>(p.m) + base_row * p.ld_b;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(avail < (int64_t)kOOB ? avail : (int64_t)kOOB - 1));
  const int items = p.rows_per_wg * p.tiles_per_wg * p.cpt;
  for (int b0 = 0; b0 < items; b0 += kThreads * kUnroll) {
    u32x4 v[kUnroll];
    Item xs[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = b0 + u * kThreads + threadIdx.x;
      xs[u].in_tile = false;
      if (it < items) {
        xs[u] = locate(p, it, gr, rblk, gc0);
        if (CHECK) {
          const bool row_ok = xs[u].r >= 0 && xs[u].r < p.M;
          xs[u].in_tile = xs[u].in_tile && row_ok && xs[u].c + V > 0 && xs[u].c < p.N;  // any valid element
        }
        if (xs[u].in_tile) v[u] = *(const u32x4*)(p.tiles + xs[u].t_off);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!xs[u].in_tile) continue;
      const Item& x = xs[u];
      if (!CHECK) {
        st16(const_cast<char*>(p.m) + x.r * p.ld_b + x.c * ESIZE, v[u]);
      } else if (x.c >= 0 && x.c + V <= p.N) {
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rs, (uint32_t)((x.r - base_row) * p.ld_b + x.c * ESIZE), 0, 0);
      } else {
        char* rowp = const_cast<char*>(p.m) + x.r * p.ld_b;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int64_t c = x.c + e;
          if (c >= 0 && c < p.N) store_elem<ESIZE>(rowp + c * ESIZE, vec_get<ESIZE>(v[u], e));
        }
      }
    }
  }
}

// Generic path (column stride != 1, tile rows that are not whole 16-byte
// vectors, or offsets past 32 bits): one tile element per lane.
struct ElemCopyParams {
  const char* m;
  char* tiles;
  int64_t M, N, ld_b, col_b;  // row / column strides of the matrix in bytes
  int64_t r0, c0, G_c;
  int64_t sr, sc;  // window step
  int64_t tm, tn;
  int64_t n;  // total tile elements
};

template <int ESIZE, bool STORE>
__global__ __launch_bounds__(kThreads) void copy_elem_kernel(ElemCopyParams p) {
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < p.n; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t j = idx % p.tn;
    const int64_t i = (idx / p.tn) % p.tm;
    const int64_t t = idx / (p.tn * p.tm);
    const int64_t gc = t % p.G_c, gr = t / p.G_c;
    const int64_t r = p.r0 + gr * p.sr + i, c = p.c0 + gc * p.sc + j;
    const bool ok = r >= 0 && r < p.M && c >= 0 && c < p.N;
    char* tp = p.tiles + idx * ESIZE;
    if (STORE) {
      if (ok) copy_elem<ESIZE>(const_cast<char*>(p.m) + r * p.ld_b + c * p.col_b, tp);
    } else {
      store_elem<ESIZE>(tp, ok ? load_elem<ESIZE>(p.m + r * p.ld_b + c * p.col_b) : 0);
    }
  }
}

template <bool STORE>
int launch(const char* name, const stg_tensor* mat, int64_t tm, int64_t tn, int64_t sr, int64_t sc, int64_t r0,
           int64_t c0, int check_bounds, void* tiles, void* stream) {
  clear_error();
  int rc;
  if ((rc = check_tensor(mat, name))) return rc;
  if (mat->rank != 2) return fail(STG_ERR_INVALID, "%s: matrix must have rank 2", name);
  if (tm < 1 || tn < 1) return fail(STG_ERR_INVALID, "%s: tile shape must be >= 1", name);
  if (sr < 1 || sc < 1) return fail(STG_ERR_INVALID, "%s: window step must be >= 1", name);
  if (tm > (1 << 20) || tn > (1 << 20) || sr > (1 << 20) || sc > (1 << 20))
    return fail(STG_ERR_RANGE, "%s: tile dimension or step exceeds 2^20", name);
  const int64_t lim = int64_t(1) << 40;
  if (r0 > lim || r0 < -lim || c0 > lim || c0 < -lim) return fail(STG_ERR_RANGE, "%s: |origin| exceeds 2^40", name);
  const int64_t M = mat->shape[0], N = mat->shape[1];
  const int64_t G_r = stg_tile_grid(M, r0, sr), G_c = stg_tile_grid(N, c0, sc);
  if (G_r == 0 || G_c == 0) return STG_OK;
  int64_t n_elems;  // tile-buffer elements, bounded like a descriptor's
  if (__builtin_mul_overflow(G_r, G_c, &n_elems) || __builtin_mul_overflow(n_elems, tm * tn, &n_elems) ||
      n_elems > (int64_t(1) << 48))
    return fail(STG_ERR_RANGE, "%s: the tile buffer would hold more than 2^48 elements", name);
  // every window inside the logical extent: the unchecked instance applies
  const bool inside = r0 >= 0 && c0 >= 0 && r0 + (G_r - 1) * sr + tm <= M && c0 + (G_c - 1) * sc + tn <= N;
  if (!check_bounds && !inside)
    return fail(STG_ERR_INVALID,
                "%s: check_bounds = 0 promises that every window lies inside the (%lld, %lld) array, but the grid "
                "reaches rows [%lld, %lld) and columns [%lld, %lld)",
                name, (long long)M, (long long)N, (long long)r0, (long long)(r0 + (G_r - 1) * sr + tm), (long long)c0,
                (long long)(c0 + (G_c - 1) * sc + tn));
  if (!tiles) return fail(STG_ERR_INVALID, "%s: null tile buffer", name);
  const int es = dtype_size(mat->dtype);
  const hipStream_t s = as_stream(stream);
  const int64_t ld_b = mat->stride[0] * es;
  const bool vec = mat->stride[1] == 1 && (tn * es) % 16 == 0 && ((uintptr_t)tiles & 15) == 0 &&
                   (tn * es) / 16 <= 64;
  if (vec) {
    CopyParams p{};
    p.m = (const char*)mat->data;
    p.tiles = (char*)tiles;
    p.M = M, p.N = N, p.ld_b = ld_b, p.r0 = r0, p.c0 = c0, p.G_c = G_c;
    p.sr = sr, p.sc = sc;
    p.tm = (int32_t)tm, p.tn = (int32_t)tn, p.esize = es;
    p.cpt = (int32_t)(tn * es / 16);
    p.tiles_per_wg = 64 / p.cpt;  // one 64-lane row segment per wavefront
    if (p.tiles_per_wg > G_c) p.tiles_per_wg = (int32_t)G_c;
    p.rows_per_wg = (int32_t)(tm < 8 ? tm : 8);
    p.row_blocks = (int32_t)((tm + p.rows_per_wg - 1) / p.rows_per_wg);
    p.span_magic = div_magic((uint32_t)(p.tiles_per_wg * p.cpt));
    p.cpt_magic = div_magic((uint32_t)p.cpt);
    p.n_cb = (uint32_t)((G_c + p.tiles_per_wg - 1) / p.tiles_per_wg);
    const int64_t n_wg = (int64_t)p.n_cb * G_r * p.row_blocks;
    // 32-bit buffer offsets relative to the workgroup's first row
    if ((int64_t)p.rows_per_wg * ld_b + N * es < kMaxOffset32 && n_wg < INT32_MAX) {
      const dim3 grid((unsigned)n_wg);
      {
#define STG_LAUNCH_VEC(ES)                                                                                    \
  inside ? launch_kernel(name, (STORE ? store_clipped_kernel<ES, false> : copy_bounded_kernel<ES, false>), grid,   \
                         dim3(kThreads), 0, s, p)                                                                  \
         : launch_kernel(name, (STORE ? store_clipped_kernel<ES, true> : copy_bounded_kernel<ES, true>), grid,     \
                         dim3(kThreads), 0, s, p)
        switch (es) {
          case 1: STG_LAUNCH_VEC(1); break;
          case 2: STG_LAUNCH_VEC(2); break;
          case 4: STG_LAUNCH_VEC(4); break;
          default: STG_LAUNCH_VEC(8); break;
        }
#undef STG_LAUNCH_VEC
        return check_launch(name);
      }
    }
  }
  ElemCopyParams p{};
  p.m = (const char*)mat->data;
  p.tiles = (char*)tiles;
  p.M = M, p.N = N, p.ld_b = ld_b, p.col_b = mat->stride[1] * es;
  p.r0 = r0, p.c0 = c0, p.G_c = G_c, p.tm = tm, p.tn = tn;
  p.sr = sr, p.sc = sc;
  p.n = G_r * G_c * tm * tn;
  const int64_t want = (p.n + kThreads - 1) / kThreads;
  const dim3 grid((unsigned)(want < 65536 ? want : 65536));
#define STG_LAUNCH_EL(ES) launch_kernel(name, (copy_elem_kernel<ES, STORE>), grid, dim3(kThreads), 0, s, p)
  switch (es) {
    case 1: STG_LAUNCH_EL(1); break;
    case 2: STG_LAUNCH_EL(2); break;
    case 4: STG_LAUNCH_EL(4); break;
    default: STG_LAUNCH_EL(8); break;
  }
#undef STG_LAUNCH_EL
  return check_launch(name);
}

}  // namespace
}  // namespace stg

using namespace stg;

extern "C" int tile_copy_bounded(const stg_tensor* src, int64_t tile_rows, int64_t tile_cols, int64_t origin_row,
                                 int64_t origin_col, void* tiles_out, void* stream) {
  return launch<false>("tile_copy_bounded", src, tile_rows, tile_cols, tile_rows, tile_cols, origin_row, origin_col, 1,
                       tiles_out, stream);
}

extern "C" int tile_store_clipped(const void* tiles_in, int64_t tile_rows, int64_t tile_cols, int64_t origin_row,
                                  int64_t origin_col, const stg_tensor* dst, void* stream) {
  return launch<true>("tile_store_clipped", dst, tile_rows, tile_cols, tile_rows, tile_cols, origin_row, origin_col, 1,
                      const_cast<void*>(tiles_in), stream);
}

extern "C" int tile_copy_windows(const stg_tensor* src, int64_t tile_rows, int64_t tile_cols, int64_t step_rows,
                                 int64_t step_cols, int64_t origin_row, int64_t origin_col, int32_t check_bounds,
                                 void* tiles_out, void* stream) {
  return launch<false>("tile_copy_windows", src, tile_rows, tile_cols, step_rows, step_cols, origin_row, origin_col,
                       check_bounds, tiles_out, stream);
}

extern "C" int tile_store_windows(const void* tiles_in, int64_t tile_rows, int64_t tile_cols, int64_t step_rows,
                                  int64_t step_cols, int64_t origin_row, int64_t origin_col, int32_t check_bounds,
                                  const stg_tensor* dst, void* stream) {
  return launch<true>("tile_store_windows", dst, tile_rows, tile_cols, step_rows, step_cols, origin_row, origin_col,
                      check_bounds, const_cast<void*>(tiles_in), stream);
}
