// Indexed tile gather, masked gather and masked scatter.
//
// Semantics (Warp, warp.tile_load_indexed: description and parameters;
// cuTile.jl Memory: gather/scatter with mask and padding_value, "Sparse
// views"): output coordinate o reads a[s] with s[d] = offset[d] + o[d] off the
// gather axis and s[axis] = offset[axis] + indices[o[axis]] on it; any
// coordinate outside [0, extent) reads zero (or the padding value), and the
// scatter skips it.  Tiles are stacked along the axis, so the tile boundaries
// only decide which index slice a workgroup stages.
//
// Two kernel shapes:
//  * row path -- the innermost dimension is contiguous in both arrays and is
//    not the gather axis.  The output is a set of rows (all coordinates but the
//    last); each workgroup resolves the index slice of its rows into an LDS
//    row table (source/destination byte offsets, validity), then every lane
//    moves 16-byte vectors.  Only vectors that straddle the column bounds take
//    the per-element path; an address is formed only for a valid coordinate.
//    The scatter compacts its active rows with wavefront ballots first, so
//    masked-out rows cost no memory traffic at all.
//  * element path -- anything else (gather along the innermost axis, strided
//    innermost dimension): one element per lane.
#include "stg_internal.h"

namespace stg {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxRowsPerWg = 256;
constexpr int kUnroll = 8;  // 16-byte vectors in flight per lane
constexpr int64_t kNoRow = INT64_MIN;

struct RowParams {
  const char* a;  // element [0,..,0] of the indexed array
  char* t;        // element [0,..,0] of the dense-side array (gather out / scatter tile)
  const int32_t* indices;
  const uint8_t* mask;  // null: all true
  int64_t n_rows;       // n_indices * rest
  int64_t rest;         // rows per index
  int64_t ax_off, ax_ext, a_ax_b, t_ax_b;
  int64_t p_n, p_off, p_ext, a_p_b, t_p_b;
  int64_t q_n, q_off, q_ext, a_q_b, t_q_b;
  int64_t a_col_b;  // offset[last] * esize
  int32_t row_bytes;
  int32_t n_chunks;
  uint32_t chunk_magic;
  int32_t lo_b, hi_b;  // valid byte range of a row (column bounds)
  int32_t rows_per_wg;
  uint32_t fill[4];
};

struct ElemParams {
  const char* a;
  char* t;
  const int32_t* indices;
  const uint8_t* mask;
  int32_t rank, axis;
  int64_t n;  // elements of the dense-side array
  int64_t tshape[4];
  int64_t a_ext[4], a_st_b[4], t_st_b[4], off[4];
  uint32_t fill[4];
};

// Resolve row g of the dense side: returns the byte offset into `a` of the
// row's first tile column (kNoRow if the row is invalid or masked out) and the
// byte offset of the row in the dense-side array.
__device__ __forceinline__ void resolve_row(const RowParams& p, int64_t g, int64_t& a_off, int64_t& t_off) {
  int64_t o_ax, op = 0, oq = 0;
  if (p.rest == 1) {
    o_ax = g;
  } else {
    o_ax = g / p.rest;
    const int64_t rr = g - o_ax * p.rest;
    op = rr / p.q_n;
    oq = rr - op * p.q_n;
  }
  const int64_t sa = p.ax_off + (int64_t)p.indices[o_ax];
  const int64_t sp = p.p_off + op, sq = p.q_off + oq;
  bool ok = sa >= 0 && sa < p.ax_ext && sp >= 0 && sp < p.p_ext && sq >= 0 && sq < p.q_ext;
  if (p.mask) ok = ok && p.mask[o_ax] != 0;
  a_off = ok ? sa * p.a_ax_b + sp * p.a_p_b + sq * p.a_q_b + p.a_col_b : kNoRow;
  t_off = o_ax * p.t_ax_b + op * p.t_p_b + oq * p.t_q_b;
}

// FULL: the row is whole 16-byte vectors and every column is in bounds
// (lo_b = 0, hi_b = row_bytes), so no vector takes the element path.
template <int ESIZE, bool FULL>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(RowParams p) {
  constexpr int V = 16 / ESIZE;
  __shared__ int64_t s_src[kMaxRowsPerWg];
  __shared__ int64_t s_dst[kMaxRowsPerWg];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * p.rows_per_wg;
  const int nr = (int)min((int64_t)p.rows_per_wg, p.n_rows - row0);
  if (tid < nr) {
    int64_t ao, to;
    resolve_row(p, row0 + tid, ao, to);
    s_src[tid] = ao;
    s_dst[tid] = to;
  }
  __syncthreads();
  const u32x4 fill = {p.fill[0], p.fill[1], p.fill[2], p.fill[3]};
  const int items = nr * p.n_chunks;
  for (int base = 0; base < items; base += kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = base + u * kThreads + tid;
      v[u] = fill;
      if (it < items) {
        const int r = (int)div_small((uint32_t)it, p.chunk_magic);
        const int b = (it - r * p.n_chunks) * 16;
        const int64_t so = s_src[r];
        if (so != kNoRow) {
          if (FULL || (b >= p.lo_b && b + 16 <= p.hi_b)) {
            v[u] = ld16(p.a + so + b);
          } else if (b + 16 > p.lo_b && b < p.hi_b) {
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const int bb = b + e * ESIZE;
              if (bb >= p.lo_b && bb < p.hi_b) vec_set<ESIZE>(v[u], e, load_elem<ESIZE>(p.a + so + bb));
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = base + u * kThreads + tid;
      if (it < items) {
        const int r = (int)div_small((uint32_t)it, p.chunk_magic);
        const int b = (it - r * p.n_chunks) * 16;
        char* d = p.t + s_dst[r] + b;
        if (FULL || b + 16 <= p.row_bytes) {
          st16(d, v[u]);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (b + e * ESIZE < p.row_bytes) store_elem<ESIZE>(d + e * ESIZE, vec_get<ESIZE>(v[u], e));
        }
      }
    }
  }
}

template <int ESIZE, bool FULL>
__global__ __launch_bounds__(kThreads) void scatter_rows_kernel(RowParams p) {
  constexpr int V = 16 / ESIZE;
  __shared__ int64_t s_dst[kMaxRowsPerWg];  // offset into a (the scatter destination)
  __shared__ int64_t s_src[kMaxRowsPerWg];  // offset into the tile
  __shared__ int s_count[kThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * p.rows_per_wg;
  const int nr = (int)min((int64_t)p.rows_per_wg, p.n_rows - row0);
  int64_t ao = kNoRow, to = 0;
  if (tid < nr) resolve_row(p, row0 + tid, ao, to);
  const bool active = ao != kNoRow;
  // compact the active rows: wavefront ballot + prefix count within the wave,
  // then an exclusive sum over the waves of the workgroup
  const uint64_t ballot = __ballot(active);
  const int in_wave = __popcll(ballot & ((uint64_t(1) << lane) - 1));
  if (lane == 0) s_count[wave] = __popcll(ballot);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    before += w < wave ? s_count[w] : 0;
    total += s_count[w];
  }
  if (active) {
    s_dst[before + in_wave] = ao;
    s_src[before + in_wave] = to;
  }
  __syncthreads();
  const int items = total * p.n_chunks;
  for (int base = 0; base < items; base += kThreads * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = base + u * kThreads + tid;
      if (it < items) {
        const int r = (int)div_small((uint32_t)it, p.chunk_magic);
        const int b = (it - r * p.n_chunks) * 16;
        if (FULL || (b >= p.lo_b && b + 16 <= p.hi_b)) v[u] = ld16(p.t + s_src[r] + b);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int it = base + u * kThreads + tid;
      if (it < items) {
        const int r = (int)div_small((uint32_t)it, p.chunk_magic);
        const int b = (it - r * p.n_chunks) * 16;
        if (FULL || (b >= p.lo_b && b + 16 <= p.hi_b)) {
          st16(const_cast<char*>(p.a) + s_dst[r] + b, v[u]);
        } else if (b + 16 > p.lo_b && b < p.hi_b) {
          const char* src = p.t + s_src[r] + b;
          char* dst = const_cast<char*>(p.a) + s_dst[r] + b;
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int bb = b + e * ESIZE;
            if (bb >= p.lo_b && bb < p.hi_b) copy_elem<ESIZE>(dst + e * ESIZE, src + e * ESIZE);
          }
        }
      }
    }
  }
}

// Element path: one dense-side element per lane, grid-stride.
__device__ __forceinline__ bool resolve_elem(const ElemParams& p, int64_t i, int64_t& a_off, int64_t& t_off,
                                             bool& masked_out) {
  int64_t o[4];
  int64_t rem = i;
  for (int d = p.rank - 1; d >= 0; --d) {
    o[d] = rem % p.tshape[d];
    rem /= p.tshape[d];
  }
  bool ok = true;
  a_off = 0;
  t_off = 0;
  for (int d = 0; d < p.rank; ++d) {
    const int64_t s = d == p.axis ? p.off[d] + (int64_t)p.indices[o[d]] : p.off[d] + o[d];
    ok = ok && s >= 0 && s < p.a_ext[d];
    a_off += s * p.a_st_b[d];
    t_off += o[d] * p.t_st_b[d];
  }
  masked_out = p.mask && p.mask[o[p.axis]] == 0;
  return ok && !masked_out;
}

template <int ESIZE>
__global__ __launch_bounds__(kThreads) void gather_elem_kernel(ElemParams p) {
  const uint64_t fill = (uint64_t)p.fill[0] | ((uint64_t)p.fill[1] << 32);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.n; i += (int64_t)gridDim.x * kThreads) {
    int64_t ao, to;
    bool masked_out;
    const bool ok = resolve_elem(p, i, ao, to, masked_out);
    store_elem<ESIZE>(p.t + to, ok ? load_elem<ESIZE>(p.a + ao) : fill);
  }
}

template <int ESIZE>
__global__ __launch_bounds__(kThreads) void scatter_elem_kernel(ElemParams p) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.n; i += (int64_t)gridDim.x * kThreads) {
    int64_t ao, to;
    bool masked_out;
    if (resolve_elem(p, i, ao, to, masked_out))
      copy_elem<ESIZE>(const_cast<char*>(p.a) + ao, p.t + to);
  }
}

// ---- host side -------------------------------------------------------------

enum class Op { Gather, GatherMasked, Scatter };

const char* op_name(Op op) {
  return op == Op::Gather ? "tile_gather" : op == Op::GatherMasked ? "tile_gather_masked" : "tile_scatter_masked";
}

int launch_rows(Op op, int esize, const RowParams& p, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b(kThreads);
  const bool full = p.lo_b == 0 && p.hi_b == p.row_bytes && p.row_bytes % 16 == 0;
#define STG_ROWS(K, E) \
  full ? launch_kernel(op_name(op), K<E, true>, g, b, 0, s, p) : launch_kernel(op_name(op), K<E, false>, g, b, 0, s, p)
  if (op == Op::Scatter) {
    switch (esize) {
      case 1: STG_ROWS(scatter_rows_kernel, 1); break;
      case 2: STG_ROWS(scatter_rows_kernel, 2); break;
      case 4: STG_ROWS(scatter_rows_kernel, 4); break;
      default: STG_ROWS(scatter_rows_kernel, 8); break;
    }
  } else {
    switch (esize) {
      case 1: STG_ROWS(gather_rows_kernel, 1); break;
      case 2: STG_ROWS(gather_rows_kernel, 2); break;
      case 4: STG_ROWS(gather_rows_kernel, 4); break;
      default: STG_ROWS(gather_rows_kernel, 8); break;
    }
  }
#undef STG_ROWS
  return check_launch(op_name(op));
}

int launch_elems(Op op, int esize, const ElemParams& p, hipStream_t s) {
  const int64_t want = (p.n + kThreads - 1) / kThreads;
  const dim3 g((unsigned)(want < 65536 ? want : 65536)), b(kThreads);
  if (op == Op::Scatter) {
    switch (esize) {
      case 1: launch_kernel(op_name(op), scatter_elem_kernel<1>, g, b, 0, s, p); break;
      case 2: launch_kernel(op_name(op), scatter_elem_kernel<2>, g, b, 0, s, p); break;
      case 4: launch_kernel(op_name(op), scatter_elem_kernel<4>, g, b, 0, s, p); break;
      default: launch_kernel(op_name(op), scatter_elem_kernel<8>, g, b, 0, s, p); break;
    }
  } else {
    switch (esize) {
      case 1: launch_kernel(op_name(op), gather_elem_kernel<1>, g, b, 0, s, p); break;
      case 2: launch_kernel(op_name(op), gather_elem_kernel<2>, g, b, 0, s, p); break;
      case 4: launch_kernel(op_name(op), gather_elem_kernel<4>, g, b, 0, s, p); break;
      default: launch_kernel(op_name(op), gather_elem_kernel<8>, g, b, 0, s, p); break;
    }
  }
  return check_launch(op_name(op));
}

// Shared argument checks and dispatch of the three entry points.  `a` is the
// indexed array; `t` the dense side (gather output, scatter input).
int run(Op op, const stg_tensor* a, const int32_t* indices, const uint8_t* mask, int64_t n_indices,
        const int64_t* tile_shape, const int64_t* offset, int32_t axis, double padding_value,
        const stg_tensor* t, void* stream) {
  clear_error();
  const char* name = op_name(op);
  int rc;
  if ((rc = check_tensor(a, name)) || (rc = check_tensor(t, name))) return rc;
  if (a->dtype != t->dtype) return fail(STG_ERR_INVALID, "%s: dtype mismatch", name);
  if (a->rank != t->rank) return fail(STG_ERR_INVALID, "%s: rank mismatch", name);
  const int rank = a->rank;
  if (axis < 0 || axis >= rank) return fail(STG_ERR_INVALID, "%s: axis %d not in [0, %d)", name, axis, rank);
  if (!tile_shape) return fail(STG_ERR_INVALID, "%s: null tile_shape", name);
  for (int d = 0; d < rank; ++d)
    if (tile_shape[d] < 1) return fail(STG_ERR_INVALID, "%s: tile_shape[%d] < 1", name, d);
  if (n_indices < 0) return fail(STG_ERR_INVALID, "%s: negative n_indices", name);
  if (n_indices % tile_shape[axis])
    return fail(STG_ERR_INVALID, "%s: n_indices %lld is not a multiple of tile_shape[axis] %lld", name,
                (long long)n_indices, (long long)tile_shape[axis]);
  if (n_indices > INT32_MAX) return fail(STG_ERR_RANGE, "%s: n_indices exceeds 2^31-1", name);
  if (n_indices > 0 && !indices) return fail(STG_ERR_INVALID, "%s: null indices", name);
  for (int d = 0; d < rank; ++d) {
    const int64_t want = d == axis ? n_indices : tile_shape[d];
    if (t->shape[d] != want)
      return fail(STG_ERR_INVALID, "%s: %s shape[%d] is %lld, expected %lld", name,
                  op == Op::Scatter ? "tile" : "out", d, (long long)t->shape[d], (long long)want);
  }
  int64_t off[4] = {0, 0, 0, 0};
  if (offset)
    for (int d = 0; d < rank; ++d) {
      if (offset[d] > (int64_t(1) << 40) || offset[d] < -(int64_t(1) << 40))
        return fail(STG_ERR_RANGE, "%s: |offset[%d]| exceeds 2^40", name, d);
      off[d] = offset[d];
    }
  uint32_t fill[4] = {0, 0, 0, 0};
  if (op == Op::GatherMasked && fill_pattern(padding_value, a->dtype, fill))
    return fail(STG_ERR_INVALID, "%s: padding_value %g not representable in the element type", name, padding_value);
  const int es = dtype_size(a->dtype);
  int64_t numel = 1;
  for (int d = 0; d < rank; ++d) numel *= t->shape[d];
  if (numel == 0) return STG_OK;
  const hipStream_t s = as_stream(stream);
  const int last = rank - 1;

  const bool row_path = rank >= 2 && axis != last && a->stride[last] == 1 && t->stride[last] == 1 &&
                        tile_shape[last] * es <= 16 * 4096;
  if (row_path) {
    RowParams p{};
    p.a = (const char*)a->data;
    p.t = (char*)t->data;
    p.indices = indices;
    p.mask = op == Op::Gather ? nullptr : mask;
    p.ax_off = off[axis];
    p.ax_ext = a->shape[axis];
    p.a_ax_b = a->stride[axis] * es;
    p.t_ax_b = t->stride[axis] * es;
    int other[2] = {-1, -1}, n_other = 0;
    for (int d = 0; d < last; ++d)
      if (d != axis) other[n_other++] = d;
    auto dim = [&](int d, int64_t& n, int64_t& o, int64_t& ext, int64_t& ab, int64_t& tb) {
      if (d < 0) {
        n = 1, o = 0, ext = 1, ab = 0, tb = 0;
      } else {
        n = tile_shape[d], o = off[d], ext = a->shape[d], ab = a->stride[d] * es, tb = t->stride[d] * es;
      }
    };
    dim(other[0], p.p_n, p.p_off, p.p_ext, p.a_p_b, p.t_p_b);
    dim(other[1], p.q_n, p.q_off, p.q_ext, p.a_q_b, p.t_q_b);
    p.rest = p.p_n * p.q_n;
    p.n_rows = n_indices * p.rest;
    const int64_t W = tile_shape[last];
    p.a_col_b = off[last] * es;
    p.row_bytes = (int32_t)(W * es);
    p.n_chunks = (int32_t)((W * es + 15) / 16);
    p.chunk_magic = div_magic((uint32_t)p.n_chunks);
    int64_t lo = -off[last] > 0 ? -off[last] : 0;
    int64_t hi = a->shape[last] - off[last] < W ? a->shape[last] - off[last] : W;
    if (hi <= lo) lo = hi = 0;
    p.lo_b = (int32_t)(lo * es);
    p.hi_b = (int32_t)(hi * es);
    for (int i = 0; i < 4; ++i) p.fill[i] = fill[i];
    // about eight 16-byte vectors per lane, but keep enough workgroups in
    // flight to cover all 256 CUs several times over
    int64_t rows = (kThreads * kUnroll) / p.n_chunks;
    rows = rows < 1 ? 1 : rows > kMaxRowsPerWg ? kMaxRowsPerWg : rows;
    while (rows > 1 && (p.n_rows + rows - 1) / rows < 2048) rows /= 2;
    if (rows * p.n_chunks > 65535) rows = 65535 / p.n_chunks;
    p.rows_per_wg = (int32_t)rows;
    const int64_t grid = (p.n_rows + rows - 1) / rows;
    if (grid > INT32_MAX) return fail(STG_ERR_RANGE, "%s: too many rows", name);
    return launch_rows(op, es, p, grid, s);
  }
  ElemParams p{};
  p.a = (const char*)a->data;
  p.t = (char*)t->data;
  p.indices = indices;
  p.mask = op == Op::Gather ? nullptr : mask;
  p.rank = rank;
  p.axis = axis;
  p.n = numel;
  for (int d = 0; d < rank; ++d) {
    p.tshape[d] = t->shape[d];
    p.a_ext[d] = a->shape[d];
    p.a_st_b[d] = a->stride[d] * es;
    p.t_st_b[d] = t->stride[d] * es;
    p.off[d] = off[d];
  }
  for (int i = 0; i < 4; ++i) p.fill[i] = fill[i];
  return launch_elems(op, es, p, s);
}

}  // namespace
}  // namespace stg

using namespace stg;

extern "C" int tile_gather(const stg_tensor* a, const int32_t* indices, int64_t n_indices,
                           const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                           const stg_tensor* out, void* stream) {
  return run(Op::Gather, a, indices, nullptr, n_indices, tile_shape, offset, axis, 0.0, out, stream);
}

extern "C" int tile_gather_masked(const stg_tensor* a, const int32_t* indices, const uint8_t* mask,
                                  int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                                  int32_t axis, double padding_value, const stg_tensor* out, void* stream) {
  return run(Op::GatherMasked, a, indices, mask, n_indices, tile_shape, offset, axis, padding_value, out, stream);
}

extern "C" int tile_scatter_masked(const stg_tensor* a, const int32_t* indices, const uint8_t* mask,
                                   int64_t n_indices, const int64_t* tile_shape, const int64_t* offset,
                                   int32_t axis, const stg_tensor* tile, void* stream) {
  return run(Op::Scatter, a, indices, mask, n_indices, tile_shape, offset, axis, 0.0, tile, stream);
}
