// Ragged varlen 3-D tile load and store.
//
// Semantics (Mojo, layout.tma_async.RaggedTMA3DTile: description, parameters
// BM / BN / middle_dim / group, comptime BM_seq, and the per-copy arguments
// ragged_idx / dynamic_dim / middle_idx of async_copy_from_col and
// async_copy_batched): sequences are packed row after row with no padding; a
// tile of BM = BM_seq * group rows covers BM_seq consecutive sequence
// positions starting at ragged_idx for head middle_idx (group heads fused per
// position when group > 1), and only dynamic_dim of those positions belong to
// the sequence.  The load writes the rest of the tile as zero; the store
// writes only the positions that belong, and no column past depth (the page
// masks the part of the box that overhangs the array).
//
// The page reaches this with a TMA descriptor whose outermost coordinate folds
// the (rows, middle_dim) selectors into one, (ragged_idx + dynamic_dim) *
// middle_dim + middle_idx, from a base pointer BM_seq rows in front of the data
// so that the box's out-of-range rows are the ones past the sequence.  gfx950
// has no TMA; the equivalent here is a buffer resource rebased at the tile's
// first row with num_records ending at the last row of the array: every 16-byte
// vector of an invalid position is given an offset past num_records, so a load
// returns zeros and a store is dropped, and no storage in front of the pointer
// is needed.
//
// Work mapping: a tile is split into slices of kThreads 16-byte vectors, one
// vector per lane, and each slice is one workgroup (4 KiB; a 128 x 128 bf16
// tile is eight of them).  Slices are numbered so that consecutive ones --
// the slices of one tile, and the tiles of neighbouring heads, which share the
// packed rows -- run on the same XCD.  Measured against one workgroup per
// tile, this moves the 128 x 128 bf16 tiles 4-13% faster (load and store,
// group 1 and 4).
// A wavefront moves 64 x 16 bytes per instruction.  With group > 1 the `group`
// heads of one position are adjacent in memory, so each position is a single
// contiguous run of group * depth elements.
#include "stg_internal.h"

namespace stg {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;  // vectors per lane; a slice is kThreads * kUnroll vectors

struct RaggedParams {
  char* x;      // the packed 3-D array (load: source, store: destination)
  char* tiles;  // dense (n_tiles, BM, BN) tile buffer (load: output, store: input)
  const uint32_t* ragged_idx;
  const uint32_t* dynamic_dim;
  const uint32_t* middle_idx;
  int64_t total_rows;
  int64_t row_b;   // bytes per packed row: middle_dim * group * depth * esize
  int64_t head_b;  // bytes per head: depth * esize
  int64_t tile_b;  // bytes per output tile: BM * BN * esize
  int32_t middle_dim, group, bm_seq;
  int32_t col0_b;     // col0 * esize
  int32_t out_row_b;  // BN * esize
  int32_t valid_b;    // bytes of an output row backed by source columns
  int32_t cpr;        // 16-byte chunks per output row
  uint32_t cpr_magic, group_magic;
  int32_t items;      // BM * cpr
  uint32_t slices;    // workgroups per tile: ceil(items / (kThreads * kUnroll)), at most 256
  uint32_t slices_magic;  // ceil(2^32 / slices), 0 when slices == 1
};

// Tile of workgroup `wg` (wg < 2^31): wg / slices by a multiply-high whose
// estimate is at most one too large (the magic's rounding error times wg is
// below 1/2), then one correction.  All scalar, so the tile's three schedule
// words are fetched together right after the kernel arguments.
__device__ __forceinline__ uint32_t tile_of(const RaggedParams& p, uint32_t wg) {
  if (p.slices == 1) return wg;
  uint32_t q = __umulhi(wg, p.slices_magic);
  if (q * p.slices > wg) --q;
  return q;
}

// Tile k's view of the packed array: the positions that exist (below
// dynamic_dim, inside the array, valid head), the address of its first element
// and a buffer resource over the rest of the array from there.
struct TileView {
  int64_t dyn;
  char* base;
  __amdgpu_buffer_rsrc_t rs;
};

__device__ __forceinline__ TileView tile_view(const RaggedParams& p, int64_t k) {
  const int64_t ri = p.ragged_idx[k];
  const int64_t mi = p.middle_idx[k];
  int64_t dyn = p.dynamic_dim[k];
  if (ri + dyn > p.total_rows) dyn = p.total_rows > ri ? p.total_rows - ri : 0;
  if (mi >= p.middle_dim) dyn = 0;
  const int64_t base_row = ri < p.total_rows ? ri : 0;
  char* base = p.x + base_row * p.row_b + mi * p.group * p.head_b + p.col0_b;
  int64_t avail = (p.total_rows - base_row) * p.row_b - mi * p.group * p.head_b - p.col0_b;
  if (dyn <= 0 || avail < 0) avail = 0;
  return {dyn, base, make_rsrc(base, (uint32_t)(avail < (int64_t)kOOB ? avail : (int64_t)kOOB - 1))};
}

// FULL: every output row is whole 16-byte vectors, all backed by source
// columns (BN * esize a multiple of 16, col0 + BN <= depth), and the tile is
// a whole number of slices, so no vector needs the element path or
// a bounds test and vector `it` of the tile sits at byte 16 * it of its
// output -- the common case (128 x 128 bf16), and about 5% faster.
template <int ESIZE, bool FULL>
__global__ __launch_bounds__(kThreads) void ragged_load_kernel(RaggedParams p) {
  constexpr int V = 16 / ESIZE;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = tile_of(p, wg);
  const TileView tv = tile_view(p, k);
  const int64_t dyn = tv.dyn;
  const char* base = tv.base;
  const __amdgpu_buffer_rsrc_t rs = tv.rs;
  char* out = p.tiles + k * p.tile_b;
  const int b0 = (int)(wg - k * p.slices) * (kThreads * kUnroll);
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int it = b0 + u * kThreads + threadIdx.x;
    v[u] = (u32x4){0, 0, 0, 0};
    if (FULL || it < p.items) {
      const int j = (int)div_small((uint32_t)it, p.cpr_magic);  // tile row = s * group + g
      const int b = (it - j * p.cpr) * 16;
      const int s = (int)div_small((uint32_t)j, p.group_magic);
      const int g = j - s * p.group;
      const bool row_ok = s < dyn;
      const uint32_t roff = (uint32_t)(s * p.row_b + g * p.head_b);
      const bool full = row_ok && (FULL || b + 16 <= p.valid_b);
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, full ? roff + b : kOOB, 0, 0);
      if (!FULL && row_ok && !full && b < p.valid_b) {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (b + e * ESIZE < p.valid_b) vec_set<ESIZE>(v[u], e, load_elem<ESIZE>(base + roff + b + e * ESIZE));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int it = b0 + u * kThreads + threadIdx.x;
    if (FULL) {
      st16(out + (int64_t)it * 16, v[u]);
    } else if (it < p.items) {
      const int j = (int)div_small((uint32_t)it, p.cpr_magic);
      const int b = (it - j * p.cpr) * 16;
      char* d = out + (int64_t)j * p.out_row_b + b;
      if (b + 16 <= p.out_row_b) {
        st16(d, v[u]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (b + e * ESIZE < p.out_row_b) store_elem<ESIZE>(d + e * ESIZE, vec_get<ESIZE>(v[u], e));
      }
    }
  }
}

// Store direction: tile vector `it` (row j = s * group + g, bytes b..b+15 of
// the row) goes to position s, head slot g of the tile's view when s < dyn;
// only those vectors are read from the tile.  A vector with no place in the
// array gets an offset past num_records and its store is dropped; a vector
// that crosses the end of depth is written element by element up to it.
// FULL as for the load.
template <int ESIZE, bool FULL>
__global__ __launch_bounds__(kThreads) void ragged_store_kernel(RaggedParams p) {
  constexpr int V = 16 / ESIZE;
  const uint32_t wg = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t k = tile_of(p, wg);
  const TileView tv = tile_view(p, k);
  const char* in = p.tiles + k * p.tile_b;
  const int b0 = (int)(wg - k * p.slices) * (kThreads * kUnroll);
  u32x4 v[kUnroll];
  uint32_t off[kUnroll];  // byte offset of the vector in the view, kOOB when it has no place
  int bb[kUnroll];        // byte of the vector within its row; -1 when nothing is stored
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int it = b0 + u * kThreads + threadIdx.x;
    off[u] = kOOB;
    bb[u] = -1;
    v[u] = (u32x4){0, 0, 0, 0};
    if (FULL || it < p.items) {
      const int j = (int)div_small((uint32_t)it, p.cpr_magic);
      const int b = (it - j * p.cpr) * 16;
      const int s = (int)div_small((uint32_t)j, p.group_magic);
      const int g = j - s * p.group;
      if (s < tv.dyn && b < p.valid_b) {
        bb[u] = b;
        off[u] = (uint32_t)(s * p.row_b + g * p.head_b) + b;
        const char* src = in + (int64_t)j * p.out_row_b + b;
        if (FULL || b + 16 <= p.out_row_b) {
          v[u] = ld16(src);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (b + e * ESIZE < p.out_row_b) vec_set<ESIZE>(v[u], e, load_elem<ESIZE>(src + e * ESIZE));
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const bool full = bb[u] >= 0 && (FULL || bb[u] + 16 <= p.valid_b);
    __builtin_amdgcn_raw_buffer_store_b128(v[u], tv.rs, full ? off[u] : kOOB, 0, 0);
    if (!FULL && bb[u] >= 0 && !full) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if (bb[u] + e * ESIZE < p.valid_b) store_elem<ESIZE>(tv.base + off[u] + e * ESIZE, vec_get<ESIZE>(v[u], e));
    }
  }
}

// Shared argument checks and parameter setup of both directions.
int ragged_setup(const char* name, const void* x, int32_t dtype, int64_t total_rows, int32_t middle_dim,
                 int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0, const uint32_t* ragged_idx,
                 const uint32_t* dynamic_dim, const uint32_t* middle_idx, int64_t n_tiles, const void* tiles,
                 RaggedParams& p, int& es) {
  es = dtype_size(dtype);
  if (!es) return fail(STG_ERR_UNSUPPORTED, "%s: unknown dtype %d", name, dtype);
  if (total_rows < 0 || n_tiles < 0) return fail(STG_ERR_INVALID, "%s: negative size", name);
  if (middle_dim < 1 || group < 1 || depth < 1 || BM < 1 || BN < 1)
    return fail(STG_ERR_INVALID, "%s: middle_dim, group, depth, BM and BN must be >= 1", name);
  if (BM % group) return fail(STG_ERR_INVALID, "%s: BM %d is not a multiple of group %d", name, BM, group);
  if (col0 < 0 || col0 >= depth) return fail(STG_ERR_INVALID, "%s: col0 %d not in [0, depth)", name, col0);
  // a packed row (middle_dim x group x depth elements) must fit the 32-bit
  // offsets of one tile's rows; checked factor by factor so that the product
  // cannot overflow first
  if ((int64_t)depth * es >= kMaxOffset32 || (int64_t)middle_dim * group >= kMaxOffset32 / ((int64_t)depth * es) ||
      total_rows > (int64_t(1) << 40))
    return fail(STG_ERR_RANGE, "%s: packed rows of %d x %d x %d elements, or %lld rows, too large", name,
                middle_dim, group, depth, (long long)total_rows);
  if (n_tiles == 0) return STG_OK;
  if (!tiles || !ragged_idx || !dynamic_dim || !middle_idx)
    return fail(STG_ERR_INVALID, "%s: null tile buffer or tile triples", name);
  if (total_rows > 0 && !x) return fail(STG_ERR_INVALID, "%s: null packed array", name);
  p = RaggedParams{};
  p.x = (char*)x;
  p.tiles = (char*)tiles;
  p.ragged_idx = ragged_idx;
  p.dynamic_dim = dynamic_dim;
  p.middle_idx = middle_idx;
  p.total_rows = total_rows;
  p.head_b = (int64_t)depth * es;
  p.row_b = (int64_t)middle_dim * group * p.head_b;
  p.middle_dim = middle_dim;
  p.group = group;
  p.bm_seq = BM / group;
  p.col0_b = col0 * es;
  p.out_row_b = BN * es;
  p.tile_b = (int64_t)BM * BN * es;
  const int64_t valid_cols = depth - col0 < BN ? depth - col0 : BN;
  p.valid_b = (int32_t)(valid_cols * es);
  p.cpr = (p.out_row_b + 15) / 16;
  if ((int64_t)BM * p.cpr > 65535 || p.cpr >= 32768 || group >= 32768)
    return fail(STG_ERR_RANGE, "%s: tile of %d x %d elements is too large", name, BM, BN);
  if ((int64_t)p.bm_seq * p.row_b + p.out_row_b >= kMaxOffset32)
    return fail(STG_ERR_RANGE, "%s: BM_seq rows span more than 2^31 bytes", name);
  p.items = BM * p.cpr;
  p.slices = (uint32_t)((p.items + kThreads * kUnroll - 1) / (kThreads * kUnroll));
  p.slices_magic = p.slices == 1 ? 0u : (uint32_t)(((uint64_t(1) << 32) + p.slices - 1) / p.slices);
  if (n_tiles > INT32_MAX / (int64_t)p.slices) return fail(STG_ERR_RANGE, "%s: too many tiles", name);
  p.cpr_magic = div_magic((uint32_t)p.cpr);
  p.group_magic = div_magic((uint32_t)group);
  return STG_OK;
}

bool ragged_full(const RaggedParams& p) {
  return p.out_row_b % 16 == 0 && p.valid_b == p.out_row_b && p.items % (kThreads * kUnroll) == 0;
}

}  // namespace
}  // namespace stg

using namespace stg;

extern "C" int ragged_tile_load(const void* src, int32_t dtype, int64_t total_rows, int32_t middle_dim,
                                int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                                const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                                const uint32_t* middle_idx, int64_t n_tiles, void* tiles_out, void* stream) {
  clear_error();
  const char* name = "ragged_tile_load";
  RaggedParams p;
  int es, rc;
  if ((rc = ragged_setup(name, src, dtype, total_rows, middle_dim, group, depth, BM, BN, col0, ragged_idx,
                         dynamic_dim, middle_idx, n_tiles, tiles_out, p, es)) || n_tiles == 0)
    return rc;
  const hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)(n_tiles * p.slices)), block(kThreads);
  const bool full = ragged_full(p);
#define STG_RAGGED(K, E) \
  full ? launch_kernel(name, K<E, true>, grid, block, 0, s, p) : launch_kernel(name, K<E, false>, grid, block, 0, s, p)
  switch (es) {
    case 1: STG_RAGGED(ragged_load_kernel, 1); break;
    case 2: STG_RAGGED(ragged_load_kernel, 2); break;
    case 4: STG_RAGGED(ragged_load_kernel, 4); break;
    default: STG_RAGGED(ragged_load_kernel, 8); break;
  }
  return check_launch(name);
}

extern "C" int ragged_tile_store(const void* tiles_in, int32_t dtype, int64_t total_rows, int32_t middle_dim,
                                 int32_t group, int32_t depth, int32_t BM, int32_t BN, int32_t col0,
                                 const uint32_t* ragged_idx, const uint32_t* dynamic_dim,
                                 const uint32_t* middle_idx, int64_t n_tiles, void* dst, void* stream) {
  clear_error();
  const char* name = "ragged_tile_store";
  RaggedParams p;
  int es, rc;
  if ((rc = ragged_setup(name, dst, dtype, total_rows, middle_dim, group, depth, BM, BN, col0, ragged_idx,
                         dynamic_dim, middle_idx, n_tiles, tiles_in, p, es)) || n_tiles == 0)
    return rc;
  const hipStream_t s = as_stream(stream);
  const dim3 grid((unsigned)(n_tiles * p.slices)), block(kThreads);
  const bool full = ragged_full(p);
  switch (es) {
    case 1: STG_RAGGED(ragged_store_kernel, 1); break;
    case 2: STG_RAGGED(ragged_store_kernel, 2); break;
    case 4: STG_RAGGED(ragged_store_kernel, 4); break;
    default: STG_RAGGED(ragged_store_kernel, 8); break;
  }
#undef STG_RAGGED
  return check_launch(name);
}
