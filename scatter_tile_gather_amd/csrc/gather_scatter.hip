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
//
// Backward of the gather (Warp, warp.tile_load_indexed, description: the load
// is differentiable; its backward adds the output gradient into a.grad at
// each location the forward read, atomically): the scatter kernels with every
// store replaced by a hardware float atomic add (fp32 or fp64, relaxed, device
// scope), unmasked; rows whose source is out of range are compacted away like
// masked-out scatter rows.  Repeated indices add up in an unspecified order.
// The chip retires about 77 G lane-wise float atomic adds per second whatever
// the table size, so with a caller-provided workspace the row layout takes an
// atomic-free path instead: the terms are grouped by destination row with a
// two-level counting sort done in LDS, and a reduction in which one group of
// lanes owns four consecutive destination rows, adds their terms and writes
// each row once with plain stores (rows with more than 64 terms excepted).
#include "stg_internal.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

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
// Workgroups are numbered XCD by XCD, so that consecutive output rows are
// written from one L2 (2% faster on the masked-gather workload; the scatter,
// whose writes land at random rows, gains nothing from it).
template <int ESIZE, bool FULL>
__global__ __launch_bounds__(kThreads) void gather_rows_kernel(RowParams p) {
  constexpr int V = 16 / ESIZE;
  __shared__ int64_t s_src[kMaxRowsPerWg];
  __shared__ int64_t s_dst[kMaxRowsPerWg];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * p.rows_per_wg;
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
          st16_nt(d, v[u]);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e)
            if (b + e * ESIZE < p.row_bytes) store_elem<ESIZE>(d + e * ESIZE, vec_get<ESIZE>(v[u], e));
        }
      }
    }
  }
}

// a.grad[...] += value, hardware float atomics (fp32 / fp64 only)
template <int ESIZE>
__device__ __forceinline__ void accum_elem(char* dst, uint64_t bits) {
  if constexpr (ESIZE == 4) {
    unsafeAtomicAdd((float*)dst, __uint_as_float((uint32_t)bits));
  } else if constexpr (ESIZE == 8) {
    unsafeAtomicAdd((double*)dst, __longlong_as_double((long long)bits));
  }
}

template <int ESIZE>
__device__ __forceinline__ void accum16(char* dst, const u32x4& v) {
#pragma unroll
  for (int e = 0; e < 16 / ESIZE; ++e) accum_elem<ESIZE>(dst + e * ESIZE, vec_get<ESIZE>(v, e));
}

template <int ESIZE, bool FULL, bool ACCUM>
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
          if (ACCUM)
            accum16<ESIZE>(const_cast<char*>(p.a) + s_dst[r] + b, v[u]);
          else
            st16_nt(const_cast<char*>(p.a) + s_dst[r] + b, v[u]);
        } else if (b + 16 > p.lo_b && b < p.hi_b) {
          const char* src = p.t + s_src[r] + b;
          char* dst = const_cast<char*>(p.a) + s_dst[r] + b;
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const int bb = b + e * ESIZE;
            if (bb >= p.lo_b && bb < p.hi_b) {
              if (ACCUM)
                accum_elem<ESIZE>(dst + e * ESIZE, load_elem<ESIZE>(src + e * ESIZE));
              else
                copy_elem<ESIZE>(dst + e * ESIZE, src + e * ESIZE);
            }
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

template <int ESIZE, bool ACCUM>
__global__ __launch_bounds__(kThreads) void scatter_elem_kernel(ElemParams p) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.n; i += (int64_t)gridDim.x * kThreads) {
    int64_t ao, to;
    bool masked_out;
    if (resolve_elem(p, i, ao, to, masked_out)) {
      if (ACCUM)
        accum_elem<ESIZE>(const_cast<char*>(p.a) + ao, load_elem<ESIZE>(p.t + to));
      else
        copy_elem<ESIZE>(const_cast<char*>(p.a) + ao, p.t + to);
    }
  }
}

// ---- sorted (segmented) backward -------------------------------------------
//
// The terms (grad_out rows) are grouped by destination row with a two-level
// counting sort, every step of it in LDS: destination rows fall into at most
// 4096 buckets of 2^shift consecutive rows;
//  1. each workgroup counts the bucket of each of its 4096 terms (LDS
//     atomics) and writes its counts as one column of a bucket-major table;
//  2. an exclusive scan of that table gives every (bucket, workgroup) pair
//     its place, so that each bucket's terms form one contiguous run;
//  3. each workgroup sorts its terms by bucket in LDS and writes them, as
//     (row, term) pairs, into those runs -- contiguous stretches, not single
//     scattered words;
//  4. one workgroup per bucket counts its terms per row (LDS atomics over a
//     window of 4096 rows), scans the counts into the rows' segment offsets
//     and places each term id into its row's segment.
// The reduce kernel then sums each row's segment.  The order of the terms
// inside a segment follows the LDS atomics and is unspecified.  The sort's
// only global atomics reserve list places for long segments' pieces (one per
// workgroup and window) and, for buckets of more than 65,536 terms, count and
// place their terms; the sums of long segments (more than 64 terms) are split
// into pieces added with float atomics, all other rows are stored once.  (A
// histogram of returning global atomics took 0.25 ms of the 4M-term
// workload; the four steps take 0.09 ms.)
//
// Destination row id of grad_out row g: (sa * p_ext + sp) * q_ext + sq, dense
// in [0, R) with R = ax_ext * p_ext * q_ext; -1 when the row has no in-range
// source.
__device__ __forceinline__ int32_t dest_row_id(const RowParams& p, int64_t g, int64_t& t_off) {
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
  t_off = o_ax * p.t_ax_b + op * p.t_p_b + oq * p.t_q_b;
  const bool ok = sa >= 0 && sa < p.ax_ext && sp >= 0 && sp < p.p_ext && sq >= 0 && sq < p.q_ext;
  return ok ? (int32_t)((sa * p.p_ext + sp) * p.q_ext + sq) : -1;
}

constexpr int kScanBlock = 1024;  // counts per scan block (256 threads x 4)

// exclusive scan within a workgroup of NT values (one per thread)
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t v, int32_t& total) {
  __shared__ int32_t s_w[NT / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  int32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wave ? s_w[w] : 0;
    total += s_w[w];
  }
  __syncthreads();
  return before + x - v;
}
__device__ __forceinline__ int32_t wg_exclusive_scan(int32_t v, int32_t& total) {
  return block_exclusive_scan<kThreads>(v, total);
}

// block b: sum of count[b*1024 .. b*1024+1023]
__global__ __launch_bounds__(kThreads) void seg_bsum_kernel(const int32_t* count, int64_t R, int32_t* bsum) {
  const int64_t i0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * 4;
  int32_t v = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (i0 + e < R) v += count[i0 + e];
  int32_t total;
  wg_exclusive_scan(v, total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// one workgroup: exclusive scan of the nb block sums in place (running carry)
__global__ __launch_bounds__(kThreads) void seg_bscan_kernel(int32_t* bsum, int64_t nb) {
  int32_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kThreads) {
    const int64_t i = b0 + threadIdx.x;
    const int32_t v = i < nb ? bsum[i] : 0;
    int32_t total;
    const int32_t ex = wg_exclusive_scan(v, total);
    if (i < nb) bsum[i] = carry + ex;
    carry += total;
  }
}

// Up to this many scan blocks, seg_offs sums the block sums before its own
// itself (each workgroup reads at most this many) instead of a separate
// one-workgroup scan launch: one launch fewer (about 4 us), both workloads.
constexpr int64_t kScanFuse = 4096;

// offs[i] = exclusive prefix of count; offs[R] = number of valid terms.
// bsum: the blocks' exclusive prefixes when `scanned`, else their sums.
__global__ __launch_bounds__(kThreads) void seg_offs_kernel(int32_t* count, int64_t R, const int32_t* bsum,
                                                            int32_t* offs, int scanned) {
  const int64_t i0 = (int64_t)blockIdx.x * kScanBlock + threadIdx.x * 4;
  int32_t c[4], v = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = i0 + e < R ? count[i0 + e] : 0;
    v += c[e];
  }
  int32_t base;
  if (scanned) {
    base = bsum[blockIdx.x];
  } else {
    int32_t part = 0;
    for (int64_t j = threadIdx.x; j < (int64_t)blockIdx.x; j += kThreads) part += bsum[j];
    wg_exclusive_scan(part, base);
  }
  int32_t total;
  int32_t run = base + wg_exclusive_scan(v, total);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (i0 + e < R) offs[i0 + e] = run;
    if (i0 + e == R - 1) offs[R] = run + c[e];
    run += c[e];
  }
}

constexpr int kChunk = 4096;                    // terms per workgroup in steps 1 and 3
constexpr int kChunkPer = kChunk / kThreads;    // 16 per lane
constexpr int kMaxBuckets = 4096;
constexpr int kWindow = 4096;                   // destination rows per pass in step 4
constexpr int kBuildThreads = 1024;
constexpr int kSegChunk = 64;                  // terms per reduce group; longer segments are split
constexpr int kMaxPieces = 4096;               // pieces of one segment at most
constexpr int kHotPairs = 16384;               // a bucket with more terms is built by many workgroups
                                               // (one workgroup takes ~50 us over 60,000 terms)
constexpr int kSlice = 16384;                  // terms per workgroup of a hot bucket
constexpr int kHotCountWorkgroups = 256;       // build-launch workgroups counting hot slices
constexpr int kSplitWorkgroups = 1024;         // workgroups on the long segments' pieces, at most
// Consecutive rounds of list entries per block of such a workgroup.  A block
// puts that many of a hot row's pieces (the longest ones) one after another
// on one workgroup, so more rounds save atomics but lengthen the slowest
// workgroup: Zipf(1.1) over 4M terms, pieces 642 us with one round per block,
// 619 / 608 / 619 with 2 / 3 / 4, 700 with 8, 929 with 16.
constexpr int kSplitRounds = 3;

// Terms per piece of a segment of c terms: kSegChunk, or longer for a row so
// hot that kSegChunk-term pieces would number more than kMaxPieces (their
// partial sums all meet in atomics on that one row).
__device__ __forceinline__ int32_t seg_piece(int32_t c) {
  return c <= kSegChunk * kMaxPieces ? kSegChunk : (c + kMaxPieces - 1) / kMaxPieces;
}

// Step 1: cnt1[b * n_chunks + w] = terms of chunk w whose row is in bucket b.
__global__ __launch_bounds__(kThreads) void seg_count_kernel(RowParams p, int shift, int nb, int64_t n_chunks,
                                                             int32_t* cnt1, int32_t* n_split, int32_t* n_hot,
                                                             int32_t* gcur, int64_t R) {
  __shared__ int32_t lh[kMaxBuckets];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) {  // the build appends long segments' pieces and hot buckets' slices
    *n_split = 0;
    *n_hot = 0;
  }
  // the hot buckets' per-row counters, added to by the build launch
  for (int64_t r = (int64_t)blockIdx.x * kThreads + tid; r < R; r += (int64_t)gridDim.x * kThreads) gcur[r] = 0;
  for (int b = tid; b < nb; b += kThreads) lh[b] = 0;
  __syncthreads();
  const int64_t g0 = (int64_t)blockIdx.x * kChunk;
#pragma unroll 4
  for (int i = 0; i < kChunkPer; ++i) {
    const int64_t g = g0 + i * kThreads + tid;
    if (g < p.n_rows) {
      int64_t t_off;
      const int32_t r = dest_row_id(p, g, t_off);
      if (r >= 0) atomicAdd(&lh[r >> shift], 1);
    }
  }
  __syncthreads();
  for (int b = tid; b < nb; b += kThreads) cnt1[(int64_t)b * n_chunks + blockIdx.x] = lh[b];
}

// Step 3: sort chunk w's terms by bucket in LDS and write each bucket's
// stretch of (row << 32 | term) pairs at its place pos1[b * n_chunks + w].
__global__ __launch_bounds__(kThreads) void seg_bucket_kernel(RowParams p, int shift, int nb, int64_t n_chunks,
                                                              const int32_t* pos1, uint64_t* pairs) {
  __shared__ int32_t lh[kMaxBuckets];  // counts; chunk-local starts; then place minus local start
  __shared__ uint64_t srt[kChunk];     // the chunk's pairs in bucket order
  const int tid = threadIdx.x;
  const int64_t w = blockIdx.x;
  for (int b = tid; b < nb; b += kThreads) lh[b] = 0;
  __syncthreads();
  const int64_t g0 = w * kChunk;
  int32_t rr[kChunkPer], rk[kChunkPer];
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    const int64_t g = g0 + i * kThreads + tid;
    rr[i] = -1;
    rk[i] = 0;
    if (g < p.n_rows) {
      int64_t t_off;
      rr[i] = dest_row_id(p, g, t_off);
      if (rr[i] >= 0) rk[i] = atomicAdd(&lh[rr[i] >> shift], 1);
    }
  }
  __syncthreads();
  // exclusive scan of lh[0, nb): lane t owns the per consecutive counts from t * per
  const int per = (nb + kThreads - 1) / kThreads;  // <= 16
  int32_t sum = 0;
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < nb) sum += lh[b];
  }
  int32_t total;
  int32_t run = wg_exclusive_scan(sum, total);
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < nb) {
      const int32_t c = lh[b];
      lh[b] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kChunkPer; ++i) {
    if (rr[i] >= 0) {
      const int64_t g = g0 + i * kThreads + tid;
      srt[lh[rr[i] >> shift] + rk[i]] = ((uint64_t)(uint32_t)rr[i] << 32) | (uint32_t)g;
    }
  }
  __syncthreads();
  // pair k of the sorted chunk, in bucket b, goes to pos1[b * n_chunks + w] + (k - local start of b)
  for (int e = 0; e < per; ++e) {
    const int b = tid * per + e;
    if (b < nb) lh[b] = pos1[(int64_t)b * n_chunks + w] - lh[b];
  }
  __syncthreads();
  for (int k = tid; k < total; k += kThreads) {
    const uint64_t pr = srt[k];
    pairs[(int64_t)lh[(int)(pr >> 32) >> shift] + k] = pr;
  }
}

// After a window's scan: list the pieces of this thread's rows
// w0 + kPer * tid + e whose segments are long (c[e] > kSegChunk), a row's
// pieces consecutive and in order; one global atomic per workgroup reserves
// the places (long rows can be many in a skewed bucket, and atomics on one
// counter serialize).  Each wavefront writes the entries of its own long
// rows: the form for buckets with few long rows.
template <int kPer>
__device__ __forceinline__ void list_pieces_waves(const int32_t (&c)[kPer], int64_t w0, uint64_t* split_list,
                                            int32_t* n_split) {
  __shared__ int32_t s_at;
  int32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e)
    if (c[e] > kSegChunk) mine += (c[e] + seg_piece(c[e]) - 1) / seg_piece(c[e]);
  int32_t total;
  int32_t at = block_exclusive_scan<kBuildThreads>(mine, total);
  if (total == 0) return;  // uniform: the same total in every thread
  if (threadIdx.x == 0) s_at = atomicAdd(n_split, total);
  __syncthreads();
  at += s_at;
  __syncthreads();  // s_at is read before the next window may set it
  // the entries are written by whole wavefronts, one long row at a time (a
  // hot row has up to kMaxPieces of them)
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int extra = c[e] > kSegChunk ? (c[e] + seg_piece(c[e]) - 1) / seg_piece(c[e]) : 0;
    for (uint64_t pend = __ballot(extra > 0); pend; pend &= pend - 1) {
      const int L = __builtin_ctzll(pend);
      const int n_e = __shfl(extra, L), at_e = __shfl(at, L);
      const int64_t row = w0 + (int64_t)((threadIdx.x & ~63) + L) * kPer + e;
      for (int q = lane; q < n_e; q += 64) split_list[at_e + q] = ((uint64_t)row << 32) | (uint32_t)q;
    }
    at += extra;
  }
}

// Pieces of a segment of c terms in the long-segment list (0 for a short one).
__device__ __forceinline__ int32_t seg_n_pieces(int32_t c) {
  return c > kSegChunk ? (c + seg_piece(c) - 1) / seg_piece(c) : 0;
}

// The same list for the window [w0, w0 + kWindow) of a hot bucket, whose
// rows can have up to kMaxPieces entries each, too many for one wavefront to
// write: c holds the terms of this thread's rows, the window's entries go to
// split_list[base ..), and this workgroup writes entries [share_lo,
// share_hi) of them -- a hot bucket's entries are shared out among its slice
// workgroups -- each thread finding an entry's row by binary search over the
// rows' first places in LDS.  Returns the window's number of entries (the
// same in every thread).
template <int kPer>
__device__ __forceinline__ int32_t list_pieces_share(const int32_t (&c)[kPer], int64_t w0, uint64_t* split_list,
                                                     int64_t base, int64_t share_num, int64_t share_den) {
  constexpr int kRows = kPer * kBuildThreads;
  static_assert(kRows == 1 << 12, "the binary search below takes 12 steps");
  __shared__ int32_t s_first[kRows];  // first place of each row's pieces, relative to base
  int32_t mine = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) mine += seg_n_pieces(c[e]);
  int32_t total;
  int32_t at = block_exclusive_scan<kBuildThreads>(mine, total);
  if (total == 0) return 0;  // uniform: the same total in every thread
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    s_first[threadIdx.x * kPer + e] = at;
    at += seg_n_pieces(c[e]);
  }
  __syncthreads();
  const int32_t lo = (int32_t)(total * share_num / share_den), hi = (int32_t)(total * (share_num + 1) / share_den);
  for (int32_t q = lo + (int32_t)threadIdx.x; q < hi; q += kBuildThreads) {
    // the entry's row: the last row whose first place is at or before q
    // (rows without pieces have an empty range and are passed over)
    int r0 = 0, r1 = kRows - 1;
#pragma unroll
    for (int step = 0; step < 12; ++step) {
      const int mid = (r0 + r1 + 1) >> 1;
      if (s_first[mid] <= q) r0 = mid; else r1 = mid - 1;
    }
    split_list[base + q] = ((uint64_t)(w0 + r0) << 32) | (uint32_t)(q - s_first[r0]);
  }
  __syncthreads();  // s_first is rewritten by the next window
  return total;
}

// Hot buckets, step 4 spread over workgroups: (a) each slice of kSlice terms
// counts its terms per row (LDS) and adds the counts into gcur (global
// atomics, one per row and slice) -- done by the build launch's extra
// workgroups while the other buckets build; (b) one workgroup per hot bucket
// scans the counts into segment offsets, sets gcur to them and reserves the
// long segments' piece entries; (c) each slice counts again, reserves its
// place in each row's segment with one global atomic per row, places its
// term ids and lists its share of the piece entries.  Slices are (bucket <<
// 32 | slice); step (c) strides over the *n_hot entries of hot_list.
struct HotSlice {
  int64_t p0, p1, row_lo, row_hi;
};
__device__ __forceinline__ HotSlice hot_slice(uint64_t e, int64_t R, int shift, int64_t n_chunks, const int32_t* pos1) {
  const int b = (int)(e >> 32), g = (int)(uint32_t)e;
  const int64_t s0 = pos1[(int64_t)b * n_chunks], s1 = pos1[(int64_t)(b + 1) * n_chunks];
  HotSlice h;
  h.p0 = s0 + (int64_t)g * kSlice;
  h.p1 = min(s1, h.p0 + kSlice);
  h.row_lo = (int64_t)b << shift;
  h.row_hi = min(R, (int64_t)(b + 1) << shift);
  return h;
}

// LDS counts of the slice's terms with rows in [w0, w0 + W)
__device__ __forceinline__ void hot_window_count(const uint64_t* pairs, int64_t p0, int64_t p1, int64_t w0, int64_t W,
                                                 int32_t* cnt) {
  constexpr int kU = 8;
  const int tid = threadIdx.x;
  for (int j = tid; j < kWindow; j += kBuildThreads) cnt[j] = 0;
  __syncthreads();
  for (int64_t i0 = p0; i0 < p1; i0 += kU * kBuildThreads) {
    uint64_t pr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + u * kBuildThreads + tid;
      pr[u] = i < p1 ? pairs[i] : ~uint64_t(0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t d = (int64_t)(pr[u] >> 32) - w0;
      if (d >= 0 && d < W) atomicAdd(&cnt[d], 1);
    }
  }
  __syncthreads();
}

// The build launch's workgroups past the buckets' count the hot buckets'
// terms per row into gcur (zeroed by seg_count), one kSlice-term slice at a
// time, while the other buckets build: each finds the slices from the bucket
// sizes -- the same slices the hot buckets' own workgroups list for
// seg_hot_place -- and takes every ne-th of them.
__device__ __forceinline__ void hot_count_role(int64_t R, int shift, int nb, int64_t n_chunks, const int32_t* pos1,
                                               const uint64_t* pairs, int32_t* gcur, int e, int ne, int32_t* cnt) {
  constexpr int kPer = kMaxBuckets / kBuildThreads;  // 4
  __shared__ int32_t s_first[kMaxBuckets];          // first slice of each bucket
  const int tid = threadIdx.x;
  int32_t ns[kPer], mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int bb = tid * kPer + q;
    ns[q] = 0;
    if (bb < nb) {
      const int64_t size = pos1[(int64_t)(bb + 1) * n_chunks] - pos1[(int64_t)bb * n_chunks];
      if (size > kHotPairs) ns[q] = (int32_t)((size + kSlice - 1) / kSlice);
    }
    mine += ns[q];
  }
  int32_t total;
  int32_t at = block_exclusive_scan<kBuildThreads>(mine, total);
  if (total == 0) return;  // uniform in the workgroup
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    s_first[tid * kPer + q] = at;
    at += ns[q];
  }
  __syncthreads();
  for (int k = e; k < total; k += ne) {
    // the slice's bucket: the last bucket whose first slice is at or before k
    int lo = 0, hi = kMaxBuckets - 1;
#pragma unroll
    for (int step = 0; step < 12; ++step) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_first[mid] <= k) lo = mid; else hi = mid - 1;
    }
    const HotSlice h = hot_slice(((uint64_t)lo << 32) | (uint32_t)(k - s_first[lo]), R, shift, n_chunks, pos1);
    for (int64_t w0 = h.row_lo; w0 < h.row_hi; w0 += kWindow) {
      const int64_t W = min((int64_t)kWindow, h.row_hi - w0);
      hot_window_count(pairs, h.p0, h.p1, w0, W, cnt);
      for (int j = tid; j < W; j += kBuildThreads)
        if (cnt[j]) atomicAdd(&gcur[w0 + j], cnt[j]);
      __syncthreads();
    }
  }
}

// Step 4: one workgroup per bucket.  Its pairs are pairs[s0, s1); its rows
// [b << shift, min((b + 1) << shift, R)) are taken kWindow at a time: count
// the terms per row, scan the counts into segment offsets (offs), then place
// each term id at its row's cursor (perm).  offs[R] = number of terms.
__global__ __launch_bounds__(kBuildThreads) void seg_build_kernel(int64_t R, int shift, int nb, int64_t n_chunks,
                                                                  const int32_t* pos1, const uint64_t* pairs,
                                                                  int32_t* offs, int32_t* perm,
                                                                  uint64_t* split_list, int32_t* n_split,
                                                                  int32_t* gcur, int32_t* hot, uint64_t* hot_list,
                                                                  int32_t* n_hot) {
  __shared__ int32_t cur[kWindow];
  constexpr int kPer = kWindow / kBuildThreads;  // 4
  constexpr int kU = 8;                          // pairs in flight per lane
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (b >= nb) {
    hot_count_role(R, shift, nb, n_chunks, pos1, pairs, gcur, b - nb, (int)gridDim.x - nb, cur);
    return;
  }
  const int64_t s0 = pos1[(int64_t)b * n_chunks], s1 = pos1[(int64_t)(b + 1) * n_chunks];
  const int64_t row_lo = (int64_t)b << shift;
  const int64_t row_hi = min(R, (int64_t)(b + 1) << shift);
  if (b == nb - 1 && tid == 0) offs[R] = (int32_t)s1;
  if (s1 - s0 > kHotPairs) {
    // a hot bucket: one workgroup would stream all its terms alone; it is
    // built with one workgroup per kSlice terms (counted by this launch's
    // extra workgroups, then seg_hot_scan and seg_hot_place).  List its
    // slices.
    if (tid == 0) {
      hot[b] = 1;
      const int ns = (int)((s1 - s0 + kSlice - 1) / kSlice);
      const int at = atomicAdd(n_hot, ns);
      for (int g = 0; g < ns; ++g) hot_list[at + g] = ((uint64_t)b << 32) | (uint32_t)g;
    }
    return;
  }
  if (tid == 0) hot[b] = 0;
  int64_t base = s0;
  for (int64_t w0 = row_lo; w0 < row_hi; w0 += kWindow) {
    const int64_t W = min((int64_t)kWindow, row_hi - w0);
    for (int j = tid; j < kWindow; j += kBuildThreads) cur[j] = 0;
    __syncthreads();
    for (int64_t i0 = s0; i0 < s1; i0 += kU * kBuildThreads) {
      uint64_t pr[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kBuildThreads + tid;
        pr[u] = i < s1 ? pairs[i] : ~uint64_t(0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t d = (int64_t)(pr[u] >> 32) - w0;  // the end marker gives d >= 2^31
        if (d >= 0 && d < W) atomicAdd(&cur[d], 1);
      }
    }
    __syncthreads();
    int32_t c[kPer], v = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      c[e] = cur[tid * kPer + e];
      v += c[e];
    }
    int32_t total;
    int32_t run = (int32_t)base + block_exclusive_scan<kBuildThreads>(v, total);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = tid * kPer + e;
      if (j < W) offs[w0 + j] = run;
      cur[j] = run;
      run += c[e];
    }
    list_pieces_waves(c, w0, split_list, n_split);
    __syncthreads();
    for (int64_t i0 = s0; i0 < s1; i0 += kU * kBuildThreads) {
      uint64_t pr[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kBuildThreads + tid;
        pr[u] = i < s1 ? pairs[i] : ~uint64_t(0);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t d = (int64_t)(pr[u] >> 32) - w0;
        if (d >= 0 && d < W) perm[atomicAdd(&cur[d], 1)] = (int32_t)(uint32_t)pr[u];
      }
    }
    base += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBuildThreads) void seg_hot_scan_kernel(int64_t R, int shift, int64_t n_chunks,
                                                                     const int32_t* pos1, int32_t* hot,
                                                                     int32_t* offs, int32_t* gcur, int32_t* n_split) {
  constexpr int kPer = kWindow / kBuildThreads;  // 4
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (!hot[b]) return;
  const int64_t s0 = pos1[(int64_t)b * n_chunks];
  const int64_t row_lo = (int64_t)b << shift;
  const int64_t row_hi = min(R, (int64_t)(b + 1) << shift);
  int64_t base = s0;
  int32_t pieces = 0;  // the bucket's long-segment pieces (this thread's rows)
  for (int64_t w0 = row_lo; w0 < row_hi; w0 += kWindow) {
    const int64_t W = min((int64_t)kWindow, row_hi - w0);
    int32_t c[kPer], v = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = tid * kPer + e;
      c[e] = j < W ? gcur[w0 + j] : 0;
      v += c[e];
      pieces += seg_n_pieces(c[e]);
    }
    int32_t total;
    int32_t run = (int32_t)base + block_exclusive_scan<kBuildThreads>(v, total);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = tid * kPer + e;
      if (j < W) {
        offs[w0 + j] = run;
        gcur[w0 + j] = run;
      }
      run += c[e];
    }
    base += total;
  }
  // one place in the piece list for all of the bucket's entries; the slice
  // workgroups of seg_hot_place write them.  hot[b] keeps that place + 1.
  int32_t n_pieces;
  block_exclusive_scan<kBuildThreads>(pieces, n_pieces);
  if (tid == 0) hot[b] = 1 + (n_pieces ? atomicAdd(n_split, n_pieces) : 0);
}

__global__ __launch_bounds__(kBuildThreads) void seg_hot_place_kernel(int64_t R, int shift, int64_t n_chunks,
                                                                      const int32_t* pos1, const uint64_t* pairs,
                                                                      const uint64_t* hot_list, const int32_t* n_hot,
                                                                      const int32_t* hot, const int32_t* offs,
                                                                      int32_t* gcur, int32_t* perm,
                                                                      uint64_t* split_list) {
  __shared__ int32_t cnt[kWindow];
  constexpr int kU = 8;
  constexpr int kPer = kWindow / kBuildThreads;  // 4
  const int tid = threadIdx.x;
  const int nh = *n_hot;
  for (int e = blockIdx.x; e < nh; e += gridDim.x) {
    const HotSlice h = hot_slice(hot_list[e], R, shift, n_chunks, pos1);
    // this slice's share of the bucket's long-segment piece list: segment
    // lengths from the offsets the scan wrote, entries from the place it
    // reserved (one share per slice, so a bucket of many slices -- the
    // hottest rows' thousands of pieces -- is listed by as many workgroups)
    {
      const int b = (int)(hot_list[e] >> 32), g = (int)(uint32_t)hot_list[e];
      const int64_t s0 = pos1[(int64_t)b * n_chunks], s1 = pos1[(int64_t)(b + 1) * n_chunks];
      const int64_t ns = (s1 - s0 + kSlice - 1) / kSlice;
      int64_t base = hot[b] - 1;
      for (int64_t w0 = h.row_lo; w0 < h.row_hi; w0 += kWindow) {
        const int64_t W = min((int64_t)kWindow, h.row_hi - w0);
        int32_t c[kPer];
#pragma unroll
        for (int q = 0; q < kPer; ++q) {
          const int j = tid * kPer + q;
          c[q] = j < W ? offs[w0 + j + 1] - offs[w0 + j] : 0;
        }
        base += list_pieces_share(c, w0, split_list, base, g, ns);
      }
    }
    for (int64_t w0 = h.row_lo; w0 < h.row_hi; w0 += kWindow) {
      const int64_t W = min((int64_t)kWindow, h.row_hi - w0);
      hot_window_count(pairs, h.p0, h.p1, w0, W, cnt);
      for (int j = tid; j < W; j += kBuildThreads)
        if (cnt[j]) cnt[j] = atomicAdd(&gcur[w0 + j], cnt[j]);  // this slice's place in the row's segment
      __syncthreads();
      for (int64_t i0 = h.p0; i0 < h.p1; i0 += kU * kBuildThreads) {
        uint64_t pr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t i = i0 + u * kBuildThreads + tid;
          pr[u] = i < h.p1 ? pairs[i] : ~uint64_t(0);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int64_t d = (int64_t)(pr[u] >> 32) - w0;
          if (d >= 0 && d < W) perm[atomicAdd(&cnt[d], 1)] = (int32_t)(uint32_t)pr[u];
        }
      }
      __syncthreads();
    }
  }
}

// Byte offset in grad_out of the tile row g (dest_row_id's t_off, without
// the index lookup).
__device__ __forceinline__ int64_t grad_row_off(const RowParams& p, int64_t g) {
  if (p.rest == 1) return g * p.t_ax_b;
  const int64_t o_ax = g / p.rest, rr = g - o_ax * p.rest;
  const int64_t op = rr / p.q_n, oq = rr - op * p.q_n;
  return o_ax * p.t_ax_b + op * p.t_p_b + oq * p.t_q_b;
}

constexpr int kSegBatch = 4;  // grad_out rows in flight per lane in a segment sum

// grad_out rows of segment terms k .. k+kSegBatch-1, read from perm;
// positions at or past ke repeat term ke - 1 (the caller has kb <= ke - 1),
// so the reads stay inside the segment and need no branch.
__device__ __forceinline__ void seg_batch_perm(const int32_t* perm, int32_t k, int32_t ke, int32_t (&g)[kSegBatch]) {
#pragma unroll
  for (int q = 0; q < kSegBatch; ++q) g[q] = perm[min(k + q, ke - 1)];
}

// The 16-byte chunk at byte b of a row, restricted to the valid byte window
// [lo_b, hi_b): one non-temporal 16-byte read for a chunk inside the window
// (every chunk, when ALIGNED: both window edges are multiples of 16), element
// reads for a chunk on its edge, elements outside the window reading as 0.
template <int ESIZE, bool ALIGNED>
__device__ __forceinline__ u32x4 seg_ld_chunk(const RowParams& p, const char* row, int b) {
  constexpr int V = 16 / ESIZE;
  if (ALIGNED || (b >= p.lo_b && b + 16 <= p.hi_b)) return ld16_nt(row + b);
  u32x4 v = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const int bb = b + e * ESIZE;
    if (bb >= p.lo_b && bb < p.hi_b) vec_set<ESIZE>(v, e, load_elem<ESIZE>(row + bb));
  }
  return v;
}

// Sum of terms [kb, ke) of a destination row's segment (kb < ke) over the
// 16-byte chunk at byte b of the row's window, in term order, starting from
// a.grad's values (arow) when init, else from zero; returns the sum's bits.
// kSegBatch grad_out rows are in flight at once and the next kSegBatch perm
// entries are read while they are, so the loop waits on one memory latency
// per batch.  (Reading a perm entry and its row one term at a time made each
// term wait for two latencies in a row: vector memory reads complete in
// order, and each perm read queued behind the previous term's row read.)
template <int ESIZE, bool ALIGNED>
__device__ __forceinline__ u32x4 seg_chunk_sum_w(const RowParams& p, const int32_t* perm, const char* arow, int32_t kb,
                                                 int32_t ke, int b, bool init) {
  constexpr int V = 16 / ESIZE;
  u32x4 a0 = {0, 0, 0, 0};
  if (init) a0 = seg_ld_chunk<ESIZE, ALIGNED>(p, arow, b);
  int32_t g[kSegBatch];
  seg_batch_perm(perm, kb, ke, g);
  float accf[V];
  double acc[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    accf[e] = __uint_as_float((uint32_t)vec_get<ESIZE>(a0, e));
    acc[e] = __longlong_as_double((long long)vec_get<ESIZE>(a0, e));
  }
  for (int32_t k = kb; k < ke; k += kSegBatch) {
    u32x4 v[kSegBatch];
#pragma unroll
    for (int q = 0; q < kSegBatch; ++q)
      v[q] = k + q < ke ? seg_ld_chunk<ESIZE, ALIGNED>(p, p.t + grad_row_off(p, g[q]), b) : (u32x4){0, 0, 0, 0};
    seg_batch_perm(perm, k + kSegBatch, ke, g);
#pragma unroll
    for (int q = 0; q < kSegBatch; ++q) {
      if (k + q >= ke) break;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint64_t bits = vec_get<ESIZE>(v[q], e);
        if (ESIZE == 4)
          accf[e] += __uint_as_float((uint32_t)bits);
        else
          acc[e] += __longlong_as_double((long long)bits);
      }
    }
  }
  u32x4 out = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < V; ++e)
    vec_set<ESIZE>(out, e, ESIZE == 4 ? (uint64_t)__float_as_uint(accf[e]) : (uint64_t)__double_as_longlong(acc[e]));
  return out;
}

template <int ESIZE>
__device__ __forceinline__ u32x4 seg_chunk_sum(const RowParams& p, const int32_t* perm, const char* arow, int32_t kb,
                                               int32_t ke, int b, bool init) {
  return ((p.lo_b | p.hi_b) & 15) == 0 ? seg_chunk_sum_w<ESIZE, true>(p, perm, arow, kb, ke, b, init)
                                       : seg_chunk_sum_w<ESIZE, false>(p, perm, arow, kb, ke, b, init);
}

// Write a chunk sum into a.grad: plain stores (store) or float atomics adding
// a partial sum (the row's segment is split over several groups).
template <int ESIZE>
__device__ __forceinline__ void seg_chunk_out(const RowParams& p, char* arow, int b, u32x4 out, bool store) {
  constexpr int V = 16 / ESIZE;
  if (!store) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int bb = b + e * ESIZE;
      if (bb >= p.lo_b && bb < p.hi_b) accum_elem<ESIZE>(arow + bb, vec_get<ESIZE>(out, e));
    }
  } else if (b >= p.lo_b && b + 16 <= p.hi_b) {
    st16_nt(arow + b, out);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int bb = b + e * ESIZE;
      if (bb >= p.lo_b && bb < p.hi_b) store_elem<ESIZE>(arow + bb, vec_get<ESIZE>(out, e));
    }
  }
}

// First 16-byte chunk of lane `sub` of a group of LPR lanes; the lane then
// takes every LPR-th chunk of the row's valid window.
__device__ __forceinline__ int seg_first_b(const RowParams& p, int sub) { return p.lo_b - p.lo_b % 16 + sub * 16; }

// Terms [kb, ke) of a destination row's segment, summed by one group of LPR
// lanes, each lane over its chunks of the row.  init: start from a.grad's
// values and store the row (plain stores); otherwise start from zero and add
// the partial sums into a.grad with float atomics.
template <int ESIZE, int LPR>
__device__ __forceinline__ void seg_sum_terms(const RowParams& p, const int32_t* perm, char* arow, int32_t kb,
                                              int32_t ke, int sub, bool init) {
  for (int b = seg_first_b(p, sub); b < p.hi_b; b += LPR * 16)
    seg_chunk_out<ESIZE>(p, arow, b, seg_chunk_sum<ESIZE>(p, perm, arow, kb, ke, b, init), init);
}

__device__ __forceinline__ char* seg_arow(const RowParams& p, int64_t r) {
  if (p.q_ext == 1 && p.p_ext == 1) return const_cast<char*>(p.a) + r * p.a_ax_b + p.a_col_b;
  const int64_t sq = r % p.q_ext, rr = r / p.q_ext;
  const int64_t sp = rr % p.p_ext, sa = rr / p.p_ext;
  return const_cast<char*>(p.a) + sa * p.a_ax_b + sp * p.a_p_b + sq * p.a_q_b + p.a_col_b;
}

constexpr int kRowsPerGroup = 4;  // consecutive destination rows per group in the reduce (a Four<>)

// Four values picked by a lane-varying index with selects: a register array
// indexed that way is placed in scratch memory.
template <class T>
struct Four {
  T x0, x1, x2, x3;
  __device__ __forceinline__ T pick(int i) const { return i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : x3; }
};

// Row (0 .. kRowsPerGroup - 1) of term kk of a group's stream.
__device__ __forceinline__ int seg_row_of(const int32_t (&o)[kRowsPerGroup + 1], int32_t kk) {
  int jj = 0;
#pragma unroll
  for (int m = 1; m < kRowsPerGroup; ++m) jj += kk >= o[m];
  return jj;
}

template <int ESIZE>
__device__ __forceinline__ void seg_acc_start(const u32x4& a0, float (&accf)[16 / ESIZE], double (&acc)[16 / ESIZE]) {
#pragma unroll
  for (int e = 0; e < 16 / ESIZE; ++e) {
    accf[e] = __uint_as_float((uint32_t)vec_get<ESIZE>(a0, e));
    acc[e] = __longlong_as_double((long long)vec_get<ESIZE>(a0, e));
  }
}

template <int ESIZE>
__device__ __forceinline__ u32x4 seg_acc_bits(const float (&accf)[16 / ESIZE], const double (&acc)[16 / ESIZE]) {
  u32x4 out = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 16 / ESIZE; ++e)
    vec_set<ESIZE>(out, e, ESIZE == 4 ? (uint64_t)__float_as_uint(accf[e]) : (uint64_t)__double_as_longlong(acc[e]));
  return out;
}

// The segments of kRowsPerGroup consecutive destination rows lie back to
// back in perm, [o[0], o[kRowsPerGroup]), and are summed here as one stream
// of terms over the 16-byte chunk at byte b: batches of grad_out rows stay in
// flight across row boundaries, and each row, once its last term is added,
// is stored from a.grad's value plus its terms in term order.  Rows with an
// empty segment are not touched.  (One row per group left the rows' reads
// idle while the group waited on the row's offsets and then its perm
// entries.)
template <int ESIZE, bool ALIGNED>
__device__ __forceinline__ void seg_stream_chunk(const RowParams& p, const int32_t* perm,
                                                 const int32_t (&o)[kRowsPerGroup + 1],
                                                 const Four<char*>& arow, int b) {
  constexpr int V = 16 / ESIZE;
  const int32_t kb = o[0], ke = o[kRowsPerGroup];
  if (kb >= ke) return;
  const u32x4 z = {0, 0, 0, 0};
  const Four<u32x4> init = {o[1] > o[0] ? seg_ld_chunk<ESIZE, ALIGNED>(p, arow.x0, b) : z,
                            o[2] > o[1] ? seg_ld_chunk<ESIZE, ALIGNED>(p, arow.x1, b) : z,
                            o[3] > o[2] ? seg_ld_chunk<ESIZE, ALIGNED>(p, arow.x2, b) : z,
                            o[4] > o[3] ? seg_ld_chunk<ESIZE, ALIGNED>(p, arow.x3, b) : z};
  int32_t g[kSegBatch];
  seg_batch_perm(perm, kb, ke, g);
  float accf[V];
  double acc[V];
  int cur = seg_row_of(o, kb);
  seg_acc_start<ESIZE>(init.pick(cur), accf, acc);
  for (int32_t k = kb; k < ke; k += kSegBatch) {
    u32x4 v[kSegBatch];
#pragma unroll
    for (int q = 0; q < kSegBatch; ++q)
      v[q] = k + q < ke ? seg_ld_chunk<ESIZE, ALIGNED>(p, p.t + grad_row_off(p, g[q]), b) : (u32x4){0, 0, 0, 0};
    seg_batch_perm(perm, k + kSegBatch, ke, g);
#pragma unroll
    for (int q = 0; q < kSegBatch; ++q) {
      if (k + q >= ke) break;
      const int jj = seg_row_of(o, k + q);
      if (jj != cur) {
        seg_chunk_out<ESIZE>(p, arow.pick(cur), b, seg_acc_bits<ESIZE>(accf, acc), true);
        cur = jj;
        seg_acc_start<ESIZE>(init.pick(cur), accf, acc);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint64_t bits = vec_get<ESIZE>(v[q], e);
        if (ESIZE == 4)
          accf[e] += __uint_as_float((uint32_t)bits);
        else
          acc[e] += __longlong_as_double((long long)bits);
      }
    }
  }
  seg_chunk_out<ESIZE>(p, arow.pick(cur), b, seg_acc_bits<ESIZE>(accf, acc), true);
}

// One group of LPR lanes per kRowsPerGroup consecutive destination rows sums
// each row's segment onto a.grad's values and stores the row once.  A
// segment longer than kSegChunk terms is left to seg_split_wg, which adds
// its pieces onto a.grad with float atomics; a group holding such a row takes
// its other rows one at a time.  Rows with an empty segment are not touched.
template <int ESIZE, int LPR>
__device__ __forceinline__ void seg_reduce_wg(const RowParams& p, int64_t R, const int32_t* offs, const int32_t* perm,
                                              int64_t wg) {
  const int sub = threadIdx.x % LPR;
  const int64_t r0 = (wg * (kThreads / LPR) + threadIdx.x / LPR) * kRowsPerGroup;
  if (r0 >= R) return;
  int32_t o[kRowsPerGroup + 1];
#pragma unroll
  for (int j = 0; j <= kRowsPerGroup; ++j) o[j] = offs[min(r0 + j, R)];
  if (o[0] == o[kRowsPerGroup]) return;  // no terms
  bool longseg = false;
#pragma unroll
  for (int j = 0; j < kRowsPerGroup; ++j) longseg = longseg || o[j + 1] - o[j] > kSegChunk;
  // rows past R have empty segments and are never read or written
  const Four<char*> arow = {seg_arow(p, r0), seg_arow(p, min(r0 + 1, R - 1)), seg_arow(p, min(r0 + 2, R - 1)),
                            seg_arow(p, min(r0 + 3, R - 1))};
  if (longseg) {
#pragma unroll
    for (int j = 0; j < kRowsPerGroup; ++j) {
      const int32_t k0 = o[j], k1 = o[j + 1];
      if (k0 == k1 || k1 - k0 > kSegChunk) continue;
      seg_sum_terms<ESIZE, LPR>(p, perm, arow.pick(j), k0, k1, sub, true);
    }
    return;
  }
  const bool aligned = ((p.lo_b | p.hi_b) & 15) == 0;
  for (int b = seg_first_b(p, sub); b < p.hi_b; b += LPR * 16) {
    if (aligned)
      seg_stream_chunk<ESIZE, true>(p, perm, o, arow, b);
    else
      seg_stream_chunk<ESIZE, false>(p, perm, o, arow, b);
  }
}

// Elementwise sum of two chunk sums.
template <int ESIZE>
__device__ __forceinline__ u32x4 seg_add(u32x4 a, const u32x4& x) {
#pragma unroll
  for (int el = 0; el < 16 / ESIZE; ++el) {
    if (ESIZE == 4)
      vec_set<4>(a, el, __float_as_uint(__uint_as_float((uint32_t)vec_get<4>(a, el)) +
                                        __uint_as_float((uint32_t)vec_get<4>(x, el))));
    else
      vec_set<8>(a, el, (uint64_t)__double_as_longlong(__longlong_as_double((long long)vec_get<8>(a, el)) +
                                                       __longlong_as_double((long long)vec_get<8>(x, el))));
  }
  return a;
}

// The pieces of long segments, from the list the segment build wrote:
// entry (row << 32 | piece), piece >= 0; *n_split entries, a row's pieces
// consecutive.  A workgroup takes blocks of kSplitRounds rounds of
// kThreads / LPR consecutive entries, one entry per group and round, the
// blocks strided over the workgroups.  When a round's entries all belong to
// one row (the common case for a hot row), the groups' partial sums are added
// together in LDS; for rows one pass of a group's lanes covers, that sum is
// also carried from round to round while the row stays the same, and goes out
// in one set of atomics when it changes.  A hot row's elements then meet one
// set of atomics per workgroup and block instead of one per round (the
// hottest rows' 4096 pieces had met in 512 atomic sets on each element).
template <int ESIZE, int LPR>
__device__ __forceinline__ void seg_split_wg(const RowParams& p, const int32_t* offs, const int32_t* perm,
                                             const uint64_t* split_list, const int32_t* n_split, int64_t wg,
                                             int64_t n_wg) {
  constexpr int G = kThreads / LPR;  // groups per workgroup
  constexpr int B = kSplitRounds * G;  // entries per block
  __shared__ u32x4 part[G][LPR];
  __shared__ int64_t s_row[G];
  const int sub = threadIdx.x % LPR, grp = threadIdx.x / LPR;
  const int n = *n_split;
  const bool single_b = p.hi_b <= seg_first_b(p, 0) + LPR * 16;
  const int bc = seg_first_b(p, 0) + sub * 16;  // this lane's chunk when single_b
  int64_t carry_row = -1;                       // row of the carried sum (group 0's lanes hold it)
  u32x4 carry = {0, 0, 0, 0};
  for (int64_t blk = wg * B; blk < n; blk += n_wg * B) {
    for (int64_t e0 = blk; e0 < blk + B && e0 < n; e0 += G) {
      const int64_t g = e0 + grp;
      int64_t r = -1;
      int32_t kb = 0, ke = 0;
      if (g < n) {
        const uint64_t e = split_list[g];
        r = (int64_t)(e >> 32);
        const int32_t piece = (int32_t)(uint32_t)e;
        const int32_t len = seg_piece(offs[r + 1] - offs[r]);
        kb = offs[r] + piece * len;
        ke = min(offs[r + 1], kb + len);
      }
      if (sub == 0) s_row[grp] = r;
      __syncthreads();
      // partly unrolled here and in the sums below: with 32 groups (LPR 8) a
      // full unroll holds every group's value in registers at once
      bool one_row = true;
#pragma unroll 4
      for (int q = 1; q < G; ++q) one_row = one_row && s_row[q] == s_row[0];
      if (one_row && single_b) {  // every entry valid and of one row, one chunk per lane
        part[grp][sub] = bc < p.hi_b ? seg_chunk_sum<ESIZE>(p, perm, seg_arow(p, r), kb, ke, bc, false)
                                     : (u32x4){0, 0, 0, 0};
        __syncthreads();
        if (grp == 0) {
          u32x4 sum = part[0][sub];
#pragma unroll 4
          for (int q = 1; q < G; ++q) sum = seg_add<ESIZE>(sum, part[q][sub]);
          if (r == carry_row) {
            carry = seg_add<ESIZE>(carry, sum);
          } else {
            if (carry_row >= 0 && bc < p.hi_b) seg_chunk_out<ESIZE>(p, seg_arow(p, carry_row), bc, carry, false);
            carry = sum;
          }
        }
        carry_row = r;  // the same in every lane
      } else if (one_row) {
        char* arow = seg_arow(p, r);
        // the same trip count in every lane (barriers inside): lanes whose
        // chunk lies past the window add zeros and write nothing
        for (int b0 = seg_first_b(p, 0); b0 < p.hi_b; b0 += LPR * 16) {
          const int b = b0 + sub * 16;
          part[grp][sub] = b < p.hi_b ? seg_chunk_sum<ESIZE>(p, perm, arow, kb, ke, b, false) : (u32x4){0, 0, 0, 0};
          __syncthreads();
          if (grp == 0 && b < p.hi_b) {
            u32x4 sum = part[0][sub];
#pragma unroll 4
            for (int q = 1; q < G; ++q) sum = seg_add<ESIZE>(sum, part[q][sub]);
            seg_chunk_out<ESIZE>(p, arow, b, sum, false);
          }
          __syncthreads();
        }
      } else if (r >= 0) {
        seg_sum_terms<ESIZE, LPR>(p, perm, seg_arow(p, r), kb, ke, sub, false);
      }
      __syncthreads();  // s_row and part are rewritten by the next round
    }
  }
  // the last carried sum (atomics commute with the ones issued meanwhile)
  if (grp == 0 && carry_row >= 0 && bc < p.hi_b) seg_chunk_out<ESIZE>(p, seg_arow(p, carry_row), bc, carry, false);
}

// Both sums in one launch: workgroups [0, n_split_wg) take the pieces of the
// long segments (grid-striding over the list), the rest take the short
// segments, kThreads / LPR groups of kRowsPerGroup rows each.  The two touch
// disjoint destination rows (a row's segment is either short or split), so
// nothing orders them, and the short segments' groups fill the slots the
// pieces leave free instead of waiting for the last piece.
template <int ESIZE, int LPR>
__global__ __launch_bounds__(kThreads) void seg_sum_kernel(RowParams p, int64_t R, const int32_t* offs,
                                                           const int32_t* perm, const uint64_t* split_list,
                                                           const int32_t* n_split, int n_split_wg) {
  if ((int)blockIdx.x < n_split_wg)
    seg_split_wg<ESIZE, LPR>(p, offs, perm, split_list, n_split, blockIdx.x, n_split_wg);
  else
    seg_reduce_wg<ESIZE, LPR>(p, R, offs, perm, (int64_t)blockIdx.x - n_split_wg);
}

// ---- host side -------------------------------------------------------------

enum class Op { Gather, GatherMasked, Scatter, GatherBackward };

const char* op_name(Op op) {
  return op == Op::Gather         ? "tile_gather"
         : op == Op::GatherMasked ? "tile_gather_masked"
         : op == Op::Scatter      ? "tile_scatter_masked"
                                  : "tile_gather_backward";
}

int launch_rows(Op op, int esize, const RowParams& p, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b(kThreads);
  const bool full = p.lo_b == 0 && p.hi_b == p.row_bytes && p.row_bytes % 16 == 0;
#define STG_ROWS(K, E) \
  full ? launch_kernel(op_name(op), K<E, true>, g, b, 0, s, p) : launch_kernel(op_name(op), K<E, false>, g, b, 0, s, p)
#define STG_ROWS_S(E, A)                                                                        \
  full ? launch_kernel(op_name(op), scatter_rows_kernel<E, true, A>, g, b, 0, s, p)              \
       : launch_kernel(op_name(op), scatter_rows_kernel<E, false, A>, g, b, 0, s, p)
  if (op == Op::GatherBackward) {
    if (esize == 4)
      STG_ROWS_S(4, true);
    else
      STG_ROWS_S(8, true);
  } else if (op == Op::Scatter) {
    switch (esize) {
      case 1: STG_ROWS_S(1, false); break;
      case 2: STG_ROWS_S(2, false); break;
      case 4: STG_ROWS_S(4, false); break;
      default: STG_ROWS_S(8, false); break;
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
#undef STG_ROWS_S
  return check_launch(op_name(op));
}

int launch_elems(Op op, int esize, const ElemParams& p, hipStream_t s) {
  const int64_t want = (p.n + kThreads - 1) / kThreads;
  const dim3 g((unsigned)(want < 65536 ? want : 65536)), b(kThreads);
  if (op == Op::GatherBackward) {
    if (esize == 4)
      launch_kernel(op_name(op), scatter_elem_kernel<4, true>, g, b, 0, s, p);
    else
      launch_kernel(op_name(op), scatter_elem_kernel<8, true>, g, b, 0, s, p);
  } else if (op == Op::Scatter) {
    switch (esize) {
      case 1: launch_kernel(op_name(op), scatter_elem_kernel<1, false>, g, b, 0, s, p); break;
      case 2: launch_kernel(op_name(op), scatter_elem_kernel<2, false>, g, b, 0, s, p); break;
      case 4: launch_kernel(op_name(op), scatter_elem_kernel<4, false>, g, b, 0, s, p); break;
      default: launch_kernel(op_name(op), scatter_elem_kernel<8, false>, g, b, 0, s, p); break;
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

// Segmented backward: workspace layout and size (bytes) for R destination
// rows and n_rows grad_out rows.
struct SegLayout {
  int shift;                   // bucket = destination row >> shift
  int64_t nbk, n_chunks, L1;   // buckets, term chunks of kChunk, nbk * n_chunks
  int64_t nb1;                 // scan blocks over the L1 counts
  int64_t n_pieces;            // capacity of the long-segment piece list
  int64_t n_slices;            // capacity of the hot-bucket slice list
  int64_t offs, perm, pairs, cnt1, pos1, bsum, split, n_split, gcur, hot, hot_list, n_hot, bytes;  // byte offsets
};

// Workspace: offs int32[R + 1] | perm int32[n_rows] | pairs uint64[n_rows] |
// cnt1 int32[L1] | pos1 int32[L1 + 1] | bsum int32[nb1] | split uint64[2 * n_rows
// / kSegChunk + 1] | n_split int32 | gcur int32[R] | hot int32[nbk] | hot_list
// uint64[n_rows / kSlice + n_rows / kHotPairs + 1] | n_hot int32, each 256-byte
// aligned.
// At most 512 buckets while they span at most kWindow rows (R <= 2^21), then
// up to kMaxBuckets of kWindow rows (R <= 2^24); past that, kMaxBuckets
// buckets of several windows each.
SegLayout seg_layout(int64_t R, int64_t n_rows) {
  SegLayout L;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  int lg = 0;
  while ((int64_t(1) << lg) < R) ++lg;
  L.shift = lg > 9 ? lg - 9 : 0;
  if (L.shift > 12) L.shift = std::max(12, lg - 12);
  L.nbk = R > 0 ? ((R - 1) >> L.shift) + 1 : 0;
  L.n_chunks = (n_rows + kChunk - 1) / kChunk;
  L.L1 = L.nbk * L.n_chunks;
  L.nb1 = (L.L1 + kScanBlock - 1) / kScanBlock;
  L.offs = 0;
  L.perm = up(L.offs + (R + 1) * 4);
  L.pairs = up(L.perm + n_rows * 4);
  L.cnt1 = up(L.pairs + n_rows * 8);
  L.pos1 = up(L.cnt1 + L.L1 * 4);
  L.bsum = up(L.pos1 + (L.L1 + 1) * 4);
  L.n_pieces = 2 * n_rows / kSegChunk + 1;  // ceil(c / piece) < 2 c / kSegChunk for c > kSegChunk
  L.n_slices = n_rows / kSlice + n_rows / kHotPairs + 1;
  L.split = up(L.bsum + L.nb1 * 4);
  L.n_split = up(L.split + L.n_pieces * 8);
  L.gcur = up(L.n_split + 4);
  L.hot = up(L.gcur + R * 4);
  L.hot_list = up(L.hot + L.nbk * 4);
  L.n_hot = up(L.hot_list + L.n_slices * 8);
  L.bytes = up(L.n_hot + 4);
  return L;
}

int launch_segmented(const char* name, int esize, const RowParams& p, int64_t R, char* ws, hipStream_t s) {
  const SegLayout L = seg_layout(R, p.n_rows);
  if (L.L1 >= INT32_MAX)
    return fail(STG_ERR_RANGE, "%s: %lld destination rows with %lld terms exceed the grouped path's tables", name,
                (long long)R, (long long)p.n_rows);
  if (p.n_rows == 0) return STG_OK;  // nothing to add
  int32_t* offs = (int32_t*)(ws + L.offs);
  int32_t* perm = (int32_t*)(ws + L.perm);
  uint64_t* pairs = (uint64_t*)(ws + L.pairs);
  int32_t* cnt1 = (int32_t*)(ws + L.cnt1);
  int32_t* pos1 = (int32_t*)(ws + L.pos1);
  int32_t* bsum = (int32_t*)(ws + L.bsum);
  uint64_t* split = (uint64_t*)(ws + L.split);
  int32_t* n_split = (int32_t*)(ws + L.n_split);
  int32_t* gcur = (int32_t*)(ws + L.gcur);
  int32_t* hot = (int32_t*)(ws + L.hot);
  uint64_t* hot_list = (uint64_t*)(ws + L.hot_list);
  int32_t* n_hot = (int32_t*)(ws + L.n_hot);
  const int nbk = (int)L.nbk;
  const dim3 chunks((unsigned)L.n_chunks), blk(kThreads);
  launch_kernel("tile_gather_backward/count", seg_count_kernel, chunks, blk, 0, s, p, L.shift, nbk, L.n_chunks, cnt1,
                n_split, n_hot, gcur, R);
  launch_kernel("tile_gather_backward/bsum", seg_bsum_kernel, dim3((unsigned)L.nb1), blk, 0, s, (const int32_t*)cnt1,
                L.L1, bsum);
  const int scanned = L.nb1 > kScanFuse;
  if (scanned) launch_kernel("tile_gather_backward/bscan", seg_bscan_kernel, dim3(1), blk, 0, s, bsum, L.nb1);
  launch_kernel("tile_gather_backward/offs", seg_offs_kernel, dim3((unsigned)L.nb1), blk, 0, s, cnt1, L.L1,
                (const int32_t*)bsum, pos1, scanned);
  launch_kernel("tile_gather_backward/bucket", seg_bucket_kernel, chunks, blk, 0, s, p, L.shift, nbk, L.n_chunks,
                (const int32_t*)pos1, pairs);
  // one workgroup per bucket, then kHotCountWorkgroups counting the hot
  // buckets' slices (usually none)
  launch_kernel("tile_gather_backward/build", seg_build_kernel, dim3((unsigned)(nbk + kHotCountWorkgroups)),
                dim3(kBuildThreads), 0, s, R,
                L.shift, nbk, L.n_chunks, (const int32_t*)pos1, (const uint64_t*)pairs, offs, perm, split, n_split,
                gcur, hot, hot_list, n_hot);
  // hot buckets (more than kHotPairs terms): many workgroups each; the
  // slice kernels stride over the list the build wrote (usually empty)
  const dim3 hgrid(256), hblk(kBuildThreads);
  launch_kernel("tile_gather_backward/hot_scan", seg_hot_scan_kernel, dim3((unsigned)nbk), hblk, 0, s, R, L.shift,
                L.n_chunks, (const int32_t*)pos1, hot, offs, gcur, n_split);
  launch_kernel("tile_gather_backward/hot_place", seg_hot_place_kernel, hgrid, hblk, 0, s, R, L.shift, L.n_chunks,
                (const int32_t*)pos1, (const uint64_t*)pairs, (const uint64_t*)hot_list, (const int32_t*)n_hot,
                (const int32_t*)hot, (const int32_t*)offs, gcur, perm, split);
  // lanes per destination row: enough for the row's chunks, at most a wavefront
  const int chunks_per_row = p.n_chunks;
  const int lpr = chunks_per_row <= 8 ? 8 : chunks_per_row <= 16 ? 16 : chunks_per_row <= 32 ? 32 : 64;
  const int64_t rows_per_wg = (int64_t)(kThreads / lpr) * kRowsPerGroup;
  // workgroups for the long segments' pieces, striding over the list the
  // build wrote (empty unless a row takes more than kSegChunk terms); they
  // come first in the grid, so the long-running ones start first
  const int64_t gpw = kThreads / lpr;
  const int n_split_wg = (int)std::min<int64_t>((L.n_pieces + gpw - 1) / gpw, kSplitWorkgroups);
  const int64_t reduce_wg = (R + rows_per_wg - 1) / rows_per_wg;
  if (n_split_wg + reduce_wg > INT32_MAX)
    return fail(STG_ERR_RANGE, "%s: %lld destination rows need more workgroups than one launch holds", name,
                (long long)R);
  const dim3 sgrid((unsigned)(n_split_wg + reduce_wg));
#define STG_SEG(E, LP)                                                                                               \
  launch_kernel("tile_gather_backward/sum", seg_sum_kernel<E, LP>, sgrid, dim3(kThreads), 0, s, p, R,                \
                (const int32_t*)offs, (const int32_t*)perm, (const uint64_t*)split, (const int32_t*)n_split,        \
                n_split_wg)
  if (esize == 4) {
    if (lpr == 8) STG_SEG(4, 8); else if (lpr == 16) STG_SEG(4, 16); else if (lpr == 32) STG_SEG(4, 32); else STG_SEG(4, 64);
  } else {
    if (lpr == 8) STG_SEG(8, 8); else if (lpr == 16) STG_SEG(8, 16); else if (lpr == 32) STG_SEG(8, 32); else STG_SEG(8, 64);
  }
#undef STG_SEG
  return check_launch(name);
}

// Debug mode, environment STG_DEBUG set to anything but "0": scatter checks
// on the host that no two active indices send rows to the same destination
// (such stores conflict, and their outcome is undefined).  It synchronizes the
// stream and copies the indices and the mask to the host.
bool debug_mode() {
  const char* e = std::getenv("STG_DEBUG");
  return e && *e && std::strcmp(e, "0") != 0;
}

int check_unique_destinations(const char* name, const int32_t* indices, const uint8_t* mask, int64_t n,
                              int64_t ax_off, int64_t ax_ext, hipStream_t s) {
  std::vector<int32_t> idx((size_t)n);
  std::vector<uint8_t> msk(mask ? (size_t)n : 0);
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(idx.data(), indices, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess ||
      (mask && hipMemcpy(msk.data(), mask, (size_t)n, hipMemcpyDeviceToHost) != hipSuccess))
    return fail(STG_ERR_LAUNCH, "%s: STG_DEBUG check cannot read the indices: %s", name,
                hipGetErrorString(hipGetLastError()));
  std::vector<int64_t> rows;
  rows.reserve((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    if (mask && !msk[(size_t)i]) continue;
    const int64_t r = ax_off + idx[(size_t)i];
    if (r >= 0 && r < ax_ext) rows.push_back(r);
  }
  std::sort(rows.begin(), rows.end());
  const auto dup = std::adjacent_find(rows.begin(), rows.end());
  if (dup != rows.end())
    return fail(STG_ERR_INVALID,
                "%s: STG_DEBUG: destination %lld along the indexed axis is written by two active indices "
                "(conflicting stores are undefined)",
                name, (long long)*dup);
  return STG_OK;
}

// Shared argument checks and dispatch of the entry points.  `a` is the
// indexed array; `t` the dense side (gather output, scatter input).
int run(Op op, const stg_tensor* a, const int32_t* indices, const uint8_t* mask, int64_t n_indices,
        const int64_t* tile_shape, const int64_t* offset, int32_t axis, double padding_value,
        const stg_tensor* t, void* stream, void* workspace = nullptr, int64_t workspace_bytes = 0) {
  clear_error();
  const char* name = op_name(op);
  int rc;
  if ((rc = check_tensor(a, name)) || (rc = check_tensor(t, name))) return rc;
  if (a->dtype != t->dtype) return fail(STG_ERR_INVALID, "%s: dtype mismatch", name);
  if (op == Op::GatherBackward && a->dtype != STG_F32 && a->dtype != STG_F64)
    return fail(STG_ERR_UNSUPPORTED, "%s: gradients must be STG_F32 or STG_F64 (hardware float atomics)", name);
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
                  op == Op::Scatter ? "tile" : op == Op::GatherBackward ? "grad_out" : "out", d,
                  (long long)t->shape[d], (long long)want);
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
  if (op == Op::Scatter && debug_mode() &&
      (rc = check_unique_destinations(name, indices, mask, n_indices, off[axis], a->shape[axis], s)))
    return rc;
  const int last = rank - 1;

  const bool row_path = rank >= 2 && axis != last && a->stride[last] == 1 && t->stride[last] == 1 &&
                        tile_shape[last] * es <= 16 * 4096;
  if (row_path) {
    RowParams p{};
    p.a = (const char*)a->data;
    p.t = (char*)t->data;
    p.indices = indices;
    p.mask = op == Op::Gather || op == Op::GatherBackward ? nullptr : mask;
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
    // about eight 16-byte vectors per lane, but keep at least 512 workgroups
    // (two per CU) while rows allow: on the 4096-row, 1 KiB-row gather a
    // kernel of 512 workgroups of 8 rows takes 3.9 us, of 2048 of 2 rows 5.0
    // (more workgroups only add dispatch and index resolution to a launch
    // that is two dependent memory round trips long), of 64 of 64 rows 6.6
    int64_t rows = (kThreads * kUnroll) / p.n_chunks;
    rows = rows < 1 ? 1 : rows > kMaxRowsPerWg ? kMaxRowsPerWg : rows;
    while (rows > 1 && (p.n_rows + rows - 1) / rows < 512) rows /= 2;
    if (rows * p.n_chunks > 65535) rows = 65535 / p.n_chunks;
    p.rows_per_wg = (int32_t)rows;
    const int64_t grid = (p.n_rows + rows - 1) / rows;
    if (grid > INT32_MAX) return fail(STG_ERR_RANGE, "%s: too many rows", name);
    if (op == Op::GatherBackward && workspace) {
      const int64_t R = p.ax_ext * p.p_ext * p.q_ext;
      // int32 term and row positions, with headroom for the kernels' strides
      // past the last one (term batches, chunks, windows, slices)
      constexpr int64_t kSegLimit = INT32_MAX - (int64_t(1) << 20);
      if (R >= kSegLimit || p.n_rows >= kSegLimit)
        return fail(STG_ERR_RANGE, "%s: the segmented path needs fewer than 2^31 - 2^20 rows and terms", name);
      if (workspace_bytes < seg_layout(R, p.n_rows).bytes)
        return fail(STG_ERR_INVALID, "%s: workspace of %lld bytes, %lld needed", name, (long long)workspace_bytes,
                    (long long)seg_layout(R, p.n_rows).bytes);
      if (((uintptr_t)workspace & 255) != 0) return fail(STG_ERR_INVALID, "%s: workspace must be 256-byte aligned", name);
      if (R == 0) return STG_OK;
      return launch_segmented(name, es, p, R, (char*)workspace, s);
    }
    return launch_rows(op, es, p, grid, s);
  }
  ElemParams p{};
  p.a = (const char*)a->data;
  p.t = (char*)t->data;
  p.indices = indices;
  p.mask = op == Op::Gather || op == Op::GatherBackward ? nullptr : mask;
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

extern "C" int tile_gather_backward(const stg_tensor* a_grad, const int32_t* indices, int64_t n_indices,
                                    const int64_t* tile_shape, const int64_t* offset, int32_t axis,
                                    const stg_tensor* grad_out, void* workspace, int64_t workspace_bytes,
                                    void* stream) {
  return run(Op::GatherBackward, a_grad, indices, nullptr, n_indices, tile_shape, offset, axis, 0.0, grad_out, stream,
             workspace, workspace_bytes);
}

extern "C" int64_t tile_gather_backward_workspace(const stg_tensor* a_grad, int64_t n_indices,
                                                  const int64_t* tile_shape, int32_t axis) {
  clear_error();
  const char* name = "tile_gather_backward_workspace";
  int rc;
  if ((rc = check_tensor(a_grad, name))) return -rc;
  const int rank = a_grad->rank, last = rank - 1;
  if (axis < 0 || axis >= rank || !tile_shape || n_indices < 0)
    return -fail(STG_ERR_INVALID, "%s: bad axis, tile_shape or n_indices", name);
  for (int d = 0; d < rank; ++d)
    if (tile_shape[d] < 1) return -fail(STG_ERR_INVALID, "%s: tile_shape[%d] < 1", name, d);
  const int es = dtype_size(a_grad->dtype);
  // the segmented path serves the row layout only (as the row kernels do)
  if (rank < 2 || axis == last || a_grad->stride[last] != 1 || tile_shape[last] * es > 16 * 4096) return 0;
  int64_t R = 1, rest = 1;
  for (int d = 0; d < last; ++d) {
    R *= a_grad->shape[d];
    if (d != axis) rest *= tile_shape[d];
  }
  return seg_layout(R, n_indices * rest).bytes;
}
