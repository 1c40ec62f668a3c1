// Bounded-edge GEMM  C = A . B  (bf16 operands, fp32 accumulation).
//
// Semantics (cuTile.jl Operations, muladd: bf16 x bf16 accumulates in f32;
// Tylo.jl Boundary tiles, "Accumulator stores and GEMM": ceiling-division
// output grid and K loop, boundary stages zero-filled, an epilogue that
// converts the f32 accumulator to the destination type and suppresses invalid
// coordinates, leaving padding untouched).
//
// gfx950 design:
//  * Workgroup tile BM x BN x 64, waves WM x WN, each wave owning a
//    (BM/WM) x (BN/WN) block of v_mfma_f32_32x32x16_bf16 accumulators.  Every
//    lane issues every MFMA; bounds only select the data that was staged.
//  * Staging (Tylo.jl Boundary tiles, opening section and "A concrete edge",
//    recast): each lane owns fixed 16-byte chunks of the A and B stage.  A
//    chunk whose eight source values are all valid is one dwordx4 buffer load
//    at its (2-byte aligned, for odd leading dimensions) offset; a chunk with
//    no valid value gets an offset past num_records and loads zeros; only a
//    chunk straddling the K or N edge is assembled element by element.  An
//    address is formed only for valid coordinates.
//  * LDS: A is row-major with K contiguous (the MFMA A operand is eight
//    consecutive K values of one row) and the 16-byte chunk index is XOR-
//    swizzled by the tile-local row, so the 32 rows an MFMA operand read
//    touches spread over all banks.  The swizzle is a function of the
//    tile-local (window) coordinate, and zero-filled chunks go through the
//    same mapping, so the edge does not disturb the swizzle phase (Tylo.jl
//    Boundary tiles, "A concrete edge", swizzled windows).  B stays row-major
//    (N contiguous, rows padded by 32 bytes) and the MFMA B operand -- eight
//    consecutive K values of one column -- is read with ds_read_b64_tr_b16,
//    the gfx950 LDS transpose read, so no transpose pass is needed.
//  * Two LDS stages: the global loads of stage k+1 are in flight while stage
//    k feeds the MFMAs; one barrier per K step.
//  * Grid: a main launch of 256 x 256 tiles over the columns that fill whole
//    tiles, and an edge launch of 128 x 32 tiles for the remaining columns,
//    so a one-column remainder (N = 8193) does not cost a full tile wave.
//    Tile ids are renumbered so that consecutive ids run on one XCD and walk
//    4-row-panel groups, keeping A and B panels resident in that XCD's L2.
#include "stg_internal.h"

namespace stg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BK = 64;

struct GemmParams {
  const char* A;  // bf16 (M, K), row stride lda elements
  const char* B;  // bf16 (K, N), row stride ldb elements
  char* C;
  int64_t lda, ldb, ldc;
  int64_t M, N, K;
  int64_t n_base;  // first column covered by this launch
  int32_t tiles_m, tiles_n;
  int32_t c_f32;  // 1: fp32 output, 0: bf16
};

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_CHUNKS = BM * BK / 8;
  static constexpr int B_CHUNKS = BK * BN / 8;
  static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
  static constexpr int B_PER_T = (B_CHUNKS + NT - 1) / NT;
  static constexpr int B_PITCH_B = BN * 2 + 32;  // bytes per LDS row of B
  static constexpr int A_STAGE_B = BM * BK * 2;
  static constexpr int B_STAGE_B = BK * B_PITCH_B;
  static constexpr int STAGE_B = A_STAGE_B + B_STAGE_B;
  static constexpr int EPI_PITCH_B = WTN * 2 + 16;  // bytes per row of a wave's bf16 output tile
  static constexpr int EPI_WAVE_B = WTM * EPI_PITCH_B;
  static constexpr int LDS_B = 2 * STAGE_B > WM * WN * EPI_WAVE_B ? 2 * STAGE_B : WM * WN * EPI_WAVE_B;
  static_assert(FM >= 1 && FN >= 1, "wave tile must hold whole 32x32 MFMA blocks");
};

// Byte offset of A chunk (row r, 16-byte chunk kc) inside an A stage.
__device__ __forceinline__ int a_lds(int r, int kc) { return r * (BK * 2) + ((kc ^ (r & 7)) << 4); }

// Load the eight bf16 values at (row, col .. col+7) of a row-major matrix
// whose valid region is rows < rows_valid, cols < cols_valid.  `rs` is
// based at `base` (element (row0, col0)); (r, c) are relative to it.
__device__ __forceinline__ u32x4 load_chunk(const __amdgpu_buffer_rsrc_t rs, const char* base, int64_t ld, int r,
                                            int c, bool row_ok, int64_t cols_left) {
  // cols_left: valid columns from c onward (may be <= 0)
  const bool full = row_ok && cols_left >= 8;
  const uint32_t off = full ? (uint32_t)(r * ld * 2 + c * 2) : kOOB;
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  if (row_ok && !full && cols_left > 0) {
    const uint16_t* p = (const uint16_t*)(base + r * ld * 2 + c * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e < cols_left) vec_set<2>(v, e, p[e]);
  }
  return v;
}

// Tile (tm, tn) of logical id t: consecutive ids on one XCD, grouped by 4
// row panels so neighbouring workgroups share A and B panels in L2.
__device__ __forceinline__ void tile_of(uint32_t t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int group = t / per_group;
  const int first = group * G;
  const int gm = min(G, tiles_m - first);
  const int in = t - group * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

template <class CF>
__global__ __launch_bounds__(CF::NT) __attribute__((amdgpu_waves_per_eu(1, 2))) void gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / CF::WN, wn = wave % CF::WN;
  int tm, tn;
  tile_of(xcd_remap(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * CF::BM;
  const int64_t n0 = p.n_base + (int64_t)tn * CF::BN;
  const int nk = (int)((p.K + BK - 1) / BK);

  f32x16 acc[CF::FM][CF::FN];
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int j = 0; j < CF::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[CF::A_PER_T], rb[CF::B_PER_T];
  bf16x8 fa[2][CF::FM], fb[2][CF::FN];

  auto load_stage = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    // A: rows m0.., cols k0..; B: rows k0.., cols n0..
    const char* abase = p.A + (m0 * p.lda + k0) * 2;
    const char* bbase = p.B + (k0 * p.ldb + n0) * 2;
    const int64_t a_avail = ((p.M - 1 - m0) * p.lda + (p.K - k0)) * 2;
    const int64_t b_avail = ((p.K - 1 - k0) * p.ldb + (p.N - n0)) * 2;
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(abase, (uint32_t)(a_avail <= 0 ? 0 : a_avail < (int64_t)kOOB ? a_avail : (int64_t)kOOB - 1));
    const __amdgpu_buffer_rsrc_t rsb =
        make_rsrc(bbase, (uint32_t)(b_avail <= 0 ? 0 : b_avail < (int64_t)kOOB ? b_avail : (int64_t)kOOB - 1));
#pragma unroll
    for (int q = 0; q < CF::A_PER_T; ++q) {
      const int c = tid + q * CF::NT;
      ra[q] = (u32x4){0, 0, 0, 0};
      if (c < CF::A_CHUNKS) {
        const int r = c / (BK / 8), kc = c % (BK / 8);
        ra[q] = load_chunk(rsa, abase, p.lda, r, kc * 8, m0 + r < p.M, p.K - k0 - kc * 8);
      }
    }
#pragma unroll
    for (int q = 0; q < CF::B_PER_T; ++q) {
      const int c = tid + q * CF::NT;
      rb[q] = (u32x4){0, 0, 0, 0};
      if (c < CF::B_CHUNKS) {
        const int r = c / (CF::BN / 8), nc = c % (CF::BN / 8);
        rb[q] = load_chunk(rsb, bbase, p.ldb, r, nc * 8, k0 + r < p.K, p.N - n0 - nc * 8);
      }
    }
  };
  auto store_stage = [&](int buf) {
    char* as = smem + buf * CF::STAGE_B;
    char* bs = as + CF::A_STAGE_B;
#pragma unroll
    for (int q = 0; q < CF::A_PER_T; ++q) {
      const int c = tid + q * CF::NT;
      if (c < CF::A_CHUNKS) *(u32x4*)(as + a_lds(c / (BK / 8), c % (BK / 8))) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < CF::B_PER_T; ++q) {
      const int c = tid + q * CF::NT;
      if (c < CF::B_CHUNKS) *(u32x4*)(bs + (c / (CF::BN / 8)) * CF::B_PITCH_B + (c % (CF::BN / 8)) * 16) = rb[q];
    }
  };
  // MFMA operands of K sub-step ks (16 K values) of stage `buf` into slot s
  auto read_frags = [&](int buf, int ks, int s) {
    const char* as = smem + buf * CF::STAGE_B;
    const char* bs = as + CF::A_STAGE_B;
#pragma unroll
    for (int i = 0; i < CF::FM; ++i) {
      const int r = wm * CF::WTM + i * 32 + (lane & 31);
      fa[s][i] = *(const bf16x8*)(as + a_lds(r, 2 * ks + (lane >> 5)));
    }
#pragma unroll
    for (int j = 0; j < CF::FN; ++j) {
      // transpose read: lane t of 16-lane group g points at row
      // 16ks + 8(g/2) + 4h + t/4, columns nb + 16(g%2) + 4(t%4) .. +3
      const int g = lane >> 4, t = lane & 15;
      const int col = wn * CF::WTN + j * 32 + 16 * (g & 1) + 4 * (t & 3);
      const int row = 16 * ks + 8 * (g >> 1) + (t >> 2);
      const char* p0 = bs + row * CF::B_PITCH_B + col * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * CF::B_PITCH_B));
      const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      fb[s][j] = __builtin_bit_cast(bf16x8, both);
    }
  };

  if (nk > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  if (nk > 0) read_frags(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    // next stage's global loads fly during this stage's MFMAs
    if (more) load_stage(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) read_frags(buf, ks + 1, cur ^ 1);
      // the other stage was released by the barrier that ended the last step
      if (ks == BK / 16 - 1 && more) store_stage(buf ^ 1);
#pragma unroll
      for (int i = 0; i < CF::FM; ++i)
#pragma unroll
        for (int j = 0; j < CF::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (more) read_frags(buf ^ 1, 0, 0);
  }

  // clipped epilogue: lane l, accumulator r of block (i, j) is
  // row 8(r/4) + 4(l/32) + r%4, column l%32 of that 32x32 block
  if (p.c_f32) {
#pragma unroll
    for (int i = 0; i < CF::FM; ++i)
#pragma unroll
      for (int j = 0; j < CF::FN; ++j) {
        const int64_t col = n0 + wn * CF::WTN + j * 32 + (lane & 31);
        if (col >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * CF::WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < p.M) *(float*)(p.C + (row * p.ldc + col) * 4) = acc[i][j][r];
        }
      }
    return;
  }
  // bf16: round to nearest even, stage the wave's tile in LDS (every wave has
  // its own region; the stages are no longer read), then write whole 16-byte
  // row chunks; only chunks crossing column N are written element by element
  char* ep = smem + wave * CF::EPI_WAVE_B;
#pragma unroll
  for (int i = 0; i < CF::FM; ++i)
#pragma unroll
    for (int j = 0; j < CF::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = j * 32 + (lane & 31);
        *(__bf16*)(ep + row * CF::EPI_PITCH_B + col * 2) = (__bf16)acc[i][j][r];
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = CF::WTN / 8;  // 16-byte chunks per wave-tile row
  for (int c = lane; c < CF::WTM * CPR; c += 64) {
    const int row = c / CPR, ch = c % CPR;
    const int64_t grow = m0 + wm * CF::WTM + row;
    const int64_t gcol = n0 + wn * CF::WTN + ch * 8;
    if (grow >= p.M || gcol >= p.N) continue;
    const u32x4 v = *(const u32x4*)(ep + row * CF::EPI_PITCH_B + ch * 16);
    char* dst = p.C + (grow * p.ldc + gcol) * 2;
    if (gcol + 8 <= p.N) {
      st16(dst, v);
    } else {
      for (int e = 0; e < 8; ++e)
        if (gcol + e < p.N) store_elem<2>(dst + e * 2, vec_get<2>(v, e));
    }
  }
}

using MainCfg = Cfg<256, 256, 2, 2>;
using EdgeCfg = Cfg<128, 32, 4, 1>;

template <class CF>
int launch(const char* name, GemmParams p, int64_t cols, hipStream_t s) {
  p.tiles_m = (int32_t)((p.M + CF::BM - 1) / CF::BM);
  p.tiles_n = (int32_t)((cols + CF::BN - 1) / CF::BN);
  const int64_t n_wg = (int64_t)p.tiles_m * p.tiles_n;
  if (n_wg == 0) return STG_OK;
  const size_t lds = CF::LDS_B;
  launch_kernel(name, gemm_kernel<CF>, dim3((unsigned)n_wg), dim3(CF::NT), lds, s, p);
  return check_launch("gemm_bounded");
}

bool lds_configured = false;

}  // namespace
}  // namespace stg

using namespace stg;

extern "C" int gemm_bounded(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                            int64_t M, int64_t N, int64_t K, int32_t c_dtype, void* stream) {
  clear_error();
  const char* name = "gemm_bounded";
  if (M < 0 || N < 0 || K < 0) return fail(STG_ERR_INVALID, "%s: negative size", name);
  if (c_dtype != STG_BF16 && c_dtype != STG_F32)
    return fail(STG_ERR_UNSUPPORTED, "%s: c_dtype must be STG_BF16 or STG_F32", name);
  if (lda < (K > 0 ? K : 1) || ldb < (N > 0 ? N : 1) || ldc < (N > 0 ? N : 1))
    return fail(STG_ERR_INVALID, "%s: row strides must be >= the row lengths", name);
  if (M == 0 || N == 0) return STG_OK;
  if (!C || (K > 0 && (!A || !B))) return fail(STG_ERR_INVALID, "%s: null operand", name);
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return fail(STG_ERR_RANGE, "%s: size too large", name);
  // 32-bit buffer offsets within one stage: BM rows of A, BK rows of B
  if ((int64_t)MainCfg::BM * lda * 2 + 256 >= kMaxOffset32 || (int64_t)BK * ldb * 2 + 512 >= kMaxOffset32)
    return fail(STG_ERR_RANGE, "%s: a stage of A or B spans more than 2^31 bytes", name);
  if (!lds_configured) {
    if (hipFuncSetAttribute((const void*)gemm_kernel<MainCfg>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            MainCfg::LDS_B) != hipSuccess ||
        hipFuncSetAttribute((const void*)gemm_kernel<EdgeCfg>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            EdgeCfg::LDS_B) != hipSuccess)
      return fail(STG_ERR_LAUNCH, "%s: cannot reserve LDS: %s", name, hipGetErrorString(hipGetLastError()));
    lds_configured = true;
  }
  GemmParams p{};
  p.A = (const char*)A;
  p.B = (const char*)B;
  p.C = (char*)C;
  p.lda = lda, p.ldb = ldb, p.ldc = ldc;
  p.M = M, p.N = N, p.K = K;
  p.c_f32 = c_dtype == STG_F32;
  const hipStream_t s = as_stream(stream);
  const int64_t n_main = (N / MainCfg::BN) * MainCfg::BN;
  int rc;
  p.n_base = 0;
  if (n_main > 0 && (rc = launch<MainCfg>("gemm_bounded/main", p, n_main, s))) return rc;
  p.n_base = n_main;
  if (N > n_main && (rc = launch<EdgeCfg>("gemm_bounded/edge", p, N - n_main, s))) return rc;
  return STG_OK;
}
