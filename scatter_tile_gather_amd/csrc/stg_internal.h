// Internal helpers shared by the libstg translation units (host and device).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/stg.h"

namespace stg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- host side -------------------------------------------------------------

// Record a failure message for stg_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the error state of this thread (successful calls leave it "").
void clear_error();
// STG_OK, or STG_ERR_LAUNCH with the HIP error text, after a kernel launch.
int check_launch(const char* what);

// Element size in bytes of a stg_dtype, or 0 if the code is unknown.
int dtype_size(int32_t dtype);

// Convert a double to the bit pattern of `dtype` (floats: nearest-even with
// infinities on overflow; integers: truncation toward zero).  Writes the
// element replicated over 16 bytes into fill[4].  Returns 0, or -1 if the
// value is not representable in an integer type.
int fill_pattern(double v, int32_t dtype, uint32_t fill[4]);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Runs f (returning bool) once per device -- the one current at the call --
// and returns its result on every later call on that device, also when the
// first calls come from several host threads.  Kernel attributes such as the
// dynamic LDS limit belong to each device's copy of a kernel, so they are set
// once on every device the library launches on.
class OncePerDevice {
 public:
  template <class F>
  bool run(F&& f) {
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= kDevices) return false;
    std::call_once(flag_[d], [&] { ok_[d] = f(); });
    return ok_[d];
  }

 private:
  static constexpr int kDevices = 64;
  std::once_flag flag_[kDevices];
  bool ok_[kDevices] = {};
};

// Validate a tensor descriptor: non-null, rank in [1,4], known dtype,
// non-negative shape and stride.  Returns STG_OK or a failure code.
int check_tensor(const stg_tensor* t, const char* name);

constexpr int64_t kMaxOffset32 = (int64_t(1) << 31) - 1;  // voffset range used by buffer ops

// Kernel tracing: while enabled on this thread, each launch carries a
// start/stop event pair inside its own dispatch packet, so the recorded time
// covers the kernel alone (not the queue gaps between dependent launches).
struct TraceEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
bool trace_enabled();
TraceEvents trace_next(const char* kernel_name);

template <typename K, typename... Args>
void launch_kernel(const char* name, K kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  if (trace_enabled()) {
    const TraceEvents ev = trace_next(name);
    if (ev.start) {
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0, args...);
      return;
    }
  }
  hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// ---- device side -----------------------------------------------------------

// 16-byte load/store at any byte alignment (the toolchain and the gfx950
// memory pipeline support unaligned dwordx4 accesses).
__device__ __forceinline__ u32x4 ld16(const char* p) {
  u32x4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}
__device__ __forceinline__ void st16(char* p, u32x4 v) { __builtin_memcpy(p, &v, 16); }

// Non-temporal 16-byte store (global_store_dwordx4 ... nt), any byte alignment.
// The row gather/scatter kernels write their rows this way: measured back to
// back, the masked gather runs 18% faster with it (5.8 -> 6.9 TB/s) and the
// masked scatter to random rows 27% faster (4.9 -> 6.2 TB/s).  It is not a
// general win: the clipped tile stores into a matrix run about 25% slower
// with it, and the tile-buffer writes of the copy and ragged kernels gain
// nothing, so those keep plain stores.
typedef u32x4 u32x4_unaligned __attribute__((aligned(1)));
__device__ __forceinline__ void st16_nt(char* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4_unaligned*)p); }

// Non-temporal 16-byte load (global_load_dwordx4 ... nt), any byte alignment.
// The grouped gather backward reads its grad_out rows (each once, in random
// order) and a.grad's chunks this way: the uniform 4M-term workload runs 7%
// faster (reduce 0.597 -> 0.550 ms) and the pieces of hot rows 10% faster.
// The forward row kernels keep plain loads: with this one the masked gather,
// whose table rows are read about four times each, drops from 6.9 to 5.6
// TB/s, and the masked scatter, reading contiguous tile rows, from 6.2 to 5.1.
__device__ __forceinline__ u32x4 ld16_nt(const char* p) {
  return __builtin_nontemporal_load((const u32x4_unaligned*)p);
}

// Buffer resource over [base, base + bytes) with the gfx9 raw-buffer format
// word: loads whose offset lies past num_records return zero and stores past
// it are dropped, which is how invalid vectors are zero-filled or clipped
// without forming an address outside the logical extent.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset beyond any num_records used here

// Copy one element of ESIZE bytes (aligned to its own size) between pointers.
template <int ESIZE>
__device__ __forceinline__ void copy_elem(char* dst, const char* src) {
  if constexpr (ESIZE == 1) *(uint8_t*)dst = *(const uint8_t*)src;
  if constexpr (ESIZE == 2) *(uint16_t*)dst = *(const uint16_t*)src;
  if constexpr (ESIZE == 4) *(uint32_t*)dst = *(const uint32_t*)src;
  if constexpr (ESIZE == 8) *(uint64_t*)dst = *(const uint64_t*)src;
}

// Element e of a 16-byte register vector, for ESIZE-byte elements.
template <int ESIZE>
__device__ __forceinline__ uint64_t vec_get(const u32x4& v, int e) {
  if constexpr (ESIZE == 8) return (uint64_t)v[2 * e] | ((uint64_t)v[2 * e + 1] << 32);
  if constexpr (ESIZE == 4) return v[e];
  if constexpr (ESIZE == 2) return (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
  if constexpr (ESIZE == 1) return (v[e >> 2] >> ((e & 3) * 8)) & 0xFFu;
  return 0;
}
template <int ESIZE>
__device__ __forceinline__ void vec_set(u32x4& v, int e, uint64_t x) {
  if constexpr (ESIZE == 8) {
    v[2 * e] = (uint32_t)x;
    v[2 * e + 1] = (uint32_t)(x >> 32);
  }
  if constexpr (ESIZE == 4) v[e] = (uint32_t)x;
  if constexpr (ESIZE == 2) {
    const int sh = (e & 1) * 16;
    v[e >> 1] = (v[e >> 1] & ~(0xFFFFu << sh)) | ((uint32_t)x << sh);
  }
  if constexpr (ESIZE == 1) {
    const int sh = (e & 3) * 8;
    v[e >> 2] = (v[e >> 2] & ~(0xFFu << sh)) | ((uint32_t)x << sh);
  }
}
template <int ESIZE>
__device__ __forceinline__ uint64_t load_elem(const char* p) {
  if constexpr (ESIZE == 1) return *(const uint8_t*)p;
  if constexpr (ESIZE == 2) return *(const uint16_t*)p;
  if constexpr (ESIZE == 4) return *(const uint32_t*)p;
  return *(const uint64_t*)p;
}
template <int ESIZE>
__device__ __forceinline__ void store_elem(char* p, uint64_t x) {
  if constexpr (ESIZE == 1) *(uint8_t*)p = (uint8_t)x;
  if constexpr (ESIZE == 2) *(uint16_t*)p = (uint16_t)x;
  if constexpr (ESIZE == 4) *(uint32_t*)p = (uint32_t)x;
  if constexpr (ESIZE == 8) *(uint64_t*)p = x;
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip, each with
// its own L2.  Renumber them so that consecutive logical ids run on the same
// XCD (a bijection on [0, total) for any total), which keeps workgroups that
// share cache lines -- neighbouring row segments, neighbouring tiles -- on one
// L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t total) {
  const uint32_t q = total >> 3, r = total & 7, xcd = w & 7, slot = w >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Exact quotient n / d for n < 2^16 and 1 <= d < 2^15, from a precomputed
// magic = ceil(2^31 / d): floor(n * magic / 2^31) differs from n / d by less
// than n / 2^31 < 1/d, which never crosses the next integer.
__device__ __forceinline__ uint32_t div_small(uint32_t n, uint32_t magic) { return __umulhi(n << 1, magic); }
inline uint32_t div_magic(uint32_t d) { return (uint32_t)(((uint64_t(1) << 31) + d - 1) / d); }

// Kernel names a bf16 GEMM call reports (errors, launch tracing).
struct GemmNames {
  const char* entry;
  const char* main;
  const char* edge;
  const char* skinny;
};

// C = A B (+ acc), bf16 operands (A (M, K), B (K, N), row strides in
// elements), fp32 accumulation, C in c_dtype (STG_BF16 or STG_F32; acc, an
// fp32 (M, N) matrix added before the store, only with STG_F32): the
// gemm_bounded kernels (gemm.hip), with the checks of gemm_bounded.
int gemm_bf16(const GemmNames& names, const void* A, int64_t lda, const void* B, int64_t ldb, const float* acc,
              int64_t ldacc, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t c_dtype, hipStream_t s);

// Block-scaled GEMM for the operand pairs, scale formats and blocks the
// scaled MFMA does not take (gemm_scaled_general.hip); arguments as
// gemm_scaled's, already checked by it.  With a workspace of at least
// gemm_scaled_general_workspace(M, N, K) bytes (256-byte aligned) the
// operands are decoded to bf16 into it once and multiplied by the bf16 GEMM;
// without one, values are decoded tile by tile inside the GEMM kernel.
int gemm_scaled_general(const void* A, int32_t a_fmt, int64_t lda, const void* a_scale, int64_t lds_a,
                        const void* Bt, int32_t b_fmt, int64_t ldb, const void* b_scale, int64_t lds_b,
                        int32_t scale_fmt, int64_t block, const float* acc, int64_t ldacc, float* C, int64_t ldc,
                        int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, hipStream_t s);
// Bytes of the decoded operands for gemm_scaled_general at this shape, or 0
// where decoding them first does not pay (or the bf16 GEMM's limits rule it
// out).
int64_t gemm_scaled_general_workspace(int64_t M, int64_t N, int64_t K);

}  // namespace stg
