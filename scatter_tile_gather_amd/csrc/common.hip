// Host-side pieces of libstg that launch nothing: error state, version, grid
// sizing, padding conversion, tensor validation and the ragged schedule.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "stg_internal.h"

namespace stg {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(STG_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return STG_OK;
}

int dtype_size(int32_t dtype) {
  switch (dtype) {
    case STG_U8: return 1;
    case STG_BF16:
    case STG_F16: return 2;
    case STG_F32:
    case STG_I32: return 4;
    case STG_F64:
    case STG_I64: return 8;
    default: return 0;
  }
}

// Round a finite or infinite double to a binary format with `eb` exponent
// bits and `mb` fraction bits, ties to even, working on the integer
// significand of the double.
static uint32_t round_bits(double v, int eb, int mb) {
  uint64_t d;
  memcpy(&d, &v, 8);
  const uint32_t sign = (uint32_t)(d >> 63) << (eb + mb);
  const int dexp = (int)((d >> 52) & 0x7FF);
  const uint64_t dfrac = d & ((uint64_t(1) << 52) - 1);
  const uint32_t inf = ((1u << eb) - 1) << mb;
  if (dexp == 0x7FF) return sign | inf | (dfrac ? (1u << (mb - 1)) : 0u);
  if (dexp == 0) return sign;  // double zero/subnormal: far below any target quantum
  const int bias = (1 << (eb - 1)) - 1;
  const uint64_t sig = dfrac | (uint64_t(1) << 52);  // value = sig * 2^(e - 52)
  int e = dexp - 1023;
  // bits of sig kept: (mb + 1) for a normal result, fewer below the normal range
  int drop = 52 - mb + ((e < 1 - bias) ? (1 - bias - e) : 0);
  uint64_t q;
  if (drop > 63) {
    q = 0;
  } else {
    q = sig >> drop;
    const uint64_t rem = sig & ((uint64_t(1) << drop) - 1);
    const uint64_t half = uint64_t(1) << (drop - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
  }
  if (e < 1 - bias) return sign | (uint32_t)q;  // subnormal (q == 2^mb is the smallest normal)
  if (q == (uint64_t(1) << (mb + 1))) {
    q >>= 1;
    ++e;
  }
  if (e > bias) return sign | inf;
  return sign | ((uint32_t)(e + bias) << mb) | (uint32_t)(q & ((uint64_t(1) << mb) - 1));
}

int fill_pattern(double v, int32_t dtype, uint32_t fill[4]) {
  switch (dtype) {
    case STG_F32: {
      const uint32_t b = round_bits(v, 8, 23);
      for (int i = 0; i < 4; ++i) fill[i] = b;
      return 0;
    }
    case STG_BF16:
    case STG_F16: {
      const uint32_t h = dtype == STG_BF16 ? round_bits(v, 8, 7) : round_bits(v, 5, 10);
      for (int i = 0; i < 4; ++i) fill[i] = h | (h << 16);
      return 0;
    }
    case STG_F64: {
      uint64_t b;
      memcpy(&b, &v, 8);
      for (int i = 0; i < 4; ++i) fill[i] = (uint32_t)(i & 1 ? b >> 32 : b);
      return 0;
    }
    case STG_I32: {
      if (!(v > -2147483649.0 && v < 2147483648.0)) return -1;
      const uint32_t b = (uint32_t)(int32_t)trunc(v);
      for (int i = 0; i < 4; ++i) fill[i] = b;
      return 0;
    }
    case STG_I64: {
      if (!(v >= -9223372036854775808.0 && v < 9223372036854775808.0)) return -1;
      const uint64_t b = (uint64_t)(int64_t)trunc(v);
      for (int i = 0; i < 4; ++i) fill[i] = (uint32_t)(i & 1 ? b >> 32 : b);
      return 0;
    }
    case STG_U8: {
      if (!(v > -1.0 && v < 256.0)) return -1;
      const uint32_t b = (uint32_t)(uint8_t)trunc(v);
      for (int i = 0; i < 4; ++i) fill[i] = b * 0x01010101u;
      return 0;
    }
    default: return -1;
  }
}

int check_tensor(const stg_tensor* t, const char* name) {
  if (!t) return fail(STG_ERR_INVALID, "%s: null tensor descriptor", name);
  if (t->rank < 1 || t->rank > 4) return fail(STG_ERR_INVALID, "%s: rank %d not in [1, 4]", name, t->rank);
  if (!dtype_size(t->dtype)) return fail(STG_ERR_UNSUPPORTED, "%s: unknown dtype %d", name, t->dtype);
  int64_t numel = 1;
  for (int d = 0; d < t->rank; ++d) {
    if (t->shape[d] < 0) return fail(STG_ERR_INVALID, "%s: negative shape[%d]", name, d);
    if (t->stride[d] < 0) return fail(STG_ERR_INVALID, "%s: negative stride[%d]", name, d);
    // extents and element counts stay far from int64 overflow, which the
    // size and offset arithmetic downstream relies on
    if (t->shape[d] > (int64_t(1) << 40) || t->stride[d] > (int64_t(1) << 40))
      return fail(STG_ERR_RANGE, "%s: shape[%d] or stride[%d] exceeds 2^40", name, d, d);
    if (__builtin_mul_overflow(numel, t->shape[d], &numel) || numel > (int64_t(1) << 48))
      return fail(STG_ERR_RANGE, "%s: more than 2^48 elements", name);
  }
  if (numel > 0 && !t->data) return fail(STG_ERR_INVALID, "%s: null data pointer", name);
  return STG_OK;
}

// ---- kernel tracing -----------------------------------------------------

namespace {
struct TraceRecord {
  const char* name;
  TraceEvents ev;
};
// Events are recycled through `pool` and kept until the process ends (they
// are not destroyed at thread exit, when the HIP runtime may be gone).
struct TraceState {
  bool on = false;
  std::vector<TraceRecord> log;
  std::vector<TraceEvents> pool;
};
thread_local TraceState g_trace;
}  // namespace

bool trace_enabled() { return g_trace.on; }

TraceEvents trace_next(const char* kernel_name) {
  TraceEvents ev;
  if (!g_trace.pool.empty()) {
    ev = g_trace.pool.back();
    g_trace.pool.pop_back();
  } else if (hipEventCreate(&ev.start) != hipSuccess || hipEventCreate(&ev.stop) != hipSuccess) {
    if (ev.start) (void)hipEventDestroy(ev.start);
    return TraceEvents{};  // untraced launch
  }
  g_trace.log.push_back({kernel_name, ev});
  return ev;
}

}  // namespace stg

using namespace stg;

extern "C" int stg_trace_enable(int on) {
  const int prev = g_trace.on ? 1 : 0;
  g_trace.on = on != 0;
  return prev;
}

extern "C" int stg_trace_read(int cap, const char** names, float* ms) {
  clear_error();
  if (cap < 0 || (cap > 0 && (!names || !ms))) return -fail(STG_ERR_INVALID, "stg_trace_read: bad output arrays");
  int n = 0;
  for (auto& r : g_trace.log) {
    if (n < cap) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, r.ev.start, r.ev.stop) != hipSuccess) {
        (void)hipGetLastError();
        t = -1.f;  // not complete: the caller did not synchronise
      }
      names[n] = r.name;
      ms[n] = t;
      ++n;
    }
    g_trace.pool.push_back(r.ev);
  }
  g_trace.log.clear();
  return n;
}

extern "C" int stg_version(void) { return 100; }  // 0.1.0

extern "C" const char* stg_last_error(void) { return g_err; }

extern "C" int64_t stg_tile_grid(int64_t extent, int64_t origin, int64_t tile) {
  if (tile <= 0) return -1;
  if (origin >= extent) return 0;
  const int64_t span = extent - origin;
  return span / tile + (span % tile != 0);
}

extern "C" int ragged_tile_schedule(const int64_t* seq_lens, int64_t n_seqs, int32_t bm_seq,
                                    int32_t middle_dim, uint32_t* ragged_idx, uint32_t* dynamic_dim,
                                    uint32_t* middle_idx, int64_t* n_tiles) {
  clear_error();
  if (!n_tiles) return fail(STG_ERR_INVALID, "ragged_tile_schedule: null n_tiles");
  if (n_seqs < 0 || (n_seqs > 0 && !seq_lens)) return fail(STG_ERR_INVALID, "ragged_tile_schedule: bad seq_lens");
  if (bm_seq < 1 || middle_dim < 1) return fail(STG_ERR_INVALID, "ragged_tile_schedule: bm_seq and middle_dim must be >= 1");
  const bool write = ragged_idx || dynamic_dim || middle_idx;
  if (write && !(ragged_idx && dynamic_dim && middle_idx))
    return fail(STG_ERR_INVALID, "ragged_tile_schedule: outputs must be all NULL or all non-NULL");
  int64_t row = 0, k = 0;
  for (int64_t s = 0; s < n_seqs; ++s) {
    const int64_t len = seq_lens[s];
    if (len < 0) return fail(STG_ERR_INVALID, "ragged_tile_schedule: negative length at %lld", (long long)s);
    for (int64_t first = 0; first < len; first += bm_seq) {
      if (row + first > 0xFFFFFFFFll) return fail(STG_ERR_RANGE, "ragged_tile_schedule: row index exceeds 32 bits");
      const int64_t rows = len - first < bm_seq ? len - first : bm_seq;
      for (int32_t m = 0; m < middle_dim; ++m, ++k) {
        if (write) {
          ragged_idx[k] = (uint32_t)(row + first);
          dynamic_dim[k] = (uint32_t)rows;
          middle_idx[k] = (uint32_t)m;
        }
      }
    }
    row += len;
  }
  *n_tiles = k;
  return STG_OK;
}
