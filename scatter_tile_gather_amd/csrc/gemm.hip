// Bounded-edge GEMM (placeholder until the MFMA kernel lands).
#include "stg_internal.h"

using namespace stg;

extern "C" int gemm_bounded(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                            int64_t M, int64_t N, int64_t K, int32_t c_dtype, void* stream) {
  clear_error();
  (void)A, (void)lda, (void)B, (void)ldb, (void)C, (void)ldc, (void)M, (void)N, (void)K, (void)c_dtype,
      (void)stream;
  return fail(STG_ERR_UNSUPPORTED, "gemm_bounded: not built yet");
}
