// Kernel-level entry points (include/ll_testing.h).
#include "../../include/ll_testing.h"
#include "api.h"
#include "gemm.h"

using namespace ll;

template <class ET>
static int gemm_dispatch(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
                         int32_t out_dtype, void* C, int64_t ldc, const float* ia, const float* ib,
                         hipStream_t s) {
  const ET* a = static_cast<const ET*>(A);
  const ET* b = static_cast<const ET*>(B);
  if (out_dtype == LL_BF16) {
    EpiStore<bf16> e{static_cast<bf16*>(C), ldc, Deq{ia, ib}};
    LL_HIP(launch_gemm_nt(a, lda, b, ldb, M, N, K, e, s));
  } else {
    EpiStore<float> e{static_cast<float*>(C), ldc, Deq{ia, ib}};
    LL_HIP(launch_gemm_nt(a, lda, b, ldb, M, N, K, e, s));
  }
  return LL_OK;
}

extern "C" int llt_gemm_nt(int32_t op_dtype, const void* A, int64_t lda, const void* B, int64_t ldb,
                           int32_t M, int32_t N, int32_t K, int32_t out_dtype, void* C, int64_t ldc,
                           const float* inv_a, const float* inv_b, void* stream) {
  LL_CHECK(op_dtype >= LLT_OP_F32 && op_dtype <= LLT_OP_E4M3, LL_ERR_INVALID_ARG, "bad op_dtype");
  LL_CHECK(out_dtype == LL_F32 || out_dtype == LL_BF16, LL_ERR_INVALID_ARG, "bad out_dtype");
  LL_CHECK(M >= 0 && N >= 0 && K >= 0, LL_ERR_INVALID_ARG, "negative size");
  const int esz = op_dtype == LLT_OP_F32 ? 4 : op_dtype == LLT_OP_BF16 ? 2 : 1;
  LL_CHECK(((int64_t)K * esz) % 128 == 0, LL_ERR_UNSUPPORTED, "K must be a multiple of 128 bytes");
  LL_CHECK(N % 8 == 0 && ldc % 8 == 0 && ldc >= N, LL_ERR_UNSUPPORTED, "N and ldc must be multiples of 8, ldc >= N");
  LL_CHECK(lda >= K && ldb >= K && (lda * esz) % 16 == 0 && (ldb * esz) % 16 == 0, LL_ERR_INVALID_ARG,
           "lda/ldb must be >= K with 16-byte aligned rows");
  LL_CHECK((inv_a == nullptr) == (inv_b == nullptr), LL_ERR_INVALID_ARG, "inv_a and inv_b: both or neither");
  if (M == 0 || N == 0) return LL_OK;
  LL_CHECK(A && B && C, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(A) && aligned16(B) && aligned16(C), LL_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (op_dtype == LLT_OP_F32) return gemm_dispatch<float>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, s);
  if (op_dtype == LLT_OP_BF16) return gemm_dispatch<bf16>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, s);
  return gemm_dispatch<fp8>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, s);
}
