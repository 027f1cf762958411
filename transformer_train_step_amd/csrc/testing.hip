// Kernel-level entry points (include/ll_testing.h).
#include "../../include/ll_testing.h"
#include "api.h"
#include "gemm.h"
#include "quant.h"

using namespace ll;

template <class ET>
static int gemm_dispatch(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K,
                         int32_t out_dtype, void* C, int64_t ldc, const float* ia, const float* ib,
                         const GemmOps& o, hipStream_t s) {
  const ET* a = static_cast<const ET*>(A);
  const ET* b = static_cast<const ET*>(B);
  if (out_dtype == LL_BF16) {
    EpiStore<bf16> e{static_cast<bf16*>(C), ldc, Deq{ia, ib}};
    LL_HIP(launch_gemm(a, lda, b, ldb, M, N, K, e, o, s));
  } else {
    EpiStore<float> e{static_cast<float*>(C), ldc, Deq{ia, ib}};
    LL_HIP(launch_gemm(a, lda, b, ldb, M, N, K, e, o, s));
  }
  return LL_OK;
}

extern "C" int llt_gemm(int32_t op_dtype, int32_t a_kmajor, int32_t b_kmajor, const void* A, int64_t lda,
                        const void* B, int64_t ldb, int32_t M, int32_t N, int32_t K, int32_t out_dtype, void* C,
                        int64_t ldc, const float* inv_a, const float* inv_b, void* ws, size_t ws_bytes,
                        void* stream) {
  LL_CHECK(op_dtype >= LLT_OP_F32 && op_dtype <= LLT_OP_E4M3, LL_ERR_INVALID_ARG, "bad op_dtype");
  LL_CHECK(out_dtype == LL_F32 || out_dtype == LL_BF16, LL_ERR_INVALID_ARG, "bad out_dtype");
  LL_CHECK(M >= 0 && N >= 0 && K >= 0, LL_ERR_INVALID_ARG, "negative size");
  const int esz = op_dtype == LLT_OP_F32 ? 4 : op_dtype == LLT_OP_BF16 ? 2 : 1;
  const int ke = 128 / esz;
  const bool ak = a_kmajor != 0, bk = b_kmajor != 0;
  LL_CHECK((ak && bk) || op_dtype == LLT_OP_BF16, LL_ERR_UNSUPPORTED, "MN-major operands need bf16");
  LL_CHECK(N % 8 == 0 && ldc % 8 == 0 && ldc >= N, LL_ERR_UNSUPPORTED, "N and ldc must be multiples of 8, ldc >= N");
  // K-major operands are read in whole K tiles: their rows must hold round_up(K, tile) elements
  const int64_t kp = round_up(K, ke);
  LL_CHECK(!ak || (lda >= kp && (lda * esz) % 16 == 0), LL_ERR_INVALID_ARG, "K-major A: lda >= K rounded to the K tile, 16-byte rows");
  LL_CHECK(!bk || (ldb >= kp && (ldb * esz) % 16 == 0), LL_ERR_INVALID_ARG, "K-major B: ldb >= K rounded to the K tile, 16-byte rows");
  LL_CHECK(ak || (lda >= M && lda % 8 == 0 && M % 8 == 0), LL_ERR_INVALID_ARG, "MN-major A: M % 8 == 0, lda >= M, lda % 8 == 0");
  LL_CHECK(bk || (ldb >= N && ldb % 8 == 0), LL_ERR_INVALID_ARG, "MN-major B: ldb >= N, ldb % 8 == 0");
  LL_CHECK((inv_a == nullptr) == (inv_b == nullptr), LL_ERR_INVALID_ARG, "inv_a and inv_b: both or neither");
  LL_CHECK(ak && bk ? true : (ws && ws_bytes >= 64 && aligned16(ws)), LL_ERR_WORKSPACE, "MN-major operands need ws >= 64 bytes");
  if (M == 0 || N == 0) return LL_OK;
  LL_CHECK(A && B && C, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(A) && aligned16(B) && aligned16(C), LL_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  GemmOps o{ak, bk, ws};
  if (!(ak && bk)) LL_HIP(fill_f32(static_cast<float*>(ws), 0.f, 16, s));
  if (op_dtype == LLT_OP_F32) return gemm_dispatch<float>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, o, s);
  if (op_dtype == LLT_OP_BF16) return gemm_dispatch<bf16>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, o, s);
  return gemm_dispatch<fp8>(A, lda, B, ldb, M, N, K, out_dtype, C, ldc, inv_a, inv_b, o, s);
}

extern "C" size_t llt_gemm_splitk_workspace_bytes(int32_t M, int32_t N, int32_t slices) {
  if (M < 0 || N < 0 || slices < 1 || slices > 16) return 0;
  return 256 + (size_t)slices * M * N * sizeof(float);
}

template <class ET>
static int splitk_dispatch(const void* A, int64_t lda, const void* B, int64_t ldb, int M, int N, int K, int slices,
                           int32_t out_dtype, void* C, int64_t ldc, float* part, Deq dq, const GemmOps& o,
                           hipStream_t s) {
  const ET* a = static_cast<const ET*>(A);
  const ET* b = static_cast<const ET*>(B);
  if (out_dtype == LL_BF16)
    LL_HIP(launch_gemm_splitk(a, lda, b, ldb, M, N, K, slices, static_cast<bf16*>(C), ldc, part, o, s, dq));
  else
    LL_HIP(launch_gemm_splitk(a, lda, b, ldb, M, N, K, slices, static_cast<float*>(C), ldc, part, o, s, dq));
  return LL_OK;
}

extern "C" int llt_gemm_splitk(int32_t op_dtype, int32_t a_kmajor, int32_t b_kmajor, const void* A, int64_t lda,
                               const void* B, int64_t ldb, int32_t M, int32_t N, int32_t K, int32_t slices,
                               int32_t out_dtype, void* C, int64_t ldc, const float* inv_a, const float* inv_b,
                               void* ws, size_t ws_bytes, void* stream) {
  LL_CHECK(op_dtype == LLT_OP_BF16 || op_dtype == LLT_OP_E4M3, LL_ERR_INVALID_ARG, "op_dtype must be bf16 or e4m3");
  LL_CHECK(out_dtype == LL_F32 || out_dtype == LL_BF16, LL_ERR_INVALID_ARG, "bad out_dtype");
  LL_CHECK(M >= 0 && N >= 0 && K >= 0, LL_ERR_INVALID_ARG, "negative size");
  LL_CHECK(slices >= 1 && slices <= 16, LL_ERR_INVALID_ARG, "slices must be in [1, 16]");
  const bool ak = a_kmajor != 0, bk = b_kmajor != 0;
  const int esz = op_dtype == LLT_OP_BF16 ? 2 : 1, ke = 128 / esz;
  LL_CHECK((ak && bk) || op_dtype == LLT_OP_BF16, LL_ERR_UNSUPPORTED, "MN-major operands need bf16");
  LL_CHECK(N % 8 == 0 && ldc % 8 == 0 && ldc >= N, LL_ERR_UNSUPPORTED, "N and ldc must be multiples of 8, ldc >= N");
  const int64_t kp = round_up(K, ke);
  LL_CHECK(!ak || (lda >= kp && (lda * esz) % 16 == 0), LL_ERR_INVALID_ARG, "K-major A: lda >= K rounded to the K tile, 16-byte rows");
  LL_CHECK(!bk || (ldb >= kp && (ldb * esz) % 16 == 0), LL_ERR_INVALID_ARG, "K-major B: ldb >= K rounded to the K tile, 16-byte rows");
  LL_CHECK(ak || (lda >= M && lda % 8 == 0 && M % 8 == 0), LL_ERR_INVALID_ARG, "MN-major A: M % 8 == 0, lda >= M, lda % 8 == 0");
  LL_CHECK(bk || (ldb >= N && ldb % 8 == 0), LL_ERR_INVALID_ARG, "MN-major B: ldb >= N, ldb % 8 == 0");
  LL_CHECK((inv_a == nullptr) == (inv_b == nullptr), LL_ERR_INVALID_ARG, "inv_a and inv_b: both or neither");
  const size_t need = llt_gemm_splitk_workspace_bytes(M, N, slices);
  LL_CHECK(ws && aligned16(ws) && ws_bytes >= need, LL_ERR_WORKSPACE,
           "ws must be 16-byte aligned and hold llt_gemm_splitk_workspace_bytes");
  if (M == 0 || N == 0) return LL_OK;
  LL_CHECK(C && ((A && B) || K == 0), LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(A) && aligned16(B) && aligned16(C), LL_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  LL_HIP(fill_f32(static_cast<float*>(ws), 0.f, 64, s));
  const GemmOps o{ak, bk, ws};
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + 256);
  if (op_dtype == LLT_OP_BF16)
    return splitk_dispatch<bf16>(A, lda, B, ldb, M, N, K, slices, out_dtype, C, ldc, part, Deq{inv_a, inv_b}, o, s);
  return splitk_dispatch<fp8>(A, lda, B, ldb, M, N, K, slices, out_dtype, C, ldc, part, Deq{inv_a, inv_b}, o, s);
}

extern "C" int llt_set_gemm_config(int32_t cfg) {
  LL_CHECK(cfg >= 0 && cfg <= 15, LL_ERR_INVALID_ARG, "cfg must be in [0, 15]");
  set_gemm_config_override(cfg);
  return LL_OK;
}

// The cast step of the quantiser alone, on four values per thread with the kernels' own quant4:
// q[i] = e4m3fn_rne(clamp(fl32(x[i] * scale), -448, 448)), the NaN code 0x7F for a NaN product.
__global__ void __launch_bounds__(256) e4m3_cast_kernel(const float* __restrict__ x, int64_t n4, float scale,
                                                        uint32_t* __restrict__ q) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const floatx4 v = reinterpret_cast<const floatx4*>(x)[i];
    const float a[4] = {v[0], v[1], v[2], v[3]};
    q[i] = quant4(a, scale);
  }
}

extern "C" int llt_e4m3_cast(const float* x, int64_t n, float scale, uint8_t* q, void* stream) {
  LL_CHECK(n >= 0 && n % 4 == 0, LL_ERR_INVALID_ARG, "n must be a non-negative multiple of 4");
  if (n == 0) return LL_OK;
  LL_CHECK(x && q, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(x) && reinterpret_cast<uintptr_t>(q) % 4 == 0, LL_ERR_INVALID_ARG,
           "x must be 16-byte and q 4-byte aligned");
  const int64_t n4 = n / 4;
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(n4, 256), 16384);
  LL_LAUNCH("e4m3_cast", e4m3_cast_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), x, n4, scale,
            reinterpret_cast<uint32_t*>(q));
  LL_HIP(hipGetLastError());
  return LL_OK;
}
