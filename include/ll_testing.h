/*
 * ll_testing.h — kernel-level entry points of libll, exported so that each hot-path kernel can be
 * checked against the oracle on its own (the layer and loss entry points in ll.h compose them).
 * Same conventions as ll.h: device pointers, caller-owned memory, validation before any launch,
 * ll_status return codes, work enqueued on `stream` without host synchronisation.
 */
#ifndef LL_TESTING_H_
#define LL_TESTING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLT_OP_F32 = 0, LLT_OP_BF16 = 1, LLT_OP_E4M3 = 2 } llt_op_dtype;

/* C[m, n] = deq * sum_k A[m, k] B[n, k]  (both operands K-contiguous, row-major), the MFMA GEMM
 * of every projection of the layer and of the LM head.
 *   op_dtype: LLT_OP_F32 (fp32 MFMA), LLT_OP_BF16 (bf16 MFMA), LLT_OP_E4M3 (e4m3 MFMA).
 *   A [M, lda], B [N, ldb]: K must be a multiple of 128 bytes of the operand type
 *   (32 fp32 / 64 bf16 / 128 e4m3); lda, ldb >= K with rows 16-byte aligned.
 *   out_dtype: LL_F32 or LL_BF16 (ll.h); C [M, ldc], N % 8 == 0, ldc % 8 == 0.
 *   inv_a, inv_b: device fp32 scalars multiplied into the result (deq = *inv_a * *inv_b), or both
 *   NULL (deq = 1). The result is rounded once to out_dtype. */
int llt_gemm_nt(int32_t op_dtype, const void* A, int64_t lda, const void* B, int64_t ldb, int32_t M,
                int32_t N, int32_t K, int32_t out_dtype, void* C, int64_t ldc, const float* inv_a,
                const float* inv_b, void* stream);

/* Launch trace: while tracing is on, every kernel launch of the library is bracketed by two HIP
 * events recorded on the launch's own stream and tagged with the kernel's name (GEMMs as
 * "gemm_<operand type>_<epilogue>"). Up to `capacity` launches are recorded per begin; later ones
 * are not traced. The events are created by llt_trace_begin (the only call here that creates
 * HIP objects) and reused until the capacity changes. Not thread-safe across concurrent
 * begin/get on different threads beyond the internal lock; host-side bookkeeping only.
 *   llt_trace_begin: reset and start recording; llt_trace_end: stop recording;
 *   llt_trace_count: launches recorded; llt_trace_get: tag and duration (ms) of launch i, waiting
 *   for its end event, and (if mnk is not NULL) the GEMM sizes M, N, K of that launch (0 for
 *   launches that are not GEMMs). */
int llt_trace_begin(int32_t capacity);
int llt_trace_end(void);
int32_t llt_trace_count(void);
int llt_trace_get(int32_t i, const char** tag, float* ms, int64_t* mnk);

#ifdef __cplusplus
}
#endif

#endif /* LL_TESTING_H_ */
