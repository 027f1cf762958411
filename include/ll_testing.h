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

#include "ll.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LLT_OP_F32 = 0, LLT_OP_BF16 = 1, LLT_OP_E4M3 = 2 } llt_op_dtype;

/* C[m, n] = deq * sum_k A(m, k) B(n, k), the MFMA GEMM of every projection of the layer and of the
 * LM head, with each operand K-major (A(m, k) = A[m * lda + k]) or MN-major (A(m, k) = A[k * lda + m]).
 *   op_dtype: LLT_OP_F32 (fp32 MFMA), LLT_OP_BF16 (bf16 MFMA), LLT_OP_E4M3 (e4m3 MFMA). MN-major
 *   operands are bf16 only (read with LDS transpose reads) and need M (resp. N) % 8 == 0.
 *   K-major operands are read in whole K tiles of 128 bytes (32 fp32 / 64 bf16 / 128 e4m3): their
 *   rows must hold K rounded up to the tile, zero beyond K. MN-major operands may end at row K.
 *   out_dtype: LL_F32 or LL_BF16 (ll.h); C [M, ldc], N % 8 == 0, ldc % 8 == 0.
 *   inv_a, inv_b: device fp32 scalars multiplied into the result (deq = *inv_a * *inv_b), or both
 *   NULL (deq = 1). The result is rounded once to out_dtype.
 *   ws: >= 64 bytes of device scratch when an operand is MN-major (a zero row), else unused. */
int llt_gemm(int32_t op_dtype, int32_t a_kmajor, int32_t b_kmajor, const void* A, int64_t lda, const void* B,
             int64_t ldb, int32_t M, int32_t N, int32_t K, int32_t out_dtype, void* C, int64_t ldc,
             const float* inv_a, const float* inv_b, void* ws, size_t ws_bytes, void* stream);

/* The same product (bf16, or e4m3 with both operands K-major) split along K: slice s (of `slices`,
 * 1..16) sums K elements [s c, min(K, (s + 1) c)), c = K / slices rounded up to the K tile (64 bf16,
 * 128 e4m3), into fp32 partials in ws; a second kernel adds the slices in order, multiplies by
 * *inv_a * *inv_b (if given) and rounds once to out_dtype. Used for weight gradients whose output
 * has too few 256 x 256 tiles to fill the chip. Layouts, padding and scales as llt_gemm.
 *   ws: >= llt_gemm_splitk_workspace_bytes(M, N, slices) bytes, 16-byte aligned (256 bytes of zero
 *   row for MN-major K tails, then slices * M * N fp32 partials). K == 0 writes zeros (A and B may
 *   then be NULL). */
size_t llt_gemm_splitk_workspace_bytes(int32_t M, int32_t N, int32_t slices);
int llt_gemm_splitk(int32_t op_dtype, int32_t a_kmajor, int32_t b_kmajor, const void* A, int64_t lda, const void* B,
                    int64_t ldb, int32_t M, int32_t N, int32_t K, int32_t slices, int32_t out_dtype, void* C,
                    int64_t ldc, const float* inv_a, const float* inv_b, void* ws, size_t ws_bytes, void* stream);

/* Process-wide override of the GEMM configuration (for measurements). Block tile, waves, bytes of K
 * per LDS tile row, LDS stages: 1 = 128 x 128, 4 waves, 128 B, 2; 2 = 256 x 256, 4 waves, 128 B, 2;
 * 3 = 256 x 256, 8 waves (2 x 4), 128 B, 2; 4 = 256 x 256, 8 waves (4 x 2), 128 B, 2;
 * 5 = 256 x 256, 8 waves (2 x 4), 64 B, 3; 6 = 256 x 256, 8 waves (4 x 2), 64 B, 3;
 * 7 = 128 x 128, 4 waves, 64 B, 3; 8 = 256 x 256, 4 waves (2 x 2), 64 B, 3, next-tile fragments
 * prefetched into registers; 9 = 256 x 256, 8 waves (4 x 2), 128 B, 2, split-phase K loop (the
 * fragments of one half of a K tile are read while the MFMAs of the other half run, the reads and
 * half the next tile's loads interleaved with those MFMAs); 10 = split-phase with 4 waves (2 x 2),
 * reads and MFMAs in separate groups; 11 = 256 x 256, 8 waves (4 x 2), 128 B, 2, split-phase K loop
 * on the 32x32 MFMAs (32x32x64 e4m3, 32x32x16 bf16; bf16 with an MN-major operand runs it as 9). e4m3 GEMMs need 128-byte K tiles and run
 * 5, 6, 7 as 3, 4, 1 and 8, 9, 10 as 4; fp32 runs 9, 10 and 11 as 4. 0 = automatic choice per GEMM shape. The LCE logits GEMM
 * always uses a 256-wide vocabulary tile (configurations 1, 7 and 8 select 9 there). */
int llt_set_gemm_config(int32_t cfg);

/* Token-embedding gather and its gradient [hn.213312.xyz translation, 设置 / Setup: token
 * embedding table; the same kernels serve the model's embedding]:
 *   out[i, :] = table[ids[i], :] (zeros for ids outside [0, rows));
 *   d_table[ids[i], :] += d_out[i, :] in fp32 (ids outside [0, rows) skipped; atomic adds).
 * dtype: LL_F32 or LL_BF16 for table/out/d_out; d % 8 == 0, d <= 4096. */
int llt_embedding_gather(int32_t dtype, const void* table, int64_t rows, int32_t d, const int32_t* ids, int64_t n,
                         void* out, void* stream);
int llt_embedding_scatter_add(int32_t dtype, const void* d_out, const int32_t* ids, int64_t n, int32_t d,
                              float* d_table, int64_t rows, void* stream);

/* RMSNorm of x [n, d] with fp32 gain g [hn.213312.xyz translation, 设置 / Setup; rms_norm_eps
 * 1e-6 in the "config appendix" of the youdonthavefriends cost analysis]:
 *   rstd = 1 / sqrt(mean(x^2) + eps) (fp32 [n]), y = round(x rstd g);
 * backward: dx = round(rstd (g dy) - x rstd^3 mean(x g dy)), dg = sum over rows of dy x rstd
 * (fp32 [d], written). d % 8 == 0, d <= 4096. */
int llt_rmsnorm_fwd(int32_t dtype, const void* x, const float* g, int64_t n, int32_t d, float eps, void* y,
                    float* rstd, void* stream);
size_t llt_rmsnorm_bwd_workspace_bytes(int64_t n, int32_t d);
int llt_rmsnorm_bwd(int32_t dtype, const void* dy, const void* x, const float* g, const float* rstd, int64_t n,
                    int32_t d, void* dx, float* dg, void* ws, size_t ws_bytes, void* stream);

/* Launch trace: while tracing is on, every kernel launch of the library is bracketed by two HIP
 * events recorded on the launch's own stream and tagged with the kernel's name (GEMMs as
 * "gemm_<operand type>_<epilogue>_<A layout><B layout>", layout k = K-major, m = MN-major). Up to `capacity` launches are recorded per begin; later ones
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
/* For a GEMM launch i of the trace: the block configuration that ran (the numbers of
 * llt_set_gemm_config, after the per-type fallbacks) and the number of K slices of its grid (1 for
 * an unsplit GEMM); both 0 for launches that are not GEMMs. */
int llt_trace_get_gemm(int32_t i, int32_t* gemm_cfg, int32_t* slices);

/* Where the layer keeps one of its intermediate tensors, so that a test can read it back: the
 * byte offset and size of sub-buffer `name` inside the `saved` buffer (region 0), the forward
 * workspace (region 1) or the backward workspace (region 2) of ll_layer_fwd / ll_layer_bwd for
 * this cfg. Host-side layout arithmetic only (no device access).
 *   saved:    "qs" (4 x {amax, scale, inv_scale, pad} fp32: hn, w_fc, r, w_proj), "xn", "qkv", "qh",
 *             "kh", "o", "lse", "attn_out", "h", "u", "m", "r1", "r2", "hn8", "hn8t", "r8t", "w18",
 *             "w18t", "w28", "w28t" (e4m3 codes, *t = transposed with the token axis padded to
 *             a multiple of 128 and zero-filled);
 *   fwd ws:   "hn" (bf16 input of the hn quantiser), "r8" (codes of r);
 *   bwd ws:   "qs" (2 x {amax, scale, inv_scale, pad}: dm, du), "dm", "du" (bf16 inputs of their
 *             quantisers), "dm8", "dm8t", "du8", "du8t", "dhn", "dh", "dattn", "dout", "dqkv", "dxn".
 * Returns LL_ERR_INVALID_ARG for an invalid cfg or a name the configuration does not hold. */
int llt_layer_buffer(const ll_layer_cfg* cfg, int32_t region, const char* name, size_t* offset, size_t* bytes);

/* The cast step of the e4m3 quantiser alone, with the same device code as ll_fp8_quant_tensorwise
 * and the layer's casts [hn.213312.xyz translation, 提升吞吐量 / Increasing throughput: FP8 with
 * dynamic scaling], for a caller-chosen scale:
 *   q[i] = e4m3fn_rne(clamp(fl32(x[i] * scale), -448, 448)), and the NaN code 0x7F where the
 *   product is NaN (so +-inf inputs give +-448 at any nonzero scale).
 * x: n fp32 values (device, 16-byte aligned); q: n bytes (device, 4-byte aligned); n % 4 == 0.
 * Asynchronous on `stream`. Used to sweep every fp32 bit pattern against a host emulator. */
int llt_e4m3_cast(const float* x, int64_t n, float scale, uint8_t* q, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LL_TESTING_H_ */
