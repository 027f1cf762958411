// ll_fp8_quant_tensorwise: the stand-alone dynamic tensorwise e4m3fn quantiser.
#include "api.h"
#include "quant.h"

using namespace ll;

extern "C" size_t ll_fp8_quant_workspace_bytes(void) { return sizeof(QScale); }

extern "C" int ll_fp8_quant_tensorwise(int32_t in_dtype, const void* x, int64_t rows, int64_t cols,
                                       int64_t ld, uint8_t* q, uint8_t* q_t, float* scale,
                                       float* inv_scale, void* ws, size_t ws_bytes, void* stream) {
  LL_CHECK(in_dtype == LL_F32 || in_dtype == LL_BF16, LL_ERR_INVALID_ARG, "in_dtype must be LL_F32 or LL_BF16");
  LL_CHECK(rows >= 0 && cols >= 0, LL_ERR_INVALID_ARG, "rows and cols must be >= 0");
  LL_CHECK(cols % 16 == 0, LL_ERR_UNSUPPORTED, "cols must be a multiple of 16");
  LL_CHECK(cols <= (int64_t)1 << 30 && rows <= ((int64_t)65535 * 64), LL_ERR_UNSUPPORTED, "tensor too large");
  LL_CHECK(ld >= cols && ld % 8 == 0, LL_ERR_INVALID_ARG, "ld must be >= cols and a multiple of 8");
  LL_CHECK(scale && inv_scale, LL_ERR_INVALID_ARG, "scale and inv_scale must not be null");
  LL_CHECK(ws, LL_ERR_INVALID_ARG, "ws must not be null");
  LL_CHECK(ws_bytes >= sizeof(QScale), LL_ERR_WORKSPACE, "workspace too small");
  LL_CHECK(aligned16(ws), LL_ERR_INVALID_ARG, "ws must be 16-byte aligned");
  const bool empty = rows == 0 || cols == 0;
  LL_CHECK(empty || x, LL_ERR_INVALID_ARG, "x must not be null");
  LL_CHECK(empty || aligned16(x), LL_ERR_INVALID_ARG, "x must be 16-byte aligned");
  LL_CHECK(!q || aligned16(q), LL_ERR_INVALID_ARG, "q must be 16-byte aligned");
  LL_CHECK(!q_t || aligned16(q_t), LL_ERR_INVALID_ARG, "q_t must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  QScale* qs = static_cast<QScale*>(ws);
  LL_HIP(fill_f32(&qs->amax, 0.f, 1, s));
  if (in_dtype == LL_BF16) {
    LL_HIP(launch_amax(static_cast<const bf16*>(x), rows, (int)cols, ld, &qs->amax, s));
    LL_HIP(launch_cast_e4m3(static_cast<const bf16*>(x), rows, (int)cols, ld, qs, q, cols, q_t, rows, rows,
                            scale, inv_scale, s));
  } else {
    LL_HIP(launch_amax(static_cast<const float*>(x), rows, (int)cols, ld, &qs->amax, s));
    LL_HIP(launch_cast_e4m3(static_cast<const float*>(x), rows, (int)cols, ld, qs, q, cols, q_t, rows, rows,
                            scale, inv_scale, s));
  }
  return LL_OK;
}

