// ll_muon_step / ll_adamw_step: the optimizer step of the little-lm training run
// [youdonthavefriends cost analysis, "config appendix": Muon (lr 0.02, momentum 0.95, weight decay
// 0) for the matrix parameters, AdamW with per-group settings for the rest; linlog.top article,
// 吞吐量优化: bf16 master weights]. Muon's Newton-Schulz coefficients and iteration count are not on
// the pages; they are those its author published (K. Jordan, "Muon: An optimizer for hidden layers
// in neural networks", 2024): X <- a X + (b A + c A A) X with A = X X^T, (a, b, c) = (3.4445,
// -4.7750, 2.0315), 5 iterations, X_0 = u / (||u||_F + 1e-7), on the wide orientation of the matrix.
#include "api.h"
#include "gemm.h"
#include "norm.h"
#include "optim.h"
#include "quant.h"

using namespace ll;

namespace {

constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f, kNsEps = 1e-7f;

struct MuonWs {
  float* ss;
  bf16* zrow;
  bf16 *u, *x0, *x1, *a, *b;
};
size_t carve_muon(void* base, int64_t rows, int64_t cols, MuonWs& w) {
  const int64_t m = std::min(rows, cols), n = std::max(rows, cols);
  Carver c(base);
  w.ss = c.take<float>(4);
  w.zrow = c.take<bf16>(128);
  w.u = c.take<bf16>(rows * cols);
  w.x0 = c.take<bf16>(m * n);
  w.x1 = c.take<bf16>(m * n);
  w.a = c.take<bf16>(m * m);
  w.b = c.take<bf16>(m * m);
  return c.bytes();
}

unsigned ew_blocks(int64_t work) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(work, 256), 8192)); }

}  // namespace

extern "C" size_t ll_muon_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0) return 0;
  MuonWs w;
  return carve_muon(nullptr, rows, cols, w);
}

extern "C" int ll_muon_step(int32_t dtype, void* w, const void* grad, void* momentum_buf, int64_t rows, int64_t cols,
                            float lr, float momentum, int32_t nesterov, float weight_decay, int32_t ns_steps,
                            void* ws, size_t ws_bytes, void* stream) {
  LL_CHECK(dtype == LL_BF16, LL_ERR_UNSUPPORTED, "Muon runs on bf16 master weights (dtype LL_BF16)");
  LL_CHECK(rows > 0 && cols > 0, LL_ERR_INVALID_ARG, "rows and cols must be > 0");
  LL_CHECK(rows % 64 == 0 && cols % 64 == 0, LL_ERR_UNSUPPORTED,
           "rows and cols must be multiples of 64 (the GEMMs read whole 64-element K tiles)");
  LL_CHECK(rows <= 65536 && cols <= 65536, LL_ERR_UNSUPPORTED, "rows and cols must be <= 65536");
  LL_CHECK(ns_steps >= 0 && ns_steps <= 16, LL_ERR_INVALID_ARG, "ns_steps must be in [0, 16]");
  LL_CHECK(nesterov == 0 || nesterov == 1, LL_ERR_INVALID_ARG, "nesterov must be 0 or 1");
  LL_CHECK(w && grad && momentum_buf && ws, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(w) && aligned16(grad) && aligned16(momentum_buf) && aligned16(ws), LL_ERR_INVALID_ARG,
           "pointers must be 16-byte aligned");
  MuonWs mw;
  const size_t need = carve_muon(nullptr, rows, cols, mw);
  LL_CHECK(ws_bytes >= need, LL_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  carve_muon(ws, rows, cols, mw);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool tall = rows > cols;
  const int m = (int)std::min(rows, cols), n = (int)std::max(rows, cols);
  const int64_t n8 = rows * cols / 8;
  bf16* W = static_cast<bf16*>(w);
  LL_HIP(fill_f32(mw.ss, 0.f, 4, s));
  LL_HIP(fill_f32(reinterpret_cast<float*>(mw.zrow), 0.f, 64, s));
  LL_LAUNCH("muon_momentum", muon_momentum_kernel<bf16>, dim3(ew_blocks(n8)), dim3(256), 0, s,
            static_cast<const bf16*>(grad), static_cast<bf16*>(momentum_buf), mw.u, n8, momentum, nesterov, mw.ss);
  LL_HIP(hipGetLastError());
  // X_0 in the wide orientation [m, n]: u / (||u|| + eps), transposed when u is tall
  bf16* x = mw.x0;
  bf16* xn = mw.x1;
  if (tall) {
    LL_LAUNCH("muon_normalise", muon_normalise_kernel<bf16>, dim3(ew_blocks(n8)), dim3(256), 0, s, mw.u, mw.x1, n8,
              mw.ss, kNsEps);
    LL_HIP(hipGetLastError());
    LL_HIP(transpose2d(mw.x1, rows, (int)cols, cols, x, rows, rows, s));
  } else {
    LL_LAUNCH("muon_normalise", muon_normalise_kernel<bf16>, dim3(ew_blocks(n8)), dim3(256), 0, s, mw.u, x, n8,
              mw.ss, kNsEps);
    LL_HIP(hipGetLastError());
  }
  // Newton-Schulz: A = X X^T (both operands X, K-major over n); B = b A + c A A (A symmetric:
  // A A = A A^T); X' = a X + B X (B K-major, X read MN-major over its m rows)
  const GemmOps mn{true, false, mw.zrow};
  for (int it = 0; it < ns_steps; ++it) {
    EpiStore<bf16> ea{mw.a, (int64_t)m, Deq{nullptr, nullptr}};
    LL_HIP(launch_gemm(x, (int64_t)n, x, (int64_t)n, m, m, n, ea, GemmOps{}, s));
    EpiLin<bf16> eb{mw.b, mw.a, (int64_t)m, kNsB, kNsC};
    LL_HIP(launch_gemm(mw.a, (int64_t)m, mw.a, (int64_t)m, m, m, m, eb, GemmOps{}, s));
    EpiLin<bf16> ex{xn, x, (int64_t)n, kNsA, 1.f};
    LL_HIP(launch_gemm(mw.b, (int64_t)m, x, (int64_t)n, m, n, m, ex, mn, s));
    std::swap(x, xn);
  }
  // W = round(W (1 - lr wd) - lr sqrt(max(1, rows / cols)) O), O in W's orientation
  const bf16* o = x;
  if (tall) {
    LL_HIP(transpose2d(x, (int64_t)m, n, (int64_t)n, mw.u, (int64_t)m, (int64_t)m, s));
    o = mw.u;
  }
  const float step = lr * std::sqrt(std::max(1.0f, (float)rows / (float)cols));
  LL_LAUNCH("muon_apply", muon_apply_kernel<bf16>, dim3(ew_blocks(n8)), dim3(256), 0, s, W, o, n8,
            1.f - lr * weight_decay, step);
  LL_HIP(hipGetLastError());
  return LL_OK;
}

extern "C" int ll_adamw_step(int32_t param_dtype, int32_t grad_dtype, void* param, const void* grad, void* exp_avg,
                             void* exp_avg_sq, int64_t n, float lr, float beta1, float beta2, float eps,
                             float weight_decay, int64_t step, void* stream) {
  LL_CHECK(param_dtype == LL_F32 || param_dtype == LL_BF16, LL_ERR_INVALID_ARG, "param_dtype must be LL_F32 or LL_BF16");
  LL_CHECK(grad_dtype == LL_F32 || grad_dtype == LL_BF16, LL_ERR_INVALID_ARG, "grad_dtype must be LL_F32 or LL_BF16");
  LL_CHECK(n >= 0, LL_ERR_INVALID_ARG, "n must be >= 0");
  LL_CHECK(step >= 1, LL_ERR_INVALID_ARG, "step must be >= 1 (the first step is 1)");
  LL_CHECK(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f, LL_ERR_INVALID_ARG, "betas must be in [0, 1)");
  LL_CHECK(eps > 0.f, LL_ERR_INVALID_ARG, "eps must be > 0");
  if (n == 0) return LL_OK;
  LL_CHECK(param && grad && exp_avg && exp_avg_sq, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(param) && aligned16(grad) && aligned16(exp_avg) && aligned16(exp_avg_sq), LL_ERR_INVALID_ARG,
           "pointers must be 16-byte aligned");
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  const AdamWArgs a{beta1, beta2, eps, 1.f - lr * weight_decay, (float)(lr / bc1), (float)(1.0 / std::sqrt(bc2))};
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(ew_blocks(cdiv(n, 4))), blk(256);
  const bool pb = param_dtype == LL_BF16, gb = grad_dtype == LL_BF16;
  if (pb && gb)
    LL_LAUNCH("adamw", (adamw_kernel<bf16, bf16>), grid, blk, 0, s, static_cast<bf16*>(param),
              static_cast<const bf16*>(grad), static_cast<bf16*>(exp_avg), static_cast<bf16*>(exp_avg_sq), n, a);
  else if (pb)
    LL_LAUNCH("adamw", (adamw_kernel<bf16, float>), grid, blk, 0, s, static_cast<bf16*>(param),
              static_cast<const float*>(grad), static_cast<bf16*>(exp_avg), static_cast<bf16*>(exp_avg_sq), n, a);
  else if (gb)
    LL_LAUNCH("adamw", (adamw_kernel<float, bf16>), grid, blk, 0, s, static_cast<float*>(param),
              static_cast<const bf16*>(grad), static_cast<float*>(exp_avg), static_cast<float*>(exp_avg_sq), n, a);
  else
    LL_LAUNCH("adamw", (adamw_kernel<float, float>), grid, blk, 0, s, static_cast<float*>(param),
              static_cast<const float*>(grad), static_cast<float*>(exp_avg), static_cast<float*>(exp_avg_sq), n, a);
  LL_HIP(hipGetLastError());
  return LL_OK;
}
