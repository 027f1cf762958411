// ll_fused_lce_fwd_bwd: chunked fused linear cross-entropy with tanh logit softcap.
#include "api.h"
#include "gemm.h"
#include "lce.h"
#include "norm.h"
#include "quant.h"

using namespace ll;

namespace {

// Vocabulary tile of the logits GEMM = the columns of one row-sum partial: 256 (256 x 256 block
// tiles, the default) or 128 (128 x 128 block tiles)
constexpr int kDefaultVocabTile = 256;
constexpr int64_t kDefaultChunk = 10240;
// block configuration of the logits GEMM with 256-wide vocabulary tiles (configuration 14: 16x16x32
// MFMAs, ping-pong K loop)
constexpr int kLogitsConfig = 14;
// block order of the logits and dH GEMMs: four tile columns (rows) at a time (~1% faster than the
// default two; the dW GEMM keeps two)
const GemmOps kGroup4Ops{true, true, nullptr, 4};

struct LcePlan {
  int64_t chunk, chunk_pad, vpad;
  int nparts, vtile;
  float* part = nullptr;
  void* z = nullptr;        // [chunk_pad, Vpad]  (z, then dz in place)
  void* wt = nullptr;       // W^T [D, Vpad], zero past V
  void* dzt = nullptr;      // dz^T [Vpad, chunk_pad]
  void* ht = nullptr;       // H_c^T [D, chunk_pad]
  void* zrow = nullptr;     // 256 zero bytes (K tails of MN-major operands)
  float* dw32 = nullptr;    // [V, D] fp32 accumulator (several chunks)
  bool single = false;      // one chunk holds every token
  float* lse = nullptr;     // [chunk]
  float* loss_acc = nullptr;
  int* nv = nullptr;
  size_t bytes = 0;
};

LcePlan plan_lce(void* ws, int es, int64_t n, int d, int64_t v, int64_t token_chunk, int vocab_tile, bool grads) {
  LcePlan p;
  p.vtile = vocab_tile > 0 ? vocab_tile : kDefaultVocabTile;
  p.chunk = token_chunk > 0 ? token_chunk : kDefaultChunk;
  if (p.chunk > n) p.chunk = n > 0 ? n : 1;
  // one chunk holds every token: the weight gradient is one contraction over all of them and is
  // rounded straight into d_weight (no fp32 accumulator across chunks); with several chunks the
  // last chunk's GEMM rounds the fp32 total into d_weight
  p.single = n > 0 && p.chunk >= n;
  p.chunk_pad = round_up(p.chunk, 64);
  p.vpad = round_up(v, 64);
  p.nparts = (int)cdiv(v, p.vtile);
  Carver c(ws);
  p.loss_acc = c.take<float>(4);
  p.nv = c.take<int>(4);
  p.zrow = c.take<char>(256);
  p.lse = c.take<float>(p.chunk_pad);
  p.part = c.take<float>(p.chunk_pad * p.nparts);
  p.z = c.take<char>((size_t)p.chunk_pad * p.vpad * es);
  if (grads) {
    p.wt = c.take<char>((size_t)d * p.vpad * es);           // W^T [D, Vpad] (K-major B of the dH GEMM)
    p.dzt = c.take<char>((size_t)p.vpad * p.chunk_pad * es);  // dz^T and H_c^T: K-major operands
    p.ht = c.take<char>((size_t)d * p.chunk_pad * es);        // of the dW GEMM
    if (!p.single) p.dw32 = c.take<float>((size_t)v * d);
  }
  p.bytes = c.bytes();
  return p;
}

template <class T>
int run_lce(const T* H, const T* W, const int32_t* y, int64_t n, int d, int64_t v, float softcap,
            int32_t ignore, float grad_scale, const LcePlan& p, float* loss, float* lse_out, T* dH, T* dW,
            int accumulate_dw, hipStream_t s) {
  const bool grads = dH != nullptr;
  constexpr bool kBf16 = std::is_same<T, bf16>::value;
  LL_HIP(fill_f32(p.loss_acc, 0.f, 4, s));
  LL_HIP(fill_f32(reinterpret_cast<float*>(p.nv), 0.f, 4, s));
  LL_HIP(fill_f32(static_cast<float*>(p.zrow), 0.f, 64, s));
  if (n > 0) {
    LL_LAUNCH("count_valid", count_valid_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 1024)), dim3(256), 0, s,
              y, n, ignore, p.nv);
    LL_HIP(hipGetLastError());
  }
  if (grads) LL_HIP(transpose2d(W, v, d, (int64_t)d, static_cast<T*>(p.wt), p.vpad, p.vpad, s));
  T* z = static_cast<T*>(p.z);
  for (int64_t r0 = 0; r0 < n; r0 += p.chunk) {
    const int rows = (int)std::min<int64_t>(p.chunk, n - r0);
    const T* Hc = H + r0 * d;
    constexpr float kLog2e = 1.4426950408889634f;
    EpiLceLogits<T> epi{z, p.vpad, p.part, p.nparts, 2.f * kLog2e / softcap, softcap * kLog2e};
    {
      // one row-sum partial per block tile of vocab_tile columns: 256 -> configuration 14 (or an
      // override with 256-wide tiles), 128 -> configuration 1 (or 7)
      const int oc = gemm_config_override();
      const int cfg = p.vtile == 128 ? (oc == 7 ? 7 : 1)
                                     : ((oc >= 2 && oc <= 6) || (oc >= 8 && oc <= 14) ? oc : kLogitsConfig);
      const hipError_t e = launch_gemm_with(cfg, Hc, (int64_t)d, W, (int64_t)d, rows, (int)v, d, epi, kGroup4Ops, s);
      LL_HIP(e);
    }
    LL_LAUNCH("lce_lse", (lce_lse_kernel<T>), dim3((unsigned)cdiv(rows, kLseRows)), dim3(256), 0, s, p.part, p.nparts, z,
              p.vpad, y + r0, rows, ignore, softcap, lse_out ? lse_out + r0 : nullptr, p.lse, p.loss_acc);
    LL_HIP(hipGetLastError());
    if (!grads) continue;
    const int rows_pad = (int)round_up(rows, 64);
    if constexpr (kBf16) {
      LL_LAUNCH("lce_dz", lce_dz_t_kernel, dim3((unsigned)(p.vpad / 64), (unsigned)(rows_pad / 64)), dim3(256), 0, s,
                z, p.vpad, p.lse, y + r0, rows, (int)v, ignore, softcap, grad_scale, p.nv,
                static_cast<T*>(p.dzt), (int64_t)rows_pad);
    } else {
      dim3 g((unsigned)cdiv(p.vpad, 64), (unsigned)cdiv(rows_pad, 64));
      LL_LAUNCH("lce_dz", (lce_dz_kernel<T>), g, dim3(256), 0, s, z, p.vpad, p.lse, y + r0, rows, rows_pad, (int)v,
                (int)p.vpad, ignore, softcap, grad_scale, p.nv, z, static_cast<T*>(p.dzt), (int64_t)rows_pad);
    }
    LL_HIP(hipGetLastError());
    EpiLceDh<T> eh{{dH + r0 * d, (int64_t)d, Deq{nullptr, nullptr}}};
    // dW += dz^T H_c: A = dz^T [Vpad, rows_pad], B = H_c^T [D, rows_pad], both K-major over the
    // chunk's tokens (zero past rows); with one chunk the exact fp32 sum over all tokens is
    // rounded straight into dW
    LL_HIP(transpose2d(Hc, rows, d, (int64_t)d, static_cast<T*>(p.ht), (int64_t)rows_pad, (int64_t)rows_pad, s));
    const T* dzt = static_cast<const T*>(p.dzt);
    const T* ht = static_cast<const T*>(p.ht);
    const T* wt = static_cast<const T*>(p.wt);
    // dH_c = dz W: A = dz [rows, Vpad] (K-major), B(n = d, k = v) = W^T[d, v] (K-major, zero past V).
    // bf16 runs dH_c and dW's GEMM in one grid, dH's long-K tiles first.
    auto grads_gemms = [&](auto ew) -> hipError_t {
      if constexpr (kBf16) {
        if (gemm_pair_ok<bf16>(p.vpad, p.vpad, rows_pad, rows_pad)) {
          EpiLceGrads<T, decltype(ew)> e{};
          e.e0 = eh;
          e.e1 = ew;
          e.a1 = dzt;
          e.lda1 = rows_pad;
          e.b1 = ht;
          e.ldb1 = rows_pad;
          e.m1 = (int)v;
          e.n1 = d;
          e.k1 = rows_pad;
          e.g1 = 2;
          return launch_gemm_pair(z, p.vpad, wt, p.vpad, rows, d, (int)p.vpad, 4, e, s);
        }
      }
      const hipError_t r = launch_gemm(z, p.vpad, wt, p.vpad, rows, d, (int)p.vpad, eh, kGroup4Ops, s);
      if (r != hipSuccess) return r;
      return launch_gemm(dzt, (int64_t)rows_pad, ht, (int64_t)rows_pad, (int)v, d, rows_pad, ew, GemmOps{}, s);
    };
    if (p.single) {
      LL_HIP(grads_gemms(EpiStore<T>{dW, (int64_t)d, Deq{nullptr, nullptr}, accumulate_dw}));
    } else if (r0 + rows < n) {
      // fp32 sums over the chunks in dw32
      LL_HIP(grads_gemms(EpiAcc32{p.dw32, (int64_t)d, r0 > 0 ? 1 : 0}));
    } else {
      // the last chunk's GEMM rounds the fp32 total into dW
      LL_HIP(grads_gemms(EpiAcc32Out<T>{p.dw32, dW, (int64_t)d, accumulate_dw}));
    }
  }
  if (grads && n == 0 && !accumulate_dw) {                 // no chunk ran: dW = 0 (unchanged when accumulating)
    LL_HIP(fill_f32(p.dw32, 0.f, v * d, s));
    LL_HIP(launch_convert(p.dw32, dW, v * d, s));
  }
  LL_LAUNCH("lce_finalize", lce_finalize_kernel, dim3(1), dim3(1), 0, s, p.loss_acc, p.nv, loss);
  LL_HIP(hipGetLastError());
  return LL_OK;
}

}  // namespace

extern "C" size_t ll_fused_lce_workspace_bytes(int32_t dtype, int64_t n, int32_t d, int64_t v, int64_t token_chunk,
                                               int32_t vocab_tile) {
  if ((dtype != LL_F32 && dtype != LL_BF16) || n < 0 || d <= 0 || v <= 0) return 0;
  if (vocab_tile != 0 && vocab_tile != 128 && vocab_tile != 256) return 0;
  const int es = dtype == LL_F32 ? 4 : 2;
  return plan_lce(nullptr, es, n, d, v, token_chunk, vocab_tile, true).bytes;
}

extern "C" int ll_fused_lce_fwd_bwd(int32_t dtype, const void* hidden, const void* weight, const int32_t* targets,
                                    int64_t n, int32_t d, int64_t v, float softcap, int32_t ignore_index,
                                    float grad_scale, int64_t token_chunk, int32_t vocab_tile, int32_t accumulate_dw,
                                    float* loss, float* lse, void* d_hidden, void* d_weight, void* ws,
                                    size_t ws_bytes, void* stream) {
  LL_CHECK(dtype == LL_F32 || dtype == LL_BF16, LL_ERR_INVALID_ARG, "dtype must be LL_F32 or LL_BF16");
  LL_CHECK(n >= 0 && d > 0 && v > 0, LL_ERR_INVALID_ARG, "need n >= 0, d > 0, v > 0");
  LL_CHECK(d % (dtype == LL_F32 ? 32 : 64) == 0, LL_ERR_UNSUPPORTED, "d must be a multiple of 64 (bf16) / 32 (fp32)");
  LL_CHECK(v % 8 == 0, LL_ERR_UNSUPPORTED, "v must be a multiple of 8");
  LL_CHECK(v < (int64_t)1 << 31 && n < (int64_t)1 << 31, LL_ERR_UNSUPPORTED, "n and v must fit in int32");
  // the row sums of exp(c) carry no running maximum: |c| <= softcap keeps v * e^softcap far below
  // the fp32 range (3.4e38) for any vocabulary up to 10^12 rows when softcap <= 60
  LL_CHECK(softcap > 0.f && softcap <= 60.f, LL_ERR_INVALID_ARG, "softcap must be in (0, 60]");
  LL_CHECK(token_chunk >= 0, LL_ERR_INVALID_ARG, "token_chunk must be >= 0");
  LL_CHECK(vocab_tile == 0 || vocab_tile == 128 || vocab_tile == 256, LL_ERR_UNSUPPORTED,
           "vocab_tile must be 0 (default 256), 128 or 256");
  LL_CHECK(accumulate_dw == 0 || accumulate_dw == 1, LL_ERR_INVALID_ARG, "accumulate_dw must be 0 or 1");
  LL_CHECK(token_chunk == 0 || token_chunk <= (int64_t)65535 * 64, LL_ERR_UNSUPPORTED, "token_chunk too large");
  LL_CHECK(loss, LL_ERR_INVALID_ARG, "loss must not be null");
  LL_CHECK((d_hidden == nullptr) == (d_weight == nullptr), LL_ERR_INVALID_ARG, "d_hidden and d_weight: both or neither");
  LL_CHECK(weight && aligned16(weight), LL_ERR_INVALID_ARG, "weight must be a 16-byte aligned device pointer");
  LL_CHECK(n == 0 || (hidden && targets && aligned16(hidden)), LL_ERR_INVALID_ARG, "hidden/targets must not be null");
  LL_CHECK(!d_hidden || (aligned16(d_hidden) && aligned16(d_weight)), LL_ERR_INVALID_ARG, "gradients must be 16-byte aligned");
  const int es = dtype == LL_F32 ? 4 : 2;
  const bool grads = d_hidden != nullptr;
  const size_t need = plan_lce(nullptr, es, n, d, v, token_chunk, vocab_tile, grads).bytes;
  LL_CHECK(ws && aligned16(ws), LL_ERR_INVALID_ARG, "ws must be a 16-byte aligned device pointer");
  LL_CHECK(ws_bytes >= need, LL_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  const LcePlan p = plan_lce(ws, es, n, d, v, token_chunk, vocab_tile, grads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LL_BF16)
    return run_lce(static_cast<const bf16*>(hidden), static_cast<const bf16*>(weight), targets, n, d, v, softcap,
                   ignore_index, grad_scale, p, loss, lse, static_cast<bf16*>(d_hidden), static_cast<bf16*>(d_weight),
                   accumulate_dw, s);
  return run_lce(static_cast<const float*>(hidden), static_cast<const float*>(weight), targets, n, d, v, softcap,
                 ignore_index, grad_scale, p, loss, lse, static_cast<float*>(d_hidden), static_cast<float*>(d_weight),
                 accumulate_dw, s);
}
