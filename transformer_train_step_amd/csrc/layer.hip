// ll_layer_fwd / ll_layer_bwd: one little-lm decoder layer [hn.213312.xyz translation, 设置 /
// Setup; youdonthavefriends cost analysis, "config appendix"], as a fixed sequence of launches on
// the caller's stream. Every GEMM is C = A B^T with both operands K-contiguous; the operands a
// GEMM needs K-contiguous along the token axis (weight gradients) are produced transposed by their
// producer (the e4m3 quantiser) or by a transpose kernel, with the token axis padded to a
// multiple of 128 and zero-filled.
#include "api.h"
#include "attn.h"
#include "flash.h"
#include "gemm.h"
#include "norm.h"
#include "quant.h"

using namespace ll;

namespace {

struct Dims {
  int64_t B, T, N, Np, Tp, ve_rows;
  int D, Hq, Hkv, DH, F, FW, QD, KVD, QKVD, vcol0;   // FW: rows of w_fc (F, or 2F for SwiGLU)
  bool fp8, bf, ve, swiglu;
  int es;
  float eps, theta;
};

int make_dims(const ll_layer_cfg* c, Dims& d) {
  LL_CHECK(c, LL_ERR_INVALID_ARG, "cfg must not be null");
  LL_CHECK(c->dtype == LL_F32 || c->dtype == LL_BF16, LL_ERR_INVALID_ARG, "cfg.dtype must be LL_F32 or LL_BF16");
  LL_CHECK(c->batch >= 0 && c->seq >= 0, LL_ERR_INVALID_ARG, "batch and seq must be >= 0");
  LL_CHECK(c->d_model > 0 && c->n_q_heads > 0 && c->n_kv_heads > 0 && c->head_dim > 0 && c->d_ff > 0,
           LL_ERR_INVALID_ARG, "dimensions must be positive");
  LL_CHECK(c->n_q_heads % c->n_kv_heads == 0, LL_ERR_INVALID_ARG, "n_q_heads must be a multiple of n_kv_heads");
  LL_CHECK(!(c->fp8_mlp && c->dtype != LL_BF16), LL_ERR_UNSUPPORTED, "fp8_mlp requires LL_BF16");
  LL_CHECK(c->head_dim == (c->dtype == LL_BF16 ? 128 : 64), LL_ERR_UNSUPPORTED,
           "head_dim must be 128 (bf16) or 64 (fp32)");
  LL_CHECK(c->d_model % 128 == 0 && c->d_ff % 128 == 0 && c->d_model <= 4096, LL_ERR_UNSUPPORTED,
           "d_model and d_ff must be multiples of 128, d_model <= 4096");
  LL_CHECK((int64_t)c->n_q_heads * c->head_dim % 32 == 0, LL_ERR_UNSUPPORTED, "n_q_heads * head_dim % 32 != 0");
  LL_CHECK(c->rms_eps >= 0.f && c->rope_theta > 0.f, LL_ERR_INVALID_ARG, "rms_eps >= 0, rope_theta > 0");
  LL_CHECK(!c->has_value_embed || c->ve_rows > 0, LL_ERR_INVALID_ARG, "ve_rows must be > 0 on value-embedding layers");
  LL_CHECK(c->batch * c->seq < ((int64_t)1 << 31) / 64, LL_ERR_UNSUPPORTED, "too many tokens");
  LL_CHECK(c->mlp_kind == LL_MLP_RELU2 || c->mlp_kind == LL_MLP_SWIGLU, LL_ERR_INVALID_ARG,
           "mlp_kind must be LL_MLP_RELU2 or LL_MLP_SWIGLU");
  LL_CHECK(!(c->mlp_kind == LL_MLP_SWIGLU && c->fp8_mlp), LL_ERR_UNSUPPORTED,
           "the SwiGLU MLP runs on bf16 / fp32 GEMMs (fp8_mlp must be 0)");
  d.B = c->batch; d.T = c->seq; d.N = d.B * d.T;
  d.Np = round_up(d.N, 128); d.Tp = round_up(d.T, 64);
  d.D = c->d_model; d.Hq = c->n_q_heads; d.Hkv = c->n_kv_heads; d.DH = c->head_dim; d.F = c->d_ff;
  d.QD = d.Hq * d.DH; d.KVD = d.Hkv * d.DH; d.QKVD = d.QD + 2 * d.KVD; d.vcol0 = d.QD + d.KVD;
  d.fp8 = c->fp8_mlp != 0; d.bf = c->dtype == LL_BF16; d.ve = c->has_value_embed != 0;
  d.swiglu = c->mlp_kind == LL_MLP_SWIGLU; d.FW = d.swiglu ? 2 * d.F : d.F;
  d.es = d.bf ? 2 : 4; d.eps = c->rms_eps; d.theta = c->rope_theta;
  d.ve_rows = d.ve ? c->ve_rows : 0;
  return LL_OK;
}

// ---------------------------------------------------------------- saved (fwd -> bwd)
struct Saved {
  void *xn, *qkv, *qh, *kh, *o, *attn_out, *h, *u, *m, *hn, *r;
  float *r1, *r2, *rq, *rk, *lse;
  uint8_t *hn8, *hn8t, *r8t, *w18, *w18t, *w28, *w28t;
  QScale* qs;          // [4]: hn, w1, r, w2
};
enum { QS_HN = 0, QS_W1 = 1, QS_R = 2, QS_W2 = 3 };

size_t carve_saved(void* base, const Dims& d, Saved& s) {
  Carver c(base);
  const size_t e = d.es;
  s.qs = c.take<QScale>(4);
  s.xn = c.take<char>(d.N * d.D * e);
  s.r1 = c.take<float>(d.N);
  s.r2 = c.take<float>(d.N);
  s.qkv = c.take<char>(d.N * d.QKVD * e);
  s.qh = c.take<char>(d.N * d.QD * e);
  s.kh = c.take<char>(d.N * d.KVD * e);
  s.rq = c.take<float>(d.N * d.Hq);
  s.rk = c.take<float>(d.N * d.Hkv);
  s.o = c.take<char>(d.N * d.QD * e);
  s.lse = c.take<float>(d.B * d.Hq * d.Tp);     // [B, Hq, Tp] (bf16) / [B, Hq, T] (fp32)
  s.attn_out = c.take<char>(d.N * d.D * e);
  s.h = c.take<char>(d.N * d.D * e);
  s.u = c.take<char>(d.N * d.FW * e);      // u, or [g | u] for SwiGLU
  s.m = c.take<char>(d.N * d.D * e);
  s.hn = s.r = nullptr;
  s.hn8 = s.hn8t = s.r8t = s.w18 = s.w18t = s.w28 = s.w28t = nullptr;
  if (d.fp8) {
    s.hn8 = c.take<uint8_t>(d.N * d.D);
    s.hn8t = c.take<uint8_t>((int64_t)d.D * d.Np);
    s.r8t = c.take<uint8_t>((int64_t)d.F * d.Np);
    s.w18 = c.take<uint8_t>((int64_t)d.F * d.D);
    s.w18t = c.take<uint8_t>((int64_t)d.D * d.F);
    s.w28 = c.take<uint8_t>((int64_t)d.D * d.F);
    s.w28t = c.take<uint8_t>((int64_t)d.F * d.D);
  } else {
    s.hn = c.take<char>(d.N * d.D * e);
    s.r = c.take<char>(d.N * d.F * e);    // r = relu(u)^2, or a = silu(g) u for SwiGLU
  }
  return c.bytes();
}

// ---------------------------------------------------------------- forward workspace
struct FwdWs {
  float2* cs;
  void *vt, *hn;
  uint8_t* r8;
};
size_t carve_fwd(void* base, const Dims& d, FwdWs& w) {
  Carver c(base);
  w.cs = c.take<float2>(d.T * (d.DH / 2) + 1);
  w.vt = d.bf ? nullptr : c.take<char>(d.B * d.KVD * d.Tp * d.es);   // fp32 kernels read V^T
  w.hn = nullptr;
  w.r8 = nullptr;
  if (d.fp8) {
    w.hn = c.take<char>(d.N * d.D * d.es);
    w.r8 = c.take<uint8_t>(d.N * d.F);
  }
  return c.bytes();
}

// ---------------------------------------------------------------- backward workspace
struct BwdWs {
  float2* cs;
  float* sk;             // fp32 partial sums of the weight gradients split along the tokens
  size_t sk_bytes;
  QScale* qs;            // [2]: dm, du
  void *dm, *du, *dhn, *dh, *dattn, *dout, *qt, *kt, *dot, *dqkv, *dxn;
  void *t0, *t1;         // transposed operand copies: W^T for mm_nn (both types), mm_tn's (fp32 only)
  const void* zrow;      // 256 zero bytes: K-tail rows of MN-major GEMM operands
  uint8_t *dm8, *dm8t, *du8, *du8t;
  float *delta, *dqh, *dkh, *dgp;
};
// Floats of split-K partial sums the backward needs: the largest slices x M x N over the weight
// gradients that split (the bf16 O-projection and QKV weight gradients; the FP8 MLP weight
// gradients run unsplit beside another GEMM), with the slice counts the launches will pick.
int64_t splitk_floats(const Dims& d) {
  int64_t f = 0;
  auto need = [&](int M, int N, int64_t K, int ke) {
    const int sl = splitk_slices(cdiv(M, 256) * cdiv(N, 256), K, ke, 8);
    if (sl > 1) f = std::max<int64_t>(f, (int64_t)sl * M * N);
  };
  if (d.bf) {
    need(d.D, d.QD, d.N, 64);
    need(d.QKVD, d.D, d.N, 64);
  }
  return f;
}

size_t carve_bwd(void* base, const Dims& d, BwdWs& w) {
  Carver c(base);
  const size_t e = d.es;
  w.cs = c.take<float2>(d.T * (d.DH / 2) + 1);
  w.sk_bytes = (size_t)splitk_floats(d) * sizeof(float);
  w.sk = w.sk_bytes ? c.take<float>(w.sk_bytes / sizeof(float)) : nullptr;
  w.qs = c.take<QScale>(2);
  w.zrow = c.take<char>(256);
  w.dm = c.take<char>(d.N * d.D * e);
  w.du = c.take<char>(d.N * d.FW * e);     // du, or [dg | du] for SwiGLU
  w.dhn = c.take<char>(d.N * d.D * e);
  w.dh = c.take<char>(d.N * d.D * e);
  w.dattn = c.take<char>(d.N * d.D * e);
  w.dout = c.take<char>(d.N * d.QD * e);
  w.qt = w.kt = w.dot = nullptr;
  if (!d.bf) {   // fp32 kernels read Q^T, K^T, dO^T
    w.qt = c.take<char>(d.B * d.QD * d.Tp * e);
    w.kt = c.take<char>(d.B * d.KVD * d.Tp * e);
    w.dot = c.take<char>(d.B * d.QD * d.Tp * e);
  }
  w.delta = c.take<float>(d.B * d.Hq * d.Tp);
  w.dqh = w.dkh = nullptr;
  if (!d.bf) {   // fp32 kernels leave dq^, dk^ for qk_post
    w.dqh = c.take<float>(d.N * d.QD);
    w.dkh = c.take<float>(d.N * d.KVD);
  }
  w.dqkv = c.take<char>(d.N * d.QKVD * e);
  w.dxn = c.take<char>(d.N * d.D * e);
  w.dgp = c.take<float>(rmsnorm_bwd_partials(d.N) * d.D + colsum_scratch_floats(d.D) + 1);
  w.t0 = w.t1 = nullptr;
  w.dm8 = w.dm8t = w.du8 = w.du8t = nullptr;
  if (!d.bf) {
    const int64_t big = std::max<int64_t>({(int64_t)d.QKVD, (int64_t)d.FW, (int64_t)d.D, (int64_t)d.QD});
    const int64_t t = std::max<int64_t>(big * d.Np, big * big);
    w.t0 = c.take<char>(t * e);
    w.t1 = c.take<char>(t * e);
  } else {
    // transposed weight of an input-gradient GEMM
    w.t0 = c.take<char>(std::max<int64_t>({(int64_t)d.QKVD * d.D, (int64_t)d.FW * d.D, (int64_t)d.QD * d.D}) * e);
  }
  if (d.fp8) {
    w.dm8 = c.take<uint8_t>(d.N * d.D);
    w.dm8t = c.take<uint8_t>((int64_t)d.D * d.Np);
    w.du8 = c.take<uint8_t>(d.N * d.F);
    w.du8t = c.take<uint8_t>((int64_t)d.F * d.Np);
  }
  return c.bytes();
}

template <class T> T* P(void* p) { return static_cast<T*>(p); }
template <class T> const T* CP(const void* p) { return static_cast<const T*>(p); }

int check_ptrs(std::initializer_list<const void*> ps, const char* what) {
  for (const void* p : ps) {
    LL_CHECK(p, LL_ERR_INVALID_ARG, std::string(what) + ": null pointer");
    LL_CHECK(aligned16(p), LL_ERR_INVALID_ARG, std::string(what) + ": pointer not 16-byte aligned");
  }
  return LL_OK;
}

hipError_t rope_table(float2* cs, const Dims& d, hipStream_t s) {
  const int64_t n = d.T * (d.DH / 2);
  if (n <= 0) return hipSuccess;
  LL_LAUNCH("rope_table", rope_table_kernel, dim3((unsigned)std::min<int64_t>(cdiv(n, 256), 4096)), dim3(256), 0, s, cs,
                     (int)d.T, d.DH / 2, (double)d.theta);
  return hipGetLastError();
}

// Backward GEMMs whose operands are not both K-major.
//   mm_nn: C = A W with A [M, K] K-major and W [K, N] row-major (the input-gradient GEMMs): W is
//          transposed first.
//   mm_tn: C = X^T Y with X [K, M], Y [K, N] row-major, K = tokens (the weight-gradient GEMMs).
//          bf16 reads X and Y in place (MN-major, LDS transpose reads); fp32 goes through
//          transposed copies (token axis padded with zeros to Kp). With a scratch buffer (sk,
//          sk_bytes) a bf16 GEMM with too few output tiles for the chip is split along the tokens.
template <class T, class Epi>
hipError_t mm_nn(const T* A, int64_t lda, const T* W, int64_t ldw, int M, int N, int K, const Epi& e, T* wT,
                 const void* zrow, hipStream_t s) {
  // W^T first (a weight: tens of MB, microseconds), then a GEMM with both operands K-major, which
  // runs ~20% faster than reading W through LDS transpose reads
  (void)zrow;
  hipError_t r = transpose2d(W, (int64_t)K, N, ldw, wT, (int64_t)K, (int64_t)K, s);
  if (r != hipSuccess) return r;
  return launch_gemm(A, lda, static_cast<const T*>(wT), (int64_t)K, M, N, K, e, GemmOps{}, s);
}
template <class T, class Epi>
hipError_t mm_tn(const T* X, int64_t ldx, const T* Y, int64_t ldy, int M, int N, int64_t K, int64_t Kp, const Epi& e,
                 T* xT, T* yT, const void* zrow, hipStream_t s, float* sk = nullptr, size_t sk_bytes = 0) {
  if constexpr (std::is_same<T, bf16>::value) {
    const GemmOps ops{false, false, zrow};
    if constexpr (std::is_same<Epi, EpiStore<T>>::value) {
      const int sl = splitk_slices(cdiv(M, 256) * cdiv(N, 256), K, 64, 8);
      if (sl > 1 && sk && !e.dq.ia && (size_t)sl * M * N * sizeof(float) <= sk_bytes && gemm_config_override() == 0)
        return launch_gemm_splitk(X, ldx, Y, ldy, M, N, (int)K, sl, e.C, e.ldc, sk, ops, s, Deq{nullptr, nullptr},
                                  e.accumulate);
    }
    return launch_gemm(X, ldx, Y, ldy, M, N, (int)K, e, ops, s);
  } else {
    hipError_t r = transpose2d(X, K, M, ldx, xT, Kp, Kp, s);
    if (r == hipSuccess) r = transpose2d(Y, K, N, ldy, yT, Kp, Kp, s);
    if (r != hipSuccess) return r;
    return launch_gemm_nt(static_cast<const T*>(xT), Kp, static_cast<const T*>(yT), Kp, M, N, (int)Kp, e, s);
  }
}

// ------------------------------------------------------------------------------------------ fwd
template <class T, int DH>
int layer_fwd_t(const Dims& d, const ll_layer_params* p, const T* x, const int32_t* ids, T* y, const Saved& sv,
                const FwdWs& w, hipStream_t s) {
  const int64_t N = d.N;
  const float* g1 = CP<float>(p->attn_norm_w);
  const float* g2 = CP<float>(p->mlp_norm_w);
  LL_HIP(rope_table(w.cs, d, s));
  LL_HIP(fill_f32(reinterpret_cast<float*>(sv.qs), 0.f, 4 * 4, s));
  // attention block
  LL_HIP(launch_rmsnorm_fwd(x, g1, P<T>(sv.xn), sv.r1, N, d.D, d.eps, (float*)nullptr, s));
  {
    // QK-norm + RoPE on the bf16 path: k^ (shared by every query block of its group) and 1/rms(k)
    // leave the QKV GEMM's epilogue; the attention forward applies them to q as it loads it (and
    // saves q^ and 1/rms(q) for the backward)
    constexpr bool kFused = std::is_same<T, bf16>::value;
    EpiQkv<T> e{P<T>(sv.qkv), d.QKVD, d.ve ? CP<T>(p->ve_table) : nullptr, d.KVD, ids, d.vcol0, d.ve_rows};
    if (kFused) {
      e.kh = P<T>(sv.kh);
      e.rk = sv.rk;
      e.cs = w.cs;
      e.kcol0 = d.QD;
      e.seq = (int)d.T;
      e.eps = d.eps;
    }
    LL_HIP(launch_gemm_nt(CP<T>(sv.xn), d.D, CP<T>(p->w_qkv), d.D, (int)N, d.QKVD, d.D, e, s));
  }
  if (N > 0) {
    if constexpr (!std::is_same<T, bf16>::value) {
      // the fp32 kernels take q^ and k^ from this pass
      const int hp = d.Hq + d.Hkv;
      const int64_t threads = N * hp * (DH / 16);   // 8 rotation pairs per lane
      LL_LAUNCH("qk_prep", (qk_prep_kernel<T, DH>), dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, s,
                CP<T>(sv.qkv), (int64_t)d.QKVD, w.cs, P<T>(sv.qh), P<T>(sv.kh), sv.rq, sv.rk, N, (int)d.T, d.Hq,
                d.Hkv, d.eps, 0, hp);
      LL_HIP(hipGetLastError());
    }
    const int nqb = (int)cdiv(d.T, 128);
    // algorithmic work, traced as 2 M N K: causal (query, key) pairs x head_dim x 2 products
    const int64_t pairs = d.B * d.Hq * d.T * (d.T + 1) / 2;
    if constexpr (std::is_same<T, bf16>::value) {
      LL_LAUNCH_MNK("attn_fwd", pairs, DH, 2, (fa_fwd_kernel<true>), dim3((unsigned)(d.B * d.Hq * nqb)), dim3(256), 0, s,
                    CP<T>(sv.qkv), (int64_t)d.QKVD, w.cs, d.eps, P<T>(sv.qh), sv.rq, CP<T>(sv.kh),
                    CP<T>(sv.qkv) + d.vcol0, (int64_t)d.QKVD, P<T>(sv.o), sv.lse, d.Tp, (int)d.B, (int)d.T, d.Hq,
                    d.Hkv);
    } else {
      LL_HIP(launch_transpose(CP<T>(sv.qkv) + d.vcol0, d.T, DH, (int64_t)d.QKVD, P<T>(w.vt), d.Tp, d.Tp,
                              (int)(d.B * d.Hkv), d.Hkv, d.T * d.QKVD, (int64_t)DH, (int64_t)DH * d.Tp, s));
      LL_LAUNCH_MNK("attn_fwd", pairs, DH, 2, (attn_fwd_kernel<T, DH>), dim3((unsigned)(d.B * d.Hq * nqb)), dim3(256),
                    0, s, CP<T>(sv.qh), CP<T>(sv.kh), CP<T>(w.vt), P<T>(sv.o), sv.lse, (int)d.B, (int)d.T, (int)d.Tp, d.Hq,
                d.Hkv);
    }
    LL_HIP(hipGetLastError());
  }
  {
    EpiResidual<T> e{P<T>(sv.h), x, P<T>(sv.attn_out), (int64_t)d.D, p->resid_attn, Deq{nullptr, nullptr}};
    LL_HIP(launch_gemm_nt(CP<T>(sv.o), d.QD, CP<T>(p->w_o), d.QD, (int)N, d.D, d.QD, e, s));
  }
  // MLP block
  if constexpr (std::is_same<T, bf16>::value) {
    if (d.fp8) {
      QScale* q = sv.qs;
      LL_HIP(launch_rmsnorm_fwd(CP<T>(sv.h), g2, P<T>(w.hn), sv.r2, N, d.D, d.eps, &q[QS_HN].amax, s));
      LL_HIP(launch_amax(CP<T>(p->w_fc), d.F, d.D, d.D, &q[QS_W1].amax, s));
      LL_HIP(launch_amax(CP<T>(p->w_proj), d.D, d.F, d.F, &q[QS_W2].amax, s));
      LL_HIP(launch_cast_e4m3(CP<T>(p->w_fc), d.F, d.D, d.D, &q[QS_W1], sv.w18, d.D, sv.w18t, d.F, d.F,
                              (float*)nullptr, (float*)nullptr, s));
      LL_HIP(launch_cast_e4m3(CP<T>(p->w_proj), d.D, d.F, d.F, &q[QS_W2], sv.w28, d.F, sv.w28t, d.D, d.D,
                              (float*)nullptr, (float*)nullptr, s));
      LL_HIP(launch_cast_e4m3(CP<T>(w.hn), N, d.D, d.D, &q[QS_HN], sv.hn8, d.D, sv.hn8t, d.Np, d.Np,
                              (float*)nullptr, (float*)nullptr, s));
      {
        // u is stored; r = relu(u)^2 only reaches HBM as e4m3 codes (the cast forms r from u)
        EpiRelu2Amax<T> e{P<T>(sv.u), (int64_t)d.F, Deq{&q[QS_HN].inv_scale, &q[QS_W1].inv_scale}, &q[QS_R].amax};
        LL_HIP(launch_gemm_nt(sv.hn8, d.D, sv.w18, d.D, (int)N, d.F, d.D, e, s));
      }
      LL_HIP((launch_cast_e4m3<T, true>(CP<T>(sv.u), N, d.F, d.F, &q[QS_R], w.r8, d.F, sv.r8t, d.Np, d.Np,
                                        (float*)nullptr, (float*)nullptr, s)));
      {
        EpiResidual<T> e{y, CP<T>(sv.h), P<T>(sv.m), (int64_t)d.D, p->resid_mlp,
                         Deq{&q[QS_R].inv_scale, &q[QS_W2].inv_scale}};
        LL_HIP(launch_gemm_nt(w.r8, d.F, sv.w28, d.F, (int)N, d.D, d.F, e, s));
      }
      return LL_OK;
    }
  }
  LL_HIP(launch_rmsnorm_fwd(CP<T>(sv.h), g2, P<T>(sv.hn), sv.r2, N, d.D, d.eps, (float*)nullptr, s));
  if (d.swiglu) {
    // g = hn W_gate^T into the first F columns of [g | u], then the up GEMM whose epilogue stores
    // u beside it and a = silu(g) u
    EpiStore<T> eg{P<T>(sv.u), (int64_t)d.FW, Deq{nullptr, nullptr}};
    LL_HIP(launch_gemm_nt(CP<T>(sv.hn), d.D, CP<T>(p->w_fc), d.D, (int)N, d.F, d.D, eg, s));
    EpiSwigluUp<T> eu{P<T>(sv.u), (int64_t)d.FW, d.F, P<T>(sv.r), (int64_t)d.F};
    LL_HIP(launch_gemm_nt(CP<T>(sv.hn), d.D, CP<T>(p->w_fc) + (int64_t)d.F * d.D, d.D, (int)N, d.F, d.D, eu, s));
  } else {
    EpiRelu2<T> e{P<T>(sv.u), P<T>(sv.r), (int64_t)d.F, Deq{nullptr, nullptr}, &sv.qs[QS_R].amax};
    LL_HIP(launch_gemm_nt(CP<T>(sv.hn), d.D, CP<T>(p->w_fc), d.D, (int)N, d.F, d.D, e, s));
  }
  {
    EpiResidual<T> e{y, CP<T>(sv.h), P<T>(sv.m), (int64_t)d.D, p->resid_mlp, Deq{nullptr, nullptr}};
    LL_HIP(launch_gemm_nt(CP<T>(sv.r), d.F, CP<T>(p->w_proj), d.F, (int)N, d.D, d.F, e, s));
  }
  return LL_OK;
}

// FP8 weight gradient C [M, N] = deq(X Y^T) over the token axis (both operands the quantiser's
// transposed codes, K-major, Np tokens), as its own launch: the path of a GEMM-configuration
// override that the two-GEMM grids below do not run.
template <class T>
hipError_t wgrad_e4m3(const uint8_t* X, const uint8_t* Y, int64_t Np, int M, int N, T* C, Deq dq, int accumulate,
                      hipStream_t s) {
  EpiStore<T> e{C, (int64_t)N, dq, accumulate};
  return launch_gemm_nt(X, Np, Y, Np, M, N, (int)Np, e, s);
}

// The FP8 MLP backward's GEMMs as two grids: each weight gradient (K = the Np tokens, unsplit) with
// the input-side GEMM of the same step, the weight gradient's long tiles first
template <class E0, class E1> struct EpiWgradRelu2Bwd : EpiPairOf<E0, E1> {
  static constexpr const char* kName = "wgrad_relu2_bwd";
};
template <class E0, class E1> struct EpiWgradDgrad : EpiPairOf<E0, E1> {
  static constexpr const char* kName = "wgrad_dgrad";
};
template <class Pair, class E0, class E1>
hipError_t wgrad_pair_e4m3(const uint8_t* X, const uint8_t* Y, int64_t Np, int M, int N, const E0& ew,
                           const uint8_t* A1, const uint8_t* B1, int64_t K1, int M1, int N1, const E1& e1,
                           hipStream_t s) {
  Pair e{};
  e.e0 = ew;
  e.e1 = e1;
  e.a1 = A1;
  e.lda1 = K1;
  e.b1 = B1;
  e.ldb1 = K1;
  e.m1 = M1;
  e.n1 = N1;
  e.k1 = (int)K1;
  e.g1 = 2;
  return launch_gemm_pair(X, Np, Y, Np, M, N, (int)Np, 2, e, s);
}

// ------------------------------------------------------------------------------------------ bwd
template <class T, int DH>
int layer_bwd_t(const Dims& d, const ll_layer_params* p, const T* x, const int32_t* ids, const Saved& sv,
                const T* dy, T* dx, const ll_layer_grads* g, const BwdWs& w, hipStream_t s) {
  const int64_t N = d.N, Np = d.Np;
  const float* g1 = CP<float>(p->attn_norm_w);
  const float* g2 = CP<float>(p->mlp_norm_w);
  LL_HIP(rope_table(w.cs, d, s));
  LL_HIP(fill_f32(reinterpret_cast<float*>(w.qs), 0.f, 2 * 4, s));
  LL_HIP(fill_f32(reinterpret_cast<float*>(const_cast<void*>(w.zrow)), 0.f, 64, s));
  const int acc = g->accumulate ? 1 : 0;
  if (!acc) {   // the residual-scalar gradients are atomic sums: start from 0 unless accumulating
    LL_HIP(fill_f32(g->resid_mlp, 0.f, 1, s));
    LL_HIP(fill_f32(g->resid_attn, 0.f, 1, s));
  }
  // MLP residual branch: dm = a_mlp dy, da_mlp = sum dy m
  LL_HIP(launch_scale_dot(dy, CP<T>(sv.m), p->resid_mlp, P<T>(w.dm), N * d.D, g->resid_mlp,
                          d.fp8 ? &w.qs[0].amax : nullptr, s));
  bool done = false;
  if constexpr (std::is_same<T, bf16>::value) {
    if (d.fp8) {
      QScale* q = sv.qs;
      QScale* qdm = &w.qs[0];
      QScale* qdu = &w.qs[1];
      LL_HIP(launch_cast_e4m3(CP<T>(w.dm), N, d.D, d.D, qdm, w.dm8, d.D, w.dm8t, Np, Np, (float*)nullptr,
                              (float*)nullptr, s));
      // dr = dm W2 (W2^T quantised is [F, D]); du = dr * 2 relu(u)
      const EpiRelu2Bwd<T> erb{P<T>(w.du), CP<T>(sv.u), (int64_t)d.F, Deq{&qdm->inv_scale, &q[QS_W2].inv_scale},
                               &qdu->amax};
      // dW2 = dm^T r   [D, F]
      const EpiStore<T> ew2{P<T>(g->w_proj), (int64_t)d.F, Deq{&qdm->inv_scale, &q[QS_R].inv_scale}, acc};
      // dW1 = du^T hn  [F, D]
      const EpiStore<T> ew1{P<T>(g->w_fc), (int64_t)d.D, Deq{&qdu->inv_scale, &q[QS_HN].inv_scale}, acc};
      // dhn = du W1 (W1^T quantised is [D, F])
      const EpiStore<T> edh{P<T>(w.dhn), (int64_t)d.D, Deq{&qdu->inv_scale, &q[QS_W1].inv_scale}};
      if (gemm_pair_ok<uint8_t>(Np, Np, d.D, d.F)) {
        LL_HIP((wgrad_pair_e4m3<EpiWgradRelu2Bwd<EpiStore<T>, EpiRelu2Bwd<T>>>(
            w.dm8t, sv.r8t, Np, d.D, d.F, ew2, w.dm8, sv.w28t, d.D, (int)N, d.F, erb, s)));
        LL_HIP(launch_cast_e4m3(CP<T>(w.du), N, d.F, d.F, qdu, w.du8, d.F, w.du8t, Np, Np, (float*)nullptr,
                                (float*)nullptr, s));
        LL_HIP((wgrad_pair_e4m3<EpiWgradDgrad<EpiStore<T>, EpiStore<T>>>(
            w.du8t, sv.hn8t, Np, d.F, d.D, ew1, w.du8, sv.w18t, d.F, (int)N, d.D, edh, s)));
      } else {
        LL_HIP(launch_gemm_nt(w.dm8, d.D, sv.w28t, d.D, (int)N, d.F, d.D, erb, s));
        LL_HIP(launch_cast_e4m3(CP<T>(w.du), N, d.F, d.F, qdu, w.du8, d.F, w.du8t, Np, Np, (float*)nullptr,
                                (float*)nullptr, s));
        LL_HIP(wgrad_e4m3(w.dm8t, sv.r8t, Np, d.D, d.F, ew2.C, ew2.dq, acc, s));
        LL_HIP(wgrad_e4m3(w.du8t, sv.hn8t, Np, d.F, d.D, ew1.C, ew1.dq, acc, s));
        LL_HIP(launch_gemm_nt(w.du8, d.F, sv.w18t, d.F, (int)N, d.D, d.F, edh, s));
      }
      done = true;
    }
  }
  if (!done) {
    if (d.swiglu) {   // da = dm W2; [dg | du] from da, g and u in the epilogue
      EpiSwigluBwd<T> e{P<T>(w.du), CP<T>(sv.u), (int64_t)d.FW, d.F};
      LL_HIP(mm_nn(CP<T>(w.dm), d.D, CP<T>(p->w_proj), d.F, (int)N, d.F, d.D, e, P<T>(w.t0), w.zrow, s));
    } else {   // dr = dm W2; du = dr * 2 relu(u)
      EpiRelu2Bwd<T> e{P<T>(w.du), CP<T>(sv.u), (int64_t)d.F, Deq{nullptr, nullptr}, &w.qs[1].amax};
      LL_HIP(mm_nn(CP<T>(w.dm), d.D, CP<T>(p->w_proj), d.F, (int)N, d.F, d.D, e, P<T>(w.t0), w.zrow, s));
    }
    {   // dW2 = dm^T r
      EpiStore<T> e{P<T>(g->w_proj), (int64_t)d.F, Deq{nullptr, nullptr}, acc};
      LL_HIP(mm_tn(CP<T>(w.dm), d.D, CP<T>(sv.r), d.F, d.D, d.F, N, Np, e, P<T>(w.t0), P<T>(w.t1), w.zrow, s));
    }
    {   // dW1 = du^T hn  ([dg | du]^T hn for SwiGLU)
      EpiStore<T> e{P<T>(g->w_fc), (int64_t)d.D, Deq{nullptr, nullptr}, acc};
      LL_HIP(mm_tn(CP<T>(w.du), d.FW, CP<T>(sv.hn), d.D, d.FW, d.D, N, Np, e, P<T>(w.t0), P<T>(w.t1), w.zrow, s));
    }
    {   // dhn = du W1
      EpiStore<T> e{P<T>(w.dhn), (int64_t)d.D, Deq{nullptr, nullptr}};
      LL_HIP(mm_nn(CP<T>(w.du), d.FW, CP<T>(p->w_fc), d.D, (int)N, d.D, d.FW, e, P<T>(w.t0), w.zrow, s));
    }
  }
  // MLP RMSNorm backward + residual, fused with the attention-branch scaling
  LL_HIP(launch_rmsnorm_bwd(CP<T>(w.dhn), CP<T>(sv.h), g2, sv.r2, dy, P<T>(w.dh), w.dgp, N, d.D, p->resid_attn,
                            P<T>(w.dattn), CP<T>(sv.attn_out), g->resid_attn, s));
  LL_HIP(launch_colsum(w.dgp, rmsnorm_bwd_partials(N), d.D, P<float>(g->mlp_norm_w),
                       w.dgp + rmsnorm_bwd_partials(N) * d.D, s, acc));
  // O projection: do = dattn W_o, dW_o = dattn^T o
  {
    EpiStore<T> e{P<T>(w.dout), (int64_t)d.QD, Deq{nullptr, nullptr}};
    LL_HIP(mm_nn(CP<T>(w.dattn), d.D, CP<T>(p->w_o), d.QD, (int)N, d.QD, d.D, e, P<T>(w.t0), w.zrow, s));
  }
  {
    EpiStore<T> e{P<T>(g->w_o), (int64_t)d.QD, Deq{nullptr, nullptr}, acc};
    LL_HIP(mm_tn(CP<T>(w.dattn), d.D, CP<T>(sv.o), d.QD, d.D, d.QD, N, Np, e, P<T>(w.t0), P<T>(w.t1), w.zrow, s,
                 w.sk, w.sk_bytes));
  }
  // attention core
  T* dqkv = P<T>(w.dqkv);
  if (N > 0) {
    const int64_t dthreads = N * d.Hq * (DH / 8);   // 8 elements per lane
    const int64_t ldl = d.bf ? d.Tp : d.T;   // row stride of lse and delta
    // algorithmic work, traced as 2 M N K: dK/dV holds the dP, dV and dK products, dQ the dQ product
    const int64_t pairs = d.B * d.Hq * d.T * (d.T + 1) / 2;
    if constexpr (std::is_same<T, bf16>::value) {
      // dQ first: it forms Delta = rowsum(dO * O) from the rows it holds and leaves it for dK/dV
      const int nb128 = (int)cdiv(d.T, 128);
      LL_LAUNCH_MNK("attn_bwd_dq", pairs, DH, 1, fa_dq_kernel, dim3((unsigned)(d.B * d.Hq * nb128)), dim3(256), 0, s, CP<T>(sv.qh),
                CP<T>(sv.kh), CP<T>(sv.qkv) + d.vcol0, (int64_t)d.QKVD, CP<T>(w.dout), CP<T>(sv.o), sv.lse, w.delta,
                ldl, CP<T>(sv.qkv), w.cs, sv.rq, dqkv, (int)d.B, (int)d.T, d.Hq, d.Hkv);
      LL_HIP(hipGetLastError());
      // 16 keys per wave: 8 waves, two per SIMD, so one wave's softmax and LDS reads overlap the
      // other's MFMAs
      constexpr int kKpw = 16;
      LL_LAUNCH_MNK("attn_bwd_dkdv", pairs, DH, 3, fa_dkdv_kernel<kKpw>, dim3((unsigned)(d.B * d.Hkv * nb128)),
                dim3(64 * (128 / kKpw)), 0, s,
                CP<T>(sv.qh), CP<T>(sv.kh), CP<T>(sv.qkv) + d.vcol0, (int64_t)d.QKVD, CP<T>(w.dout), sv.lse,
                w.delta, ldl, CP<T>(sv.qkv) + d.QD, w.cs, sv.rk, dqkv + d.QD, dqkv + d.vcol0, (int64_t)d.QKVD,
                (int)d.B, (int)d.T, d.Hq, d.Hkv);
      LL_HIP(hipGetLastError());
    } else {
      LL_LAUNCH("attn_delta", (attn_delta_kernel<T, DH>), dim3((unsigned)cdiv(dthreads, 256)), dim3(256), 0, s,
                CP<T>(w.dout), CP<T>(sv.o), w.delta, ldl, N, (int)d.T, d.Hq);
      LL_HIP(hipGetLastError());
      LL_HIP(launch_transpose(CP<T>(sv.qh), d.T, DH, (int64_t)d.QD, P<T>(w.qt), d.Tp, d.Tp, (int)(d.B * d.Hq), d.Hq,
                              d.T * d.QD, (int64_t)DH, (int64_t)DH * d.Tp, s));
      LL_HIP(launch_transpose(CP<T>(sv.kh), d.T, DH, (int64_t)d.KVD, P<T>(w.kt), d.Tp, d.Tp, (int)(d.B * d.Hkv),
                              d.Hkv, d.T * d.KVD, (int64_t)DH, (int64_t)DH * d.Tp, s));
      LL_HIP(launch_transpose(CP<T>(w.dout), d.T, DH, (int64_t)d.QD, P<T>(w.dot), d.Tp, d.Tp, (int)(d.B * d.Hq),
                              d.Hq, d.T * d.QD, (int64_t)DH, (int64_t)DH * d.Tp, s));
      const int nkb = (int)cdiv(d.T, 64);
      LL_LAUNCH_MNK("attn_bwd_dkdv", pairs, DH, 3, (attn_bwd_dkdv_kernel<T, DH>), dim3((unsigned)(d.B * d.Hkv * nkb)), dim3(256), 0, s,
                CP<T>(sv.qh), CP<T>(sv.kh), CP<T>(sv.qkv) + d.vcol0, (int64_t)d.QKVD, CP<T>(w.dout), CP<T>(w.qt),
                CP<T>(w.dot), sv.lse, w.delta, w.dkh, dqkv + d.vcol0, (int64_t)d.QKVD, (int)d.B, (int)d.T,
                (int)d.Tp, d.Hq, d.Hkv);
      LL_HIP(hipGetLastError());
      LL_LAUNCH_MNK("attn_bwd_dq", pairs, DH, 1, (attn_bwd_dq_kernel<T, DH>), dim3((unsigned)(d.B * d.Hq * nkb)), dim3(256), 0, s,
                CP<T>(sv.qh), CP<T>(sv.kh), CP<T>(sv.qkv) + d.vcol0, (int64_t)d.QKVD, CP<T>(w.dout), CP<T>(w.kt),
                sv.lse, w.delta, w.dqh, (int)d.B, (int)d.T, (int)d.Tp, d.Hq, d.Hkv);
      LL_HIP(hipGetLastError());
      // the fp32 kernels leave dq^, dk^ in fp32 (the bf16 ones apply the norm and RoPE backward in
      // their epilogues)
      const int64_t pthreads = N * (d.Hq + d.Hkv) * (DH / 16);
      LL_LAUNCH("qk_post", (qk_post_kernel<T, DH>), dim3((unsigned)cdiv(pthreads, 256)), dim3(256), 0, s, w.dqh,
                w.dkh, CP<T>(sv.qkv), (int64_t)d.QKVD, w.cs, sv.rq, sv.rk, dqkv, N, (int)d.T, d.Hq, d.Hkv);
      LL_HIP(hipGetLastError());
    }
    if (d.ve) {
      const int64_t tot = N * d.KVD;
      if (!acc) LL_HIP(fill_f32(g->ve_table, 0.f, d.ve_rows * d.KVD, s));   // overwrite: scatter-add from zero
      LL_LAUNCH("ve_scatter", (ve_scatter_kernel<T>), dim3((unsigned)std::min<int64_t>(cdiv(tot, 256), 16384)), dim3(256),
                         0, s, CP<T>(dqkv) + d.vcol0, (int64_t)d.QKVD, ids, g->ve_table, (int64_t)d.KVD, d.ve_rows, N, d.KVD);
      LL_HIP(hipGetLastError());
    }
  }
  // QKV projection: dxn = dqkv W_qkv, dW_qkv = dqkv^T xn
  {
    EpiStore<T> e{P<T>(w.dxn), (int64_t)d.D, Deq{nullptr, nullptr}};
    LL_HIP(mm_nn(CP<T>(dqkv), d.QKVD, CP<T>(p->w_qkv), d.D, (int)N, d.D, d.QKVD, e, P<T>(w.t0), w.zrow, s));
  }
  {
    EpiStore<T> e{P<T>(g->w_qkv), (int64_t)d.D, Deq{nullptr, nullptr}, acc};
    LL_HIP(mm_tn(CP<T>(dqkv), d.QKVD, CP<T>(sv.xn), d.D, d.QKVD, d.D, N, Np, e, P<T>(w.t0), P<T>(w.t1), w.zrow, s,
                 w.sk, w.sk_bytes));
  }
  // input RMSNorm backward + residual
  LL_HIP(launch_rmsnorm_bwd(CP<T>(w.dxn), x, g1, sv.r1, CP<T>(w.dh), dx, w.dgp, N, d.D, (const float*)nullptr,
                            (T*)nullptr, (const T*)nullptr, (float*)nullptr, s));
  LL_HIP(launch_colsum(w.dgp, rmsnorm_bwd_partials(N), d.D, P<float>(g->attn_norm_w),
                       w.dgp + rmsnorm_bwd_partials(N) * d.D, s, acc));
  return LL_OK;
}

}  // namespace

extern "C" size_t ll_layer_saved_bytes(const ll_layer_cfg* cfg) {
  Dims d;
  if (make_dims(cfg, d) != LL_OK) return 0;
  Saved s;
  return carve_saved(nullptr, d, s);
}

extern "C" size_t ll_layer_workspace_bytes(const ll_layer_cfg* cfg) {
  Dims d;
  if (make_dims(cfg, d) != LL_OK) return 0;
  FwdWs f;
  BwdWs b;
  return std::max(carve_fwd(nullptr, d, f), carve_bwd(nullptr, d, b));
}

extern "C" int ll_layer_fwd(const ll_layer_cfg* cfg, const ll_layer_params* p, const void* x, const int32_t* token_ids,
                            void* y, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  if (int st = make_dims(cfg, d)) return st;
  LL_CHECK(p, LL_ERR_INVALID_ARG, "params must not be null");
  if (int st = check_ptrs({p->attn_norm_w, p->w_qkv, p->w_o, p->mlp_norm_w, p->w_fc, p->w_proj, p->resid_attn,
                           p->resid_mlp}, "params")) return st;
  if (d.ve) {
    if (int st = check_ptrs({p->ve_table}, "params.ve_table")) return st;
    LL_CHECK(d.N == 0 || token_ids, LL_ERR_INVALID_ARG, "token_ids required on value-embedding layers");
  }
  if (d.N > 0) {
    if (int st = check_ptrs({x, y}, "x/y")) return st;
    LL_CHECK(x != y, LL_ERR_INVALID_ARG, "y must not alias x");
  }
  Saved sv;
  FwdWs w;
  const size_t need_s = carve_saved(nullptr, d, sv), need_w = carve_fwd(nullptr, d, w);
  LL_CHECK(saved && aligned16(saved), LL_ERR_INVALID_ARG, "saved must be a 16-byte aligned device pointer");
  LL_CHECK(ws && aligned16(ws), LL_ERR_INVALID_ARG, "ws must be a 16-byte aligned device pointer");
  LL_CHECK(saved_bytes >= need_s, LL_ERR_WORKSPACE, "saved buffer too small: need " + std::to_string(need_s));
  LL_CHECK(ws_bytes >= need_w, LL_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_w));
  carve_saved(saved, d, sv);
  carve_fwd(ws, d, w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.bf) return layer_fwd_t<bf16, 128>(d, p, CP<bf16>(x), token_ids, P<bf16>(y), sv, w, s);
  return layer_fwd_t<float, 64>(d, p, CP<float>(x), token_ids, P<float>(y), sv, w, s);
}

extern "C" int ll_layer_bwd(const ll_layer_cfg* cfg, const ll_layer_params* p, const void* x, const int32_t* token_ids,
                            const void* saved, size_t saved_bytes, const void* dy, void* dx, const ll_layer_grads* g,
                            void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  if (int st = make_dims(cfg, d)) return st;
  LL_CHECK(p && g, LL_ERR_INVALID_ARG, "params and grads must not be null");
  if (int st = check_ptrs({p->attn_norm_w, p->w_qkv, p->w_o, p->mlp_norm_w, p->w_fc, p->w_proj, p->resid_attn,
                           p->resid_mlp}, "params")) return st;
  if (int st = check_ptrs({g->attn_norm_w, g->w_qkv, g->w_o, g->mlp_norm_w, g->w_fc, g->w_proj, g->resid_attn,
                           g->resid_mlp}, "grads")) return st;
  if (d.ve) {
    if (int st = check_ptrs({p->ve_table, g->ve_table}, "ve_table")) return st;
    LL_CHECK(d.N == 0 || token_ids, LL_ERR_INVALID_ARG, "token_ids required on value-embedding layers");
  }
  if (d.N > 0) {
    if (int st = check_ptrs({x, dy, dx}, "x/dy/dx")) return st;
    LL_CHECK(dx != dy && dx != x, LL_ERR_INVALID_ARG, "dx must not alias dy or x");
  }
  Saved sv;
  BwdWs w;
  const size_t need_s = carve_saved(nullptr, d, sv), need_w = carve_bwd(nullptr, d, w);
  LL_CHECK(saved && aligned16(saved), LL_ERR_INVALID_ARG, "saved must be a 16-byte aligned device pointer");
  LL_CHECK(ws && aligned16(ws), LL_ERR_INVALID_ARG, "ws must be a 16-byte aligned device pointer");
  LL_CHECK(saved_bytes >= need_s, LL_ERR_WORKSPACE, "saved buffer too small: need " + std::to_string(need_s));
  LL_CHECK(ws_bytes >= need_w, LL_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_w));
  carve_saved(const_cast<void*>(saved), d, sv);
  carve_bwd(ws, d, w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.bf)
    return layer_bwd_t<bf16, 128>(d, p, CP<bf16>(x), token_ids, sv, CP<bf16>(dy), P<bf16>(dx), g, w, s);
  return layer_bwd_t<float, 64>(d, p, CP<float>(x), token_ids, sv, CP<float>(dy), P<float>(dx), g, w, s);
}

extern "C" int llt_layer_buffer(const ll_layer_cfg* cfg, int32_t region, const char* name, size_t* offset,
                                size_t* bytes) {
  Dims d;
  if (int st = make_dims(cfg, d)) return st;
  LL_CHECK(name && offset && bytes, LL_ERR_INVALID_ARG, "name, offset and bytes must not be null");
  LL_CHECK(region >= 0 && region <= 2, LL_ERR_INVALID_ARG, "region must be 0 (saved), 1 (fwd ws) or 2 (bwd ws)");
  // carve over a fake base (never dereferenced) to read the sub-buffer offsets
  char* const base = reinterpret_cast<char*>(uintptr_t(1) << 40);
  const std::string n(name);
  const size_t e = d.es;
  const void* p = nullptr;
  size_t sz = 0;
  if (region == 0) {
    Saved v;
    carve_saved(base, d, v);
    const struct { const char* k; const void* p; size_t sz; } t[] = {
        {"qs", v.qs, 4 * sizeof(QScale)}, {"xn", v.xn, d.N * d.D * e}, {"qkv", v.qkv, d.N * d.QKVD * e},
        {"qh", v.qh, d.N * d.QD * e}, {"kh", v.kh, d.N * d.KVD * e}, {"o", v.o, d.N * d.QD * e},
        {"lse", v.lse, d.B * d.Hq * d.Tp * sizeof(float)}, {"attn_out", v.attn_out, d.N * d.D * e},
        {"h", v.h, d.N * d.D * e}, {"u", v.u, d.N * d.F * e}, {"m", v.m, d.N * d.D * e},
        {"r1", v.r1, d.N * sizeof(float)}, {"r2", v.r2, d.N * sizeof(float)},
        {"hn8", v.hn8, (size_t)(d.N * d.D)}, {"hn8t", v.hn8t, (size_t)(d.D * d.Np)},
        {"r8t", v.r8t, (size_t)(d.F * d.Np)}, {"w18", v.w18, (size_t)d.F * d.D}, {"w18t", v.w18t, (size_t)d.D * d.F},
        {"w28", v.w28, (size_t)d.D * d.F}, {"w28t", v.w28t, (size_t)d.F * d.D}};
    for (const auto& x : t)
      if (n == x.k) { p = x.p; sz = x.sz; }
  } else if (region == 1) {
    FwdWs v;
    carve_fwd(base, d, v);
    if (n == "hn") { p = v.hn; sz = d.N * d.D * e; }
    if (n == "r8") { p = v.r8; sz = (size_t)(d.N * d.F); }
  } else {
    BwdWs v;
    carve_bwd(base, d, v);
    const struct { const char* k; const void* p; size_t sz; } t[] = {
        {"qs", v.qs, 2 * sizeof(QScale)}, {"dm", v.dm, d.N * d.D * e}, {"du", v.du, d.N * d.F * e},
        {"dm8", v.dm8, (size_t)(d.N * d.D)}, {"dm8t", v.dm8t, (size_t)(d.D * d.Np)},
        {"du8", v.du8, (size_t)(d.N * d.F)}, {"du8t", v.du8t, (size_t)(d.F * d.Np)},
        {"dhn", v.dhn, d.N * d.D * e}, {"dh", v.dh, d.N * d.D * e}, {"dattn", v.dattn, d.N * d.D * e},
        {"dout", v.dout, d.N * d.QD * e}, {"dqkv", v.dqkv, d.N * d.QKVD * e}, {"dxn", v.dxn, d.N * d.D * e}};
    for (const auto& x : t)
      if (n == x.k) { p = x.p; sz = x.sz; }
  }
  LL_CHECK(p, LL_ERR_INVALID_ARG, "no sub-buffer '" + n + "' in this region for this configuration");
  *offset = static_cast<size_t>(static_cast<const char*>(p) - base);
  *bytes = sz;
  return LL_OK;
}
