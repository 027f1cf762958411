// The whole little-lm model for one micro-batch [hn.213312.xyz translation, 设置 / Setup:
// parameter table with token embeddings, an untied LM head, 28 decoder layers and 14
// value-embedding tables on every other layer]: token-embedding gather, the decoder layers
// (ll_layer_fwd / ll_layer_bwd), a final RMSNorm, the fused linear cross-entropy head
// (ll_fused_lce_fwd_bwd), then the backward chain down to a scatter-add into the embedding
// gradient. Everything is enqueued on the caller's stream; this file only sequences launches.
#include <algorithm>
#include <vector>

#include "api.h"
#include "norm.h"
#include "quant.h"

using namespace ll;

namespace {

// out[n, :] = table[ids[n], :]; rows whose id is outside [0, rows) are written as zeros.
template <class T>
__global__ void __launch_bounds__(256)
embed_gather_kernel(const T* __restrict__ table, int64_t rows, int D, const int32_t* __restrict__ ids, int64_t N,
                    T* __restrict__ out) {
  const int segs = D / 8;
  const int64_t total = N * segs;
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < total; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = k / segs;
    const int c = (int)(k - n * segs) * 8;
    const int32_t id = ids[n];
    float v[8];
    if (id >= 0 && id < rows) {
      Vec8<T>::load(table + (int64_t)id * D + c, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    Vec8<T>::store(out + n * D + c, v);
  }
}

// dE[ids[n], :] += d[n, :] in fp32 (atomic adds; ids outside [0, rows) are skipped).
template <class T>
__global__ void __launch_bounds__(256)
embed_scatter_kernel(const T* __restrict__ d, const int32_t* __restrict__ ids, int64_t N, int D,
                     float* __restrict__ dE, int64_t rows) {
  const int segs = D / 8;
  const int64_t total = N * segs;
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < total; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = k / segs;
    const int c = (int)(k - n * segs) * 8;
    const int32_t id = ids[n];
    if (id < 0 || id >= rows) continue;
    float v[8];
    Vec8<T>::load(d + n * D + c, v);
    float* dst = dE + (int64_t)id * D + c;
#pragma unroll
    for (int i = 0; i < 8; ++i) atomicAdd(dst + i, v[i]);
  }
}

unsigned grid_for(int64_t work) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(work, 256), 16384)); }

template <class T>
hipError_t gather(const void* table, int64_t rows, int D, const int32_t* ids, int64_t N, void* out, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  LL_LAUNCH("embed_gather", (embed_gather_kernel<T>), dim3(grid_for(N * (D / 8))), dim3(256), 0, s,
            static_cast<const T*>(table), rows, D, ids, N, static_cast<T*>(out));
  return hipGetLastError();
}

template <class T>
hipError_t scatter(const void* d, const int32_t* ids, int64_t N, int D, float* dE, int64_t rows, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  LL_LAUNCH("embed_scatter", (embed_scatter_kernel<T>), dim3(grid_for(N * (D / 8))), dim3(256), 0, s,
            static_cast<const T*>(d), ids, N, D, dE, rows);
  return hipGetLastError();
}

template <class T>
hipError_t norm_fwd(const void* x, const float* g, int64_t N, int D, float eps, void* y, float* rstd, hipStream_t s) {
  return launch_rmsnorm_fwd(static_cast<const T*>(x), g, static_cast<T*>(y), rstd, N, D, eps, (float*)nullptr, s);
}

// dx = RMSNorm backward (no residual), dg = column sums of the per-wave partials in dgp (N > 0)
template <class T>
int norm_bwd(const void* dy, const void* x, const float* g, const float* rstd, int64_t N, int D, void* dx, float* dg,
             float* dgp, int accumulate, hipStream_t s) {
  LL_HIP(launch_rmsnorm_bwd(static_cast<const T*>(dy), static_cast<const T*>(x), g, rstd, (const T*)nullptr,
                            static_cast<T*>(dx), dgp, N, D, (const float*)nullptr, (T*)nullptr, (const T*)nullptr,
                            (float*)nullptr, s));
  LL_HIP(launch_colsum(dgp, rmsnorm_bwd_partials(N), D, dg, dgp + rmsnorm_bwd_partials(N) * D, s, accumulate));
  return LL_OK;
}

size_t norm_bwd_ws_bytes(int64_t N, int D) {
  return ((size_t)std::max<int64_t>(rmsnorm_bwd_partials(N), 1) * D + colsum_scratch_floats(D)) * sizeof(float);
}

int check_norm_shape(int32_t dtype, int64_t n, int32_t d) {
  LL_CHECK(dtype == LL_F32 || dtype == LL_BF16, LL_ERR_INVALID_ARG, "dtype must be LL_F32 or LL_BF16");
  LL_CHECK(n >= 0, LL_ERR_INVALID_ARG, "n must be >= 0");
  LL_CHECK(d > 0 && d % 8 == 0 && d <= kMaxDChunks * 512, LL_ERR_UNSUPPORTED, "d must be a multiple of 8, <= 4096");
  return LL_OK;
}

// ---------------------------------------------------------------- model memory plan
struct ModelPlan {
  int64_t N;
  int D, es;
  size_t layer_saved, layer_ws, lce_ws, act;
};

int make_plan(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab, int64_t token_chunk, ModelPlan& m) {
  LL_CHECK(cfg, LL_ERR_INVALID_ARG, "cfg must not be null");
  LL_CHECK(n_layers >= 1, LL_ERR_INVALID_ARG, "n_layers must be >= 1");
  LL_CHECK(vocab > 0, LL_ERR_INVALID_ARG, "vocab must be > 0");
  ll_layer_cfg c = *cfg;
  c.has_value_embed = 1;   // the larger plan (a value-embedding layer) covers both kinds of layer
  c.ve_rows = vocab;
  m.layer_saved = ll_layer_saved_bytes(&c);
  m.layer_ws = ll_layer_workspace_bytes(&c);
  LL_CHECK(m.layer_saved > 0 && m.layer_ws > 0, LL_ERR_INVALID_ARG, "invalid layer cfg: " + std::string(ll_last_error()));
  m.N = c.batch * c.seq;
  m.D = c.d_model;
  m.es = c.dtype == LL_BF16 ? 2 : 4;
  m.lce_ws = ll_fused_lce_workspace_bytes(c.dtype, std::max<int64_t>(m.N, 1), c.d_model, vocab, token_chunk, 0);
  LL_CHECK(m.lce_ws > 0, LL_ERR_INVALID_ARG, "invalid head shape: " + std::string(ll_last_error()));
  m.act = (size_t)m.N * m.D * m.es;
  return LL_OK;
}

struct ModelSaved {
  std::vector<char*> x;       // x[0..L]: inputs of each layer, x[L] feeds the final norm
  char* hn;                   // final-norm output (LCE input)
  float* rstd;                // [N]
  std::vector<char*> layer;   // per-layer saved buffers
};

size_t carve_model_saved(void* base, const ModelPlan& m, int L, ModelSaved& s) {
  Carver c(base);
  s.x.resize(L + 1);
  for (int i = 0; i <= L; ++i) s.x[i] = c.take<char>(m.act);
  s.hn = c.take<char>(m.act);
  s.rstd = c.take<float>((size_t)std::max<int64_t>(m.N, 1));
  s.layer.resize(L);
  for (int i = 0; i < L; ++i) s.layer[i] = c.take<char>(m.layer_saved);
  return c.bytes();
}

struct ModelWs {
  char* inner;                // scratch of the layer / LCE calls
  size_t inner_bytes;
  char *dh, *d0, *d1;         // dL/d(final-norm output), ping-pong dL/dx
  float* dgp;                 // final-norm gain partials
};

size_t carve_model_ws(void* base, const ModelPlan& m, ModelWs& w) {
  Carver c(base);
  w.inner_bytes = std::max(m.layer_ws, m.lce_ws);
  w.inner = c.take<char>(w.inner_bytes);
  w.dh = c.take<char>(m.act);
  w.d0 = c.take<char>(m.act);
  w.d1 = c.take<char>(m.act);
  w.dgp = c.take<float>(norm_bwd_ws_bytes(m.N, m.D) / sizeof(float));
  return c.bytes();
}

}  // namespace

// ---------------------------------------------------------------- kernel-level entry points
extern "C" int llt_embedding_gather(int32_t dtype, const void* table, int64_t rows, int32_t d, const int32_t* ids,
                                    int64_t n, void* out, void* stream) {
  if (int st = check_norm_shape(dtype, n, d)) return st;
  LL_CHECK(rows > 0, LL_ERR_INVALID_ARG, "rows must be > 0");
  if (n == 0) return LL_OK;
  LL_CHECK(table && ids && out, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(table) && aligned16(out), LL_ERR_INVALID_ARG, "table and out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LL_BF16) LL_HIP(gather<bf16>(table, rows, d, ids, n, out, s));
  else LL_HIP(gather<float>(table, rows, d, ids, n, out, s));
  return LL_OK;
}

extern "C" int llt_embedding_scatter_add(int32_t dtype, const void* d_out, const int32_t* ids, int64_t n, int32_t d,
                                         float* d_table, int64_t rows, void* stream) {
  if (int st = check_norm_shape(dtype, n, d)) return st;
  LL_CHECK(rows > 0, LL_ERR_INVALID_ARG, "rows must be > 0");
  if (n == 0) return LL_OK;
  LL_CHECK(d_out && ids && d_table, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(d_out), LL_ERR_INVALID_ARG, "d_out must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LL_BF16) LL_HIP(scatter<bf16>(d_out, ids, n, d, d_table, rows, s));
  else LL_HIP(scatter<float>(d_out, ids, n, d, d_table, rows, s));
  return LL_OK;
}

extern "C" int llt_rmsnorm_fwd(int32_t dtype, const void* x, const float* g, int64_t n, int32_t d, float eps, void* y,
                               float* rstd, void* stream) {
  if (int st = check_norm_shape(dtype, n, d)) return st;
  LL_CHECK(eps >= 0.f, LL_ERR_INVALID_ARG, "eps must be >= 0");
  if (n == 0) return LL_OK;
  LL_CHECK(x && g && y && rstd, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(aligned16(x) && aligned16(g) && aligned16(y), LL_ERR_INVALID_ARG, "x, g, y must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == LL_BF16) LL_HIP(norm_fwd<bf16>(x, g, n, d, eps, y, rstd, s));
  else LL_HIP(norm_fwd<float>(x, g, n, d, eps, y, rstd, s));
  return LL_OK;
}

extern "C" size_t llt_rmsnorm_bwd_workspace_bytes(int64_t n, int32_t d) {
  if (n < 0 || d <= 0) return 0;
  return norm_bwd_ws_bytes(n, d);
}

extern "C" int llt_rmsnorm_bwd(int32_t dtype, const void* dy, const void* x, const float* g, const float* rstd,
                               int64_t n, int32_t d, void* dx, float* dg, void* ws, size_t ws_bytes, void* stream) {
  if (int st = check_norm_shape(dtype, n, d)) return st;
  LL_CHECK(g && dg, LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(n == 0 || (dy && x && rstd && dx), LL_ERR_INVALID_ARG, "null pointer");
  LL_CHECK(n == 0 || (aligned16(dy) && aligned16(x) && aligned16(dx)), LL_ERR_INVALID_ARG, "dy, x, dx must be 16-byte aligned");
  LL_CHECK(aligned16(g), LL_ERR_INVALID_ARG, "g must be 16-byte aligned");
  LL_CHECK(ws && aligned16(ws) && ws_bytes >= norm_bwd_ws_bytes(n, d), LL_ERR_WORKSPACE,
           "workspace too small: need " + std::to_string(norm_bwd_ws_bytes(n, d)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* dgp = static_cast<float*>(ws);
  if (n == 0) {
    LL_HIP(fill_f32(dg, 0.f, d, s));
    return LL_OK;
  }
  if (dtype == LL_BF16) return norm_bwd<bf16>(dy, x, g, rstd, n, d, dx, dg, dgp, 0, s);
  return norm_bwd<float>(dy, x, g, rstd, n, d, dx, dg, dgp, 0, s);
}

// ---------------------------------------------------------------- the model
extern "C" size_t ll_model_saved_bytes(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab) {
  ModelPlan m;
  if (make_plan(cfg, n_layers, vocab, 0, m) != LL_OK) return 0;
  ModelSaved s;
  return carve_model_saved(nullptr, m, n_layers, s);
}

extern "C" size_t ll_model_workspace_bytes(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab,
                                           int64_t token_chunk) {
  ModelPlan m;
  if (make_plan(cfg, n_layers, vocab, token_chunk, m) != LL_OK) return 0;
  ModelWs w;
  return carve_model_ws(nullptr, m, w);
}

extern "C" int ll_model_fwd_bwd(const ll_layer_cfg* cfg, int32_t n_layers, int64_t vocab, const ll_model_params* p,
                                const int32_t* token_ids, const int32_t* targets, float softcap,
                                int32_t ignore_index, float grad_scale, int64_t token_chunk, float* loss,
                                const ll_model_grads* g, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                                void* stream) {
  ModelPlan m;
  if (int st = make_plan(cfg, n_layers, vocab, token_chunk, m)) return st;
  LL_CHECK(p && g, LL_ERR_INVALID_ARG, "params and grads must not be null");
  LL_CHECK(p->layers && g->layers, LL_ERR_INVALID_ARG, "params.layers and grads.layers must not be null");
  LL_CHECK(p->embed && p->final_norm_w && p->head && g->embed && g->final_norm_w && g->head && loss,
           LL_ERR_INVALID_ARG, "null pointer in params/grads/loss");
  LL_CHECK(aligned16(p->embed) && aligned16(p->final_norm_w) && aligned16(p->head) && aligned16(g->head),
           LL_ERR_INVALID_ARG, "embed, final_norm_w and head (and its gradient) must be 16-byte aligned");
  LL_CHECK(softcap > 0.f && softcap <= 60.f, LL_ERR_INVALID_ARG, "softcap must be in (0, 60]");
  LL_CHECK(m.N == 0 || (token_ids && targets), LL_ERR_INVALID_ARG, "token_ids and targets must not be null");
  ModelSaved sv;
  ModelWs w;
  const size_t need_s = carve_model_saved(nullptr, m, n_layers, sv), need_w = carve_model_ws(nullptr, m, w);
  LL_CHECK(saved && aligned16(saved), LL_ERR_INVALID_ARG, "saved must be a 16-byte aligned device pointer");
  LL_CHECK(ws && aligned16(ws), LL_ERR_INVALID_ARG, "ws must be a 16-byte aligned device pointer");
  LL_CHECK(saved_bytes >= need_s, LL_ERR_WORKSPACE, "saved buffer too small: need " + std::to_string(need_s));
  LL_CHECK(ws_bytes >= need_w, LL_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_w));
  carve_model_saved(saved, m, n_layers, sv);
  carve_model_ws(ws, m, w);
  // per-layer shapes: a layer is a value-embedding layer iff it has a table
  std::vector<ll_layer_cfg> lc(n_layers, *cfg);
  for (int i = 0; i < n_layers; ++i) {
    lc[i].has_value_embed = p->layers[i].ve_table != nullptr;
    lc[i].ve_rows = vocab;
    LL_CHECK(lc[i].has_value_embed == (g->layers[i].ve_table != nullptr), LL_ERR_INVALID_ARG,
             "layer " + std::to_string(i) + ": ve_table given in params but not in grads (or the reverse)");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = cfg->dtype == LL_BF16;
  const int acc = g->accumulate ? 1 : 0;
  const int64_t N = m.N;
  const int D = m.D;
  const float eps = cfg->rms_eps;
  // forward
  if (bf) LL_HIP(gather<bf16>(p->embed, vocab, D, token_ids, N, sv.x[0], s));
  else LL_HIP(gather<float>(p->embed, vocab, D, token_ids, N, sv.x[0], s));
  for (int i = 0; i < n_layers; ++i) {
    const int st = ll_layer_fwd(&lc[i], &p->layers[i], sv.x[i], token_ids, sv.x[i + 1], sv.layer[i], m.layer_saved,
                                w.inner, w.inner_bytes, stream);
    LL_CHECK(st == LL_OK, st, "layer " + std::to_string(i) + " forward: " + ll_last_error());
  }
  if (bf) LL_HIP(norm_fwd<bf16>(sv.x[n_layers], p->final_norm_w, N, D, eps, sv.hn, sv.rstd, s));
  else LL_HIP(norm_fwd<float>(sv.x[n_layers], p->final_norm_w, N, D, eps, sv.hn, sv.rstd, s));
  // head: loss and dL/d(final-norm output), dL/d(head)
  {
    const int st = ll_fused_lce_fwd_bwd(cfg->dtype, sv.hn, p->head, targets, N, D, vocab, softcap, ignore_index,
                                        grad_scale, token_chunk, 0, acc, loss, nullptr, w.dh, g->head, w.inner,
                                        w.inner_bytes, stream);
    LL_CHECK(st == LL_OK, st, std::string("head: ") + ll_last_error());
  }
  // backward
  if (N > 0) {
    const int st = bf ? norm_bwd<bf16>(w.dh, sv.x[n_layers], p->final_norm_w, sv.rstd, N, D, w.d0, g->final_norm_w,
                                       w.dgp, acc, s)
                      : norm_bwd<float>(w.dh, sv.x[n_layers], p->final_norm_w, sv.rstd, N, D, w.d0, g->final_norm_w,
                                        w.dgp, acc, s);
    if (st) return st;
  } else if (!acc) {
    LL_HIP(fill_f32(g->final_norm_w, 0.f, D, s));
  }
  char* dcur = w.d0;
  char* dnext = w.d1;
  for (int i = n_layers - 1; i >= 0; --i) {
    ll_layer_grads lg = g->layers[i];
    lg.accumulate = acc;
    const int st = ll_layer_bwd(&lc[i], &p->layers[i], sv.x[i], token_ids, sv.layer[i], m.layer_saved, dcur, dnext,
                                &lg, w.inner, w.inner_bytes, stream);
    LL_CHECK(st == LL_OK, st, "layer " + std::to_string(i) + " backward: " + ll_last_error());
    std::swap(dcur, dnext);
  }
  if (!acc) LL_HIP(fill_f32(g->embed, 0.f, vocab * D, s));   // overwrite: start the scatter-add from zero
  if (bf) LL_HIP(scatter<bf16>(dcur, token_ids, N, D, g->embed, vocab, s));
  else LL_HIP(scatter<float>(dcur, token_ids, N, D, g->embed, vocab, s));
  return LL_OK;
}
