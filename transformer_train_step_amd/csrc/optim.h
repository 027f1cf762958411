// Optimizer kernels of the training step [youdonthavefriends cost analysis, "config appendix":
// Muon for the matrix parameters, AdamW for the embeddings, LM head, value embeddings and scalars;
// linlog.top article, 吞吐量优化: bf16 master weights]. Muon's orthogonalisation runs on the MFMA
// GEMM of gemm.h; the elementwise parts (momentum, normalisation, update, AdamW) are HBM-bound
// passes here, each reading and writing every tensor once, fp32 arithmetic in between.
#pragma once
#include "common.h"

namespace ll {
namespace {

// Muon momentum, 8 elements per thread and iteration:
//   buf = round(mu buf + g);  u = round(g + mu buf) (Nesterov) or buf;  *ss += sum of u^2.
template <class T>
__global__ void __launch_bounds__(256) muon_momentum_kernel(const T* __restrict__ g, T* __restrict__ buf,
                                                            T* __restrict__ u, int64_t n8, float mu, int nesterov,
                                                            float* ss) {
  float acc = 0.f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float gv[8], bv[8], uv[8];
    Vec8<T>::load(g + i * 8, gv);
    Vec8<T>::load(buf + i * 8, bv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      bv[k] = Elem<T>::rnd(mu * bv[k] + gv[k]);
      uv[k] = nesterov ? Elem<T>::rnd(gv[k] + mu * bv[k]) : bv[k];
      acc += uv[k] * uv[k];
    }
    Vec8<T>::store(buf + i * 8, bv);
    Vec8<T>::store(u + i * 8, uv);
  }
  block_atomic_add(ss, acc);
}

// x = round(u / (sqrt(*ss) + eps)): the Newton-Schulz start X_0 = u / (||u||_F + eps)
template <class T>
__global__ void __launch_bounds__(256) muon_normalise_kernel(const T* __restrict__ u, T* __restrict__ x, int64_t n8,
                                                             const float* ss, float eps) {
  const float inv = 1.f / (sqrtf(*ss) + eps);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    Vec8<T>::load(u + i * 8, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] *= inv;
    Vec8<T>::store(x + i * 8, v);
  }
}

// w = round(w decay - step o): the Muon update with decoupled weight decay (decay = 1 - lr wd,
// step = lr sqrt(max(1, rows / cols)))
template <class T>
__global__ void __launch_bounds__(256) muon_apply_kernel(T* __restrict__ w, const T* __restrict__ o, int64_t n8,
                                                         float decay, float step) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float wv[8], ov[8];
    Vec8<T>::load(w + i * 8, wv);
    Vec8<T>::load(o + i * 8, ov);
#pragma unroll
    for (int k = 0; k < 8; ++k) wv[k] = wv[k] * decay - step * ov[k];
    Vec8<T>::store(w + i * 8, wv);
  }
}

// AdamW on one element (fp32 arithmetic; the stores round to the storage types):
//   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   p = p (1 - lr wd) - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
struct AdamWArgs {
  float b1, b2, eps, decay, step_size, inv_sqrt_bc2;
};
__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, const AdamWArgs& a, bool rnd_state,
                                          bool rnd_p) {
  m = a.b1 * m + (1.f - a.b1) * g;
  v = a.b2 * v + (1.f - a.b2) * (g * g);
  if (rnd_state) {
    m = round_bf(m);
    v = round_bf(v);
  }
  const float den = sqrtf(v) * a.inv_sqrt_bc2 + a.eps;
  p = p * a.decay - a.step_size * (m / den);
  if (rnd_p) p = round_bf(p);
}

// parameters and moments in P (bf16 or fp32), gradients in G; 4 elements per thread and iteration,
// the last n % 4 one at a time
template <class P, class G>
__global__ void __launch_bounds__(256) adamw_kernel(P* __restrict__ p, const G* __restrict__ g, P* __restrict__ m,
                                                    P* __restrict__ v, int64_t n, AdamWArgs a) {
  constexpr bool kB = Elem<P>::kIsBf16;
  const int64_t n4 = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += stride) {
    float pv[4], gv[4], mv[4], vv[4];
    Vec4<P>::load(p + i * 4, pv);
    Vec4<G>::load(g + i * 4, gv);
    Vec4<P>::load(m + i * 4, mv);
    Vec4<P>::load(v + i * 4, vv);
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw_one(pv[k], gv[k], mv[k], vv[k], a, kB, kB);
    Vec4<P>::store(p + i * 4, pv);
    Vec4<P>::store(m + i * 4, mv);
    Vec4<P>::store(v + i * 4, vv);
  }
  for (int64_t i = n4 * 4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    float pv = Elem<P>::ld(p, i), mv = Elem<P>::ld(m, i), vv = Elem<P>::ld(v, i);
    adamw_one(pv, Elem<G>::ld(g, i), mv, vv, a, kB, kB);
    Elem<P>::st(p, i, pv);
    Elem<P>::st(m, i, mv);
    Elem<P>::st(v, i, vv);
  }
}

}  // namespace
}  // namespace ll
