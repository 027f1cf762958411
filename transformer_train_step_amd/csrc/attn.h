// Causal grouped-query attention of the little-lm block, forward and backward, with QK-norm and
// RoPE [hn.213312.xyz translation, 设置 / Setup: RoPE, GQA 24 query / 8 KV heads, QK-norm;
// 不起作用的部分 / What didn't work: unconditional causal scaled_dot_product_attention;
// youdonthavefriends cost analysis, "config appendix": head_dim 128, rope_theta 10000].
//
// Layouts (token-major = [batch, seq, heads, head_dim], i.e. rows of the projection outputs):
//   qkv  [N, (Hq + 2 Hkv) DH]    q rows, k rows, v rows (v includes the value embedding)
//   qh   [N, Hq DH], kh [N, Hkv DH]   q^ = RoPE(QKnorm(q)), k^ = RoPE(QKnorm(k)), rounded
//   *t   [B, H, DH, Tp]          "transposed" copies (Tp = T rounded up to 64, zero padded)
//   o    [N, Hq DH];  lse [B, Hq, T] (natural log of the softmax denominators)
// MFMA conventions (16x16 tiles, see gemm.h): run(acc, first, second) adds first . second^T where
// a lane of `first` holds row (lane & 15) and one of `second` col (lane & 15); the result leaves
// lane l with col (l & 15) and rows 4 (l >> 4) + r, r = 0..3. A probability tile P computed that
// way is consumed by the next MFMA straight from registers as its `second` operand, contracting
// over P's rows: the memory operand then reads the matching rows from a transposed LDS tile in
// groups of 4 consecutive elements.
#pragma once
#include "common.h"
#include "gemm.h"

namespace ll {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ RoPE table (fp64 math)
// cs[t][i] = (cos(phi), sin(phi)), phi = t * theta^(-2i/DH), i < DH/2, t < T
__global__ void rope_table_kernel(float2* cs, int T, int half, double theta) {
  const int64_t n = (int64_t)T * half;
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(k / half), i = (int)(k % half);
    const double inv_freq = pow(theta, -2.0 * (double)i / (double)(2 * half));
    const double phi = (double)t * inv_freq;
    cs[k] = make_float2((float)cos(phi), (float)sin(phi));
  }
}

// ------------------------------------------------------------------ QK-norm + RoPE (forward)
// A head vector is handled by DH/16 consecutive lanes, each owning 8 consecutive rotation pairs
// (i, i + DH/2), i = i0 .. i0 + 7: 16-byte loads and stores, the sum of squares reduced across the
// head's lanes by DPP. Heads 0..Hq-1 of a token are q heads, Hq..Hq+Hkv-1 k heads; the kernel takes
// the Hp heads h0 .. h0 + Hp - 1 of every token (the fp32 path passes all of them; the bf16 path
// forms k^ in the QKV GEMM's epilogue and q^ in the attention forward's Q load instead).
template <class T, int DH>
__global__ void __launch_bounds__(256)
qk_prep_kernel(const T* __restrict__ qkv, int64_t ldqkv, const float2* __restrict__ cs, T* __restrict__ qh,
               T* __restrict__ kh, float* __restrict__ rq, float* __restrict__ rk, int64_t N, int T_, int Hq,
               int Hkv, float eps, int h0, int Hp) {
  constexpr int P = DH / 2, TPH = P / 8;
  static_assert(P % 8 == 0 && 64 % TPH == 0, "head_dim a multiple of 16, at most 128 per 8 lanes");
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int i0 = (int)(gid % TPH) * 8;
  const int64_t ht = gid / TPH;
  const bool valid = ht < N * Hp;
  const int64_t n = valid ? ht / Hp : 0;
  const int hh = valid ? h0 + (int)(ht % Hp) : 0;
  float a[8], b[8];
  if (valid) {
    const T* src = qkv + n * ldqkv + (int64_t)hh * DH;
    Vec8<T>::load(src + i0, a);
    Vec8<T>::load(src + P + i0, b);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = b[k] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += a[k] * a[k] + b[k] * b[k];
  ss = group_sum<TPH>(ss);
  const float r = 1.0f / sqrtf(ss / (float)DH + eps);
  if (!valid) return;
  const int t = (int)(n % T_);
  const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)t * P + i0);
  float y0[8], y1[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 cc = c4[q];                 // (cos, sin) of pairs i0 + 2q, i0 + 2q + 1
    const float cv[2] = {cc.x, cc.z}, sv[2] = {cc.y, cc.w};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int k = 2 * q + e;
      const float x0 = a[k] * r, x1 = b[k] * r;
      y0[k] = x0 * cv[e] - x1 * sv[e];
      y1[k] = x0 * sv[e] + x1 * cv[e];
    }
  }
  T* dst = hh < Hq ? qh + (n * Hq + hh) * DH : kh + (n * Hkv + (hh - Hq)) * DH;
  Vec8<T>::store(dst + i0, y0);
  Vec8<T>::store(dst + P + i0, y1);
  if (i0 == 0) {
    if (hh < Hq) rq[n * Hq + hh] = r;
    else rk[n * Hkv + (hh - Hq)] = r;
  }
}

// ------------------------------------------------------------------ backward of QK-norm + RoPE
// dq = r * dqt - q * r^3 * mean(q * dqt) with dqt = RoPE^T(dq^); written into the q/k columns of
// dqkv. dqh [N, Hq DH] and dkh [N, Hkv DH] are fp32. Lane layout as in the forward. (fp32 path; the
// bf16 dQ and dK/dV kernels apply the same backward in their epilogues.)
template <class T, int DH>
__global__ void __launch_bounds__(256)
qk_post_kernel(const float* __restrict__ dqh, const float* __restrict__ dkh, const T* __restrict__ qkv,
               int64_t ldqkv, const float2* __restrict__ cs, const float* __restrict__ rq,
               const float* __restrict__ rk, T* __restrict__ dqkv, int64_t N, int T_, int Hq, int Hkv) {
  constexpr int P = DH / 2, TPH = P / 8;
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int H = Hq + Hkv;
  const int i0 = (int)(gid % TPH) * 8;
  const int64_t ht = gid / TPH;
  const bool valid = ht < N * H;
  const int64_t n = valid ? ht / H : 0;
  const int hh = valid ? (int)(ht % H) : 0;
  float t0[8], t1[8], x0[8], x1[8], r = 0.f;
  if (valid) {
    const float* ds = hh < Hq ? dqh + (n * Hq + hh) * DH : dkh + (n * Hkv + (hh - Hq)) * DH;
    float d0[8], d1[8];
    Vec8<float>::load(ds + i0, d0);
    Vec8<float>::load(ds + P + i0, d1);
    const T* xs = qkv + n * ldqkv + (int64_t)hh * DH;
    Vec8<T>::load(xs + i0, x0);
    Vec8<T>::load(xs + P + i0, x1);
    r = hh < Hq ? rq[n * Hq + hh] : rk[n * Hkv + (hh - Hq)];
    const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)(n % T_) * P + i0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 cc = c4[q];
      const float cv[2] = {cc.x, cc.z}, sv[2] = {cc.y, cc.w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k = 2 * q + e;
        t0[k] = d0[k] * cv[e] + d1[k] * sv[e];            // rotation by -phi
        t1[k] = -d0[k] * sv[e] + d1[k] * cv[e];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) t0[k] = t1[k] = x0[k] = x1[k] = 0.f;
  }
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) dot += x0[k] * t0[k] + x1[k] * t1[k];
  dot = group_sum<TPH>(dot);
  if (!valid) return;
  const float k3 = r * r * r * dot / (float)DH;
  float o0[8], o1[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    o0[k] = r * t0[k] - x0[k] * k3;
    o1[k] = r * t1[k] - x1[k] * k3;
  }
  T* dst = dqkv + n * ldqkv + (int64_t)hh * DH;
  Vec8<T>::store(dst + i0, o0);
  Vec8<T>::store(dst + P + i0, o1);
}

// ------------------------------------------------------------------ Delta = rowsum(dO * O)
// delta [B, Hq, ldl], ldl >= T. DH/8 consecutive lanes per (token, head), 8 elements each.
template <class T, int DH>
__global__ void __launch_bounds__(256)
attn_delta_kernel(const T* __restrict__ dO, const T* __restrict__ O, float* __restrict__ delta, int64_t ldl,
                  int64_t N, int T_, int Hq) {
  constexpr int TPH = DH / 8;
  const int64_t gid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int i0 = (int)(gid % TPH) * 8;
  const int64_t ht = gid / TPH;
  const bool valid = ht < N * Hq;
  float s = 0.f;
  if (valid) {
    float a[8], b[8];
    Vec8<T>::load(dO + ht * DH + i0, a);
    Vec8<T>::load(O + ht * DH + i0, b);
#pragma unroll
    for (int k = 0; k < 8; ++k) s += a[k] * b[k];
  }
  s = group_sum<TPH>(s);
  if (!valid || i0 != 0) return;
  const int64_t n = ht / Hq;
  const int h = (int)(ht % Hq);
  const int64_t b = n / T_, t = n % T_;
  delta[(b * Hq + h) * ldl + t] = s;
}

// ------------------------------------------------------------------ value-embedding gradient
// dE[ids[n], c] += dv[n, c]   (fp32 atomics; duplicate ids accumulate)
template <class T>
__global__ void ve_scatter_kernel(const T* __restrict__ dv, int64_t lddv, const int32_t* __restrict__ ids,
                                  float* __restrict__ dE, int64_t ldE, int64_t rows, int64_t N, int C) {
  const int64_t total = N * C;
  for (int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; k < total; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = k / C;
    const int c = (int)(k - n * C);
    const int32_t id = ids[n];
    if (id >= 0 && id < rows)   // ids outside the table add nothing (as in the forward's gather)
      atomicAdd(dE + (int64_t)id * ldE + c, Elem<T>::ld(dv, n * lddv + c));
  }
}

// ------------------------------------------------------------------ LDS tiles
// Row tile: 64 rows x 256 bytes (DH elements), 16-byte chunks swizzled by (row & 15).
// Transposed tile: DH rows x 64 elements; groups of 4 elements ("units") swizzled by (row & 15).
template <class ET, int DH>
struct AttnTiles {
  static constexpr int kRowBytes = DH * (int)sizeof(ET);
  static_assert(kRowBytes == 256, "attention kernels take 256-byte head vectors (bf16 x 128 or fp32 x 64)");
  static constexpr int kKT = kRowBytes / 128;                 // 128-byte K tiles per head vector
  static constexpr int kUnit = 4 * (int)sizeof(ET);           // bytes per 4-element group
  static constexpr int kTRow = 64 * (int)sizeof(ET);          // bytes per transposed-tile row
  static constexpr int kRowTile = 64 * 256;                   // bytes
  static constexpr int kTTile = DH * kTRow;                   // bytes (= 16 KiB for both types)

  // rows r of a row tile come from src + r * ld (elements); rows >= nvalid are zero
  __device__ __forceinline__ static void load_rows(unsigned char* tile, const ET* src, int64_t ld, int nvalid) {
    uint4* t = reinterpret_cast<uint4*>(tile);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = threadIdx.x + 256 * k, row = c >> 4, ch = c & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < nvalid) v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(src + row * ld) + ch * 16);
      t[row * 16 + (ch ^ (row & 15))] = v;
    }
  }
  // transposed tile rows (DH of them) come from src + row * ld (elements), 64 elements each
  __device__ __forceinline__ static void load_trans(unsigned char* tile, const ET* src, int64_t ld) {
    constexpr int CPR = kTRow / 16;                             // 16-byte chunks per row
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = threadIdx.x + 256 * k, row = c / CPR, ch = c % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(src + row * ld) + ch * 16);
      if constexpr (sizeof(ET) == 2) {
        const int u0 = 2 * ch, u1 = 2 * ch + 1;
        *reinterpret_cast<uint2*>(tile + row * kTRow + ((u0 ^ (row & 15)) * 8)) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(tile + row * kTRow + ((u1 ^ (row & 15)) * 8)) = make_uint2(v.z, v.w);
      } else {
        *reinterpret_cast<uint4*>(tile + row * kTRow + ((ch ^ (row & 15)) * 16)) = v;
      }
    }
  }
  // first-operand fragment of rows [r0, r0 + 16) for K tile kk (32 bytes per lane)
  __device__ __forceinline__ static void frag_rows(const unsigned char* tile, int r0, int kk, uint32_t (&f)[8]) {
    const int lane = threadIdx.x & 63, row = r0 + (lane & 15), g = lane >> 4;
    const uint4* t = reinterpret_cast<const uint4*>(tile);
    const uint4 lo = t[row * 16 + ((kk * 8 + 2 * g) ^ (row & 15))];
    const uint4 hi = t[row * 16 + ((kk * 8 + 2 * g + 1) ^ (row & 15))];
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w; f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  }
  // pointer to unit u of transposed-tile row `row`
  __device__ __forceinline__ static const unsigned char* unit(const unsigned char* tile, int row, int u) {
    return tile + row * kTRow + ((u ^ (row & 15)) * kUnit);
  }
};

// second-operand fragment straight from global memory (rows of DH elements, 32 bytes per lane)
template <class ET, int DH>
__device__ __forceinline__ void frag_global(const ET* rowp, bool valid, int kk, uint32_t (&f)[8]) {
  const int g = (threadIdx.x & 63) >> 4;
  uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
  if (valid) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(rowp) + kk * 128 + g * 32);
    lo = p[0];
    hi = p[1];
  }
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w; f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
}

// acc += first . second^T contracting over 32 elements: two 16-row register tiles (p[0..3] from
// tile 2q, p[4..7] from tile 2q+1) against units u0 (elements 32q + 4g..) and u1 (32q + 16 + 4g..)
template <class ET> struct PMma;
template <> struct PMma<bf16> {
  __device__ __forceinline__ static void run(floatx4& acc, const unsigned char* u0, const unsigned char* u1,
                                             const float (&p)[8]) {
    const uint2 a0 = *reinterpret_cast<const uint2*>(u0);
    const uint2 a1 = *reinterpret_cast<const uint2*>(u1);
    const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
    uint4 b;
    b.x = f2bf2(p[0], p[1]);
    b.y = f2bf2(p[2], p[3]);
    b.z = f2bf2(p[4], p[5]);
    b.w = f2bf2(p[6], p[7]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   acc, 0, 0, 0);
  }
  // Same product with the register operand split into bf16 high and low parts (p = hi + lo to
  // about 16 significant bits), two MFMAs: the probabilities of the forward keep fp32-like
  // precision instead of bf16's 8 bits.
  __device__ __forceinline__ static void run_split(floatx4& acc, const unsigned char* u0, const unsigned char* u1,
                                                   const float (&p)[8]) {
    const uint2 a0 = *reinterpret_cast<const uint2*>(u0);
    const uint2 a1 = *reinterpret_cast<const uint2*>(u1);
    const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
    uint16_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h[i] = f2bf(p[i]);
      l[i] = f2bf(p[i] - bf2f(h[i]));
    }
    uint4 bh, bl;
    bh.x = h[0] | ((uint32_t)h[1] << 16); bh.y = h[2] | ((uint32_t)h[3] << 16);
    bh.z = h[4] | ((uint32_t)h[5] << 16); bh.w = h[6] | ((uint32_t)h[7] << 16);
    bl.x = l[0] | ((uint32_t)l[1] << 16); bl.y = l[2] | ((uint32_t)l[3] << 16);
    bl.z = l[4] | ((uint32_t)l[5] << 16); bl.w = l[6] | ((uint32_t)l[7] << 16);
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bh), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bl), acc, 0, 0, 0);
  }
};
template <> struct PMma<float> {
  __device__ __forceinline__ static void run(floatx4& acc, const unsigned char* u0, const unsigned char* u1,
                                             const float (&p)[8]) {
    const float4 a0 = *reinterpret_cast<const float4*>(u0);
    const float4 a1 = *reinterpret_cast<const float4*>(u1);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.x, p[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.y, p[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.z, p[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0.w, p[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.x, p[4], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.y, p[5], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.z, p[6], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1.w, p[7], acc, 0, 0, 0);
  }
  __device__ __forceinline__ static void run_split(floatx4& acc, const unsigned char* u0, const unsigned char* u1,
                                                   const float (&p)[8]) {
    run(acc, u0, u1, p);
  }
};

template <class ET>
__device__ __forceinline__ void store4(ET* p, const floatx4& v, float s);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, const floatx4& v, float s) {
  uint2 w;
  w.x = f2bf2(v[0] * s, v[1] * s);
  w.y = f2bf2(v[2] * s, v[3] * s);
  *reinterpret_cast<uint2*>(p) = w;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const floatx4& v, float s) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
}

// ------------------------------------------------------------------ forward
// Block: one (b, h) and 128 queries (4 waves x 32). K^ tiles of 64 keys and V^T tiles through LDS.
// S^T = K^ Q^T per 16x16 tile (lane: query col, 4 key rows), online softmax in the exp2 domain,
// O^T += V^T P^T with P split into bf16 high + low parts. Blocks with the most key tiles are dispatched first.
template <class ET, int DH>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(const ET* __restrict__ qh, const ET* __restrict__ kh, const ET* __restrict__ vt,
                ET* __restrict__ o, float* __restrict__ lse, int B, int T_, int Tp, int Hq, int Hkv) {
  using Tl = AttnTiles<ET, DH>;
  constexpr int KT = Tl::kKT, ND = DH / 16;
  __shared__ __attribute__((aligned(16))) unsigned char sK[Tl::kRowTile];
  __shared__ __attribute__((aligned(16))) unsigned char sV[Tl::kTTile];
  const int nqb = (T_ + 127) / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * Hq));
  const int bh = (int)(blockIdx.x % (B * Hq));
  const int b = bh / Hq, h = bh % Hq, hk = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int q0 = qb * 128, qw = q0 + wave * 32;
  const float sl2 = kLog2e / sqrtf((float)DH);

  uint32_t qf[2][KT][8];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = qw + j * 16 + c16;
    const ET* rowp = qh + (((int64_t)b * T_ + q) * Hq + h) * DH;
#pragma unroll
    for (int kk = 0; kk < KT; ++kk) frag_global<ET, DH>(rowp, q < T_, kk, qf[j][kk]);
  }
  floatx4 oacc[ND][2];
#pragma unroll
  for (int d = 0; d < ND; ++d) oacc[d][0] = oacc[d][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  const int qlast = min(q0 + 127, T_ - 1);
  const int nkt = qlast / 64 + 1;
  const ET* kbase = kh + ((int64_t)b * T_ * Hkv + hk) * DH;
  const ET* vbase = vt + ((int64_t)b * Hkv + hk) * DH * (int64_t)Tp;
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * 64;
    __syncthreads();
    Tl::load_rows(sK, kbase + (int64_t)k0 * Hkv * DH, (int64_t)Hkv * DH, min(64, T_ - k0));
    Tl::load_trans(sV, vbase + k0, Tp);
    __syncthreads();
    if (k0 > qw + 31) continue;                     // every key of this tile is in this wave's future
    floatx4 s[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i][0] = s[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KT; ++kk) {
        uint32_t kf[8];
        Tl::frag_rows(sK, i * 16, kk, kf);
        Mma<ET>::template run<2>(s[i][0], kf, qf[0][kk]);
        Mma<ET>::template run<2>(s[i][1], kf, qf[1][kk]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = qw + j * 16 + c16;
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + i * 16 + 4 * g + r;
          const float v = (key > q || key >= T_) ? -INFINITY : s[i][j][r] * sl2;
          s[i][j][r] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mn = fmaxf(m[j], tmax);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(m[j] - mn);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = (mn == -INFINITY) ? 0.f : exp2f(s[i][j][r] - mn);
          s[i][j][r] = p;
          ps += p;
        }
      l[j] = l[j] * alpha + ps;
      m[j] = mn;
#pragma unroll
      for (int d = 0; d < ND; ++d) oacc[d][j] *= alpha;
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float pv[8] = {s[2 * pr][j][0], s[2 * pr][j][1], s[2 * pr][j][2], s[2 * pr][j][3],
                             s[2 * pr + 1][j][0], s[2 * pr + 1][j][1], s[2 * pr + 1][j][2], s[2 * pr + 1][j][3]};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int row = d * 16 + c16;
          PMma<ET>::run_split(oacc[d][j], Tl::unit(sV, row, 8 * pr + g), Tl::unit(sV, row, 8 * pr + 4 + g), pv);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float lt = l[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int q = qw + j * 16 + c16;
    if (q >= T_) continue;
    const float inv = 1.f / lt;
    ET* orow = o + (((int64_t)b * T_ + q) * Hq + h) * DH;
#pragma unroll
    for (int d = 0; d < ND; ++d) store4<ET>(orow + d * 16 + 4 * g, oacc[d][j], inv);
    if (g == 0) lse[((int64_t)b * Hq + h) * T_ + q] = (m[j] + log2f(lt)) * kLn2;
  }
}

// ------------------------------------------------------------------ backward: dK, dV
// Block: one (b, kv head) and 64 keys (4 waves x 16 keys); loops over the Hq/Hkv query heads of
// the group and over query tiles of 64 at or after the keys. Per query tile: S = Q^ K^T and
// dP = dO V^T (lane: key col, 4 query rows), P = exp(S/sqrt(DH) - lse), dS = P (dP - Delta);
// dV^T += dO^T P and dK^T += Q^T dS with dO^T / Q^T from transposed tiles.
template <class ET, int DH>
__global__ void __launch_bounds__(256)
attn_bwd_dkdv_kernel(const ET* __restrict__ qh, const ET* __restrict__ kh, const ET* __restrict__ v, int64_t ldv,
                     const ET* __restrict__ dO, const ET* __restrict__ qt, const ET* __restrict__ dot,
                     const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dkh,
                     ET* __restrict__ dv, int64_t lddv, int B, int T_, int Tp, int Hq, int Hkv) {
  using Tl = AttnTiles<ET, DH>;
  constexpr int KT = Tl::kKT, ND = DH / 16;
  __shared__ __attribute__((aligned(16))) unsigned char sQ[Tl::kRowTile];
  __shared__ __attribute__((aligned(16))) unsigned char sD[Tl::kRowTile];
  __shared__ __attribute__((aligned(16))) unsigned char sQt[Tl::kTTile];
  __shared__ __attribute__((aligned(16))) unsigned char sDt[Tl::kTTile];
  __shared__ float sL[64], sDl[64];
  const int nkb = (T_ + 63) / 64;
  const int kb = (int)(blockIdx.x % nkb);
  const int bk = (int)(blockIdx.x / nkb);
  const int b = bk / Hkv, hk = bk % Hkv;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int kw = kb * 64 + wave * 16;
  const int key = kw + c16;
  const float sl2 = kLog2e / sqrtf((float)DH);

  uint32_t kf[KT][8], vf[KT][8];
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    frag_global<ET, DH>(kh + (((int64_t)b * T_ + key) * Hkv + hk) * DH, key < T_, kk, kf[kk]);
    frag_global<ET, DH>(v + ((int64_t)b * T_ + key) * ldv + (int64_t)hk * DH, key < T_, kk, vf[kk]);
  }
  floatx4 dva[ND], dka[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dva[d] = dka[d] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nqt = (T_ + 63) / 64;
  for (int hi = 0; hi < G; ++hi) {
    const int h = hk * G + hi;
    for (int qtile = kb; qtile < nqt; ++qtile) {
      const int q0 = qtile * 64;
      __syncthreads();
      Tl::load_rows(sQ, qh + (((int64_t)b * T_ + q0) * Hq + h) * DH, (int64_t)Hq * DH, min(64, T_ - q0));
      Tl::load_rows(sD, dO + (((int64_t)b * T_ + q0) * Hq + h) * DH, (int64_t)Hq * DH, min(64, T_ - q0));
      Tl::load_trans(sQt, qt + ((int64_t)b * Hq + h) * DH * (int64_t)Tp + q0, Tp);
      Tl::load_trans(sDt, dot + ((int64_t)b * Hq + h) * DH * (int64_t)Tp + q0, Tp);
      if (threadIdx.x < 64) {
        const int q = q0 + threadIdx.x;
        sL[threadIdx.x] = q < T_ ? lse[((int64_t)b * Hq + h) * T_ + q] * kLog2e : 0.f;
        sDl[threadIdx.x] = q < T_ ? delta[((int64_t)b * Hq + h) * T_ + q] : 0.f;
      }
      __syncthreads();
      if (q0 + 63 < kw) continue;                   // all queries before this wave's keys
      float p[4][4], ds[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        floatx4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KT; ++kk) {
          uint32_t f[8];
          Tl::frag_rows(sQ, i * 16, kk, f);
          Mma<ET>::template run<2>(s, f, kf[kk]);
          Tl::frag_rows(sD, i * 16, kk, f);
          Mma<ET>::template run<2>(dp, f, vf[kk]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ql = i * 16 + 4 * g + r, q = q0 + ql;
          const bool ok = (key <= q) && (q < T_) && (key < T_);
          const float pp = ok ? exp2f(s[r] * sl2 - sL[ql]) : 0.f;
          p[i][r] = pp;
          ds[i][r] = pp * (dp[r] - sDl[ql]);
        }
      }
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const float pv[8] = {p[2 * pr][0], p[2 * pr][1], p[2 * pr][2], p[2 * pr][3],
                             p[2 * pr + 1][0], p[2 * pr + 1][1], p[2 * pr + 1][2], p[2 * pr + 1][3]};
        const float dsv[8] = {ds[2 * pr][0], ds[2 * pr][1], ds[2 * pr][2], ds[2 * pr][3],
                              ds[2 * pr + 1][0], ds[2 * pr + 1][1], ds[2 * pr + 1][2], ds[2 * pr + 1][3]};
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const int row = d * 16 + c16;
          PMma<ET>::run(dva[d], Tl::unit(sDt, row, 8 * pr + g), Tl::unit(sDt, row, 8 * pr + 4 + g), pv);
          PMma<ET>::run(dka[d], Tl::unit(sQt, row, 8 * pr + g), Tl::unit(sQt, row, 8 * pr + 4 + g), dsv);
        }
      }
    }
  }
  if (key >= T_) return;
  const float sc = 1.f / sqrtf((float)DH);
  ET* dvrow = dv + ((int64_t)b * T_ + key) * lddv + (int64_t)hk * DH;
  float* dkrow = dkh + (((int64_t)b * T_ + key) * Hkv + hk) * DH;
#pragma unroll
  for (int d = 0; d < ND; ++d) {
    store4<ET>(dvrow + d * 16 + 4 * g, dva[d], 1.f);
    store4<float>(dkrow + d * 16 + 4 * g, dka[d], sc);
  }
}

// ------------------------------------------------------------------ backward: dQ
// Block: one (b, h) and 64 queries (4 waves x 16); loops over key tiles of 64 up to the diagonal.
// S^T = K^ Q^T and dP^T = V dO^T (lane: query col, 4 key rows); dQ^T += K^T dS^T.
template <class ET, int DH>
__global__ void __launch_bounds__(256)
attn_bwd_dq_kernel(const ET* __restrict__ qh, const ET* __restrict__ kh, const ET* __restrict__ v, int64_t ldv,
                   const ET* __restrict__ dO, const ET* __restrict__ kt, const float* __restrict__ lse,
                   const float* __restrict__ delta, float* __restrict__ dqh, int B, int T_, int Tp, int Hq, int Hkv) {
  using Tl = AttnTiles<ET, DH>;
  constexpr int KT = Tl::kKT, ND = DH / 16;
  __shared__ __attribute__((aligned(16))) unsigned char sK[Tl::kRowTile];
  __shared__ __attribute__((aligned(16))) unsigned char sV[Tl::kRowTile];
  __shared__ __attribute__((aligned(16))) unsigned char sKt[Tl::kTTile];
  const int nqb = (T_ + 63) / 64;
  const int qb = nqb - 1 - (int)(blockIdx.x / (B * Hq));
  const int bh = (int)(blockIdx.x % (B * Hq));
  const int b = bh / Hq, h = bh % Hq, hk = h / (Hq / Hkv);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int qw = qb * 64 + wave * 16, q = qw + c16;
  const float sl2 = kLog2e / sqrtf((float)DH);

  uint32_t qf[KT][8], of[KT][8];
  const bool qok = q < T_;
#pragma unroll
  for (int kk = 0; kk < KT; ++kk) {
    frag_global<ET, DH>(qh + (((int64_t)b * T_ + q) * Hq + h) * DH, qok, kk, qf[kk]);
    frag_global<ET, DH>(dO + (((int64_t)b * T_ + q) * Hq + h) * DH, qok, kk, of[kk]);
  }
  const float lq = qok ? lse[((int64_t)b * Hq + h) * T_ + q] * kLog2e : 0.f;
  const float dl = qok ? delta[((int64_t)b * Hq + h) * T_ + q] : 0.f;
  floatx4 dqa[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dqa[d] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int qlast = min(qb * 64 + 63, T_ - 1);
  const int nkt = qlast / 64 + 1;
  for (int ktile = 0; ktile < nkt; ++ktile) {
    const int k0 = ktile * 64;
    __syncthreads();
    Tl::load_rows(sK, kh + (((int64_t)b * T_ + k0) * Hkv + hk) * DH, (int64_t)Hkv * DH, min(64, T_ - k0));
    Tl::load_rows(sV, v + ((int64_t)b * T_ + k0) * ldv + (int64_t)hk * DH, ldv, min(64, T_ - k0));
    Tl::load_trans(sKt, kt + ((int64_t)b * Hkv + hk) * DH * (int64_t)Tp + k0, Tp);
    __syncthreads();
    if (k0 > qw + 15) continue;
    float dsv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KT; ++kk) {
        uint32_t f[8];
        Tl::frag_rows(sK, i * 16, kk, f);
        Mma<ET>::template run<2>(s, f, qf[kk]);
        Tl::frag_rows(sV, i * 16, kk, f);
        Mma<ET>::template run<2>(dp, f, of[kk]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + i * 16 + 4 * g + r;
        const bool ok = (key <= q) && (key < T_) && qok;
        const float pp = ok ? exp2f(s[r] * sl2 - lq) : 0.f;
        dsv[i][r] = pp * (dp[r] - dl);
      }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const float dv8[8] = {dsv[2 * pr][0], dsv[2 * pr][1], dsv[2 * pr][2], dsv[2 * pr][3],
                            dsv[2 * pr + 1][0], dsv[2 * pr + 1][1], dsv[2 * pr + 1][2], dsv[2 * pr + 1][3]};
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const int row = d * 16 + c16;
        PMma<ET>::run(dqa[d], Tl::unit(sKt, row, 8 * pr + g), Tl::unit(sKt, row, 8 * pr + 4 + g), dv8);
      }
    }
  }
  if (!qok) return;
  const float sc = 1.f / sqrtf((float)DH);
  float* dqrow = dqh + (((int64_t)b * T_ + q) * Hq + h) * DH;
#pragma unroll
  for (int d = 0; d < ND; ++d) store4<float>(dqrow + d * 16 + 4 * g, dqa[d], sc);
}

}  // namespace
}  // namespace ll
