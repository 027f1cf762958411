// RMSNorm forward/backward and the small HBM-bound kernels around the GEMMs of the layer:
// residual-scalar branch scaling with its fused gradient reduction, column sums, transposes.
// RMSNorm with eps 1e-6 and the learnable residual scalars are parts of the little-lm block
// [hn.213312.xyz translation, 设置 / Setup; youdonthavefriends cost analysis, "config appendix":
// rms_norm_eps 1e-6, layer_scale true].
#pragma once
#include "common.h"

namespace ll {
namespace {

constexpr int kMaxDChunks = 8;   // D <= 8 * 512 = 4096 (one wave covers 512 columns per pass)

// y = round(x * r * g), r = 1 / sqrt(mean(x^2) + eps); one wave per row, kNormFwdRows rows per
// block; optional amax of y. The row is loaded once into registers (every 16-byte load of the row
// issued before the first use); g is staged in LDS once per block. Instantiated per count NC of
// 512-column chunks, so the row registers hold only the chunks D has.
constexpr int kNormFwdRows = 16;
template <class T, int NC>
__global__ void __launch_bounds__(256)
rmsnorm_fwd_kernel(const T* __restrict__ x, const float* __restrict__ g, T* __restrict__ y,
                   float* __restrict__ rstd, int64_t N, int D, float eps, float* amax) {
  __shared__ float gs[NC * 512];
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4)
    *reinterpret_cast<float4*>(gs + c) = *reinterpret_cast<const float4*>(g + c);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  float mx = 0.f;
  for (int i = threadIdx.x >> 6; i < kNormFwdRows; i += 4) {
    const int64_t row = (int64_t)blockIdx.x * kNormFwdRows + i;
    if (row >= N) break;
    const T* xr = x + row * D;
    float v[NC][8];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = lane * 8 + j * 512;
      if (c < D) Vec8<T>::load(xr + c, v[j]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (lane * 8 + j * 512 < D)
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += v[j][k] * v[j][k];
    ss = group_sum<64>(ss);
    const float r = 1.0f / sqrtf(ss / (float)D + eps);
    if (lane == 0) rstd[row] = r;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = lane * 8 + j * 512;
      if (c < D) {
        float gv[8];
        Vec8<float>::load(gs + c, gv);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          v[j][k] = Elem<T>::rnd(v[j][k] * r * gv[k]);
          mx = fmaxf(mx, fabsf(v[j][k]));
        }
        Vec8<T>::store(y + row * D + c, v[j]);
      }
    }
  }
  if (amax) block_atomic_max_nonneg(amax, mx);
}

template <class T>
inline hipError_t launch_rmsnorm_fwd(const T* x, const float* g, T* y, float* rstd, int64_t N, int D,
                                     float eps, float* amax, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const dim3 grid((unsigned)cdiv(N, kNormFwdRows));
  switch (cdiv(D, 512)) {
#define LL_NORM_FWD_NC(nc)                                                                              \
  case nc:                                                                                              \
    LL_LAUNCH("rmsnorm_fwd", (rmsnorm_fwd_kernel<T, nc>), grid, dim3(256), 0, s, x, g, y, rstd, N, D, eps, amax); \
    break;
    LL_NORM_FWD_NC(1) LL_NORM_FWD_NC(2) LL_NORM_FWD_NC(3) LL_NORM_FWD_NC(4)
    LL_NORM_FWD_NC(5) LL_NORM_FWD_NC(6) LL_NORM_FWD_NC(7) LL_NORM_FWD_NC(8)
#undef LL_NORM_FWD_NC
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 8 consecutive elements kept in their storage format (16 bytes of bf16 or 32 of fp32).
template <class T> struct Seg8;
template <> struct Seg8<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float operator[](int k) const {
    const uint32_t w = k < 2 ? u.x : k < 4 ? u.y : k < 6 ? u.z : u.w;
    return (k & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct Seg8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float operator[](int k) const {
    const float4& h = k < 4 ? a : b;
    const int q = k & 3;
    return q == 0 ? h.x : q == 1 ? h.y : q == 2 ? h.z : h.w;
  }
};

// RMSNorm backward fused with the residual add (and optionally the next branch scaling):
//   out  = round(resid + r (g d) - x r^3 mean(x g d))       (d = dL/d(normed), x = norm input;
//                                                             resid NULL reads as 0)
//   dg   : per-row-group partial sums of d * x * r  -> dg_part[group][D]
//   if bout: bout = round(a * out) and *dot += sum(out * aux)   (next residual branch)
// A pair of waves owns a row group of kNormBwdRows consecutive rows and splits each row's columns
// (chunk j of thread t covers columns 8 t + 1024 j .. + 7), so a thread holds NC = D / 1024 chunks
// (3 at D = 3072: three waves per SIMD fit, where one wave per row held 6 and only one fitted).
// The two halves of mean(x g d) meet in LDS, in a fixed order, with one barrier per row (two
// alternating slots). A row's d, x, resid and aux are loaded once, all loads of the row issued
// together, and kept in their storage format; g is staged in LDS once per block.
constexpr int kNormBwdRows = 8;
constexpr int kNormBwdCols = 1024;   // columns per pass of a wave pair (128 threads x 8)

template <class T, int NC>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_kernel(const T* __restrict__ d, const T* __restrict__ x, const float* __restrict__ g,
                   const float* __restrict__ rstd, const T* __restrict__ resid, T* __restrict__ out,
                   float* __restrict__ dg_part, int64_t N, int D, const float* a, T* bout,
                   const T* aux, float* dot) {
  __shared__ float gs[NC * kNormBwdCols];
  __shared__ float red[2][2][2];   // [slot][pair][wave of the pair]
  for (int c = threadIdx.x * 4; c < D; c += 256 * 4)
    *reinterpret_cast<float4*>(gs + c) = *reinterpret_cast<const float4*>(g + c);
  __syncthreads();
  const int pair = threadIdx.x >> 7, half = (threadIdx.x >> 6) & 1, t = threadIdx.x & 127;
  const int64_t grp = (int64_t)blockIdx.x * 2 + pair;
  float dga[NC][8];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) dga[j][k] = 0.f;
  const float av = bout ? *a : 0.f;
  float dsum = 0.f;
  // every wave runs all kNormBwdRows iterations (the barrier inside must be reached by all)
  for (int i = 0; i < kNormBwdRows; ++i) {
    const int64_t row = grp * kNormBwdRows + i;
    const bool live = row < N;
    const float r = live ? rstd[row] : 0.f;
    Seg8<T> ds[NC], xs[NC], rs[NC], as[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = t * 8 + j * kNormBwdCols;
      if (live && c < D) {
        ds[j].load(d + row * D + c);
        xs[j].load(x + row * D + c);
        if (resid) rs[j].load(resid + row * D + c);
        if (bout) as[j].load(aux + row * D + c);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = t * 8 + j * kNormBwdCols;
      if (live && c < D) {
        float gv[8];
        Vec8<float>::load(gs + c, gv);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          s += xs[j][k] * gv[k] * ds[j][k];
          dga[j][k] += ds[j][k] * xs[j][k] * r;
        }
      }
    }
    s = group_sum<64>(s);
    if ((threadIdx.x & 63) == 0) red[i & 1][pair][half] = s;
    __syncthreads();
    s = (red[i & 1][pair][0] + red[i & 1][pair][1]) / (float)D;
    const float r3s = r * r * r * s;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = t * 8 + j * kNormBwdCols;
      if (live && c < D) {
        float gv[8], rv[8];
        Vec8<float>::load(gs + c, gv);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          rv[k] = Elem<T>::rnd((resid ? rs[j][k] : 0.f) + (r * (gv[k] * ds[j][k]) - xs[j][k] * r3s));
        Vec8<T>::store(out + row * D + c, rv);
        if (bout) {
          float bv[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            dsum += rv[k] * as[j][k];
            bv[k] = av * rv[k];
          }
          Vec8<T>::store(bout + row * D + c, bv);
        }
      }
    }
  }
  if (grp * kNormBwdRows < N) {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int c = t * 8 + j * kNormBwdCols;
      if (c < D) Vec8<float>::store(dg_part + grp * D + c, dga[j]);
    }
  }
  if (bout) block_atomic_add(dot, dsum);
}

// row groups (dg_part rows) for N rows: whole blocks of two groups; groups past the last row leave
// their dg_part row unwritten, so the count used by the column sum covers written rows only
inline int64_t rmsnorm_bwd_partials(int64_t N) { return cdiv(N, kNormBwdRows); }

template <class T>
inline hipError_t launch_rmsnorm_bwd(const T* d, const T* x, const float* g, const float* rstd,
                                     const T* resid, T* out, float* dg_part, int64_t N, int D,
                                     const float* a, T* bout, const T* aux, float* dot, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int64_t blocks = cdiv(cdiv(N, kNormBwdRows), 2);
  // instantiated per count of 1024-column chunks so that the register arrays hold only the
  // chunks D has
  switch (cdiv(D, kNormBwdCols)) {
#define LL_NORM_BWD_NC(nc)                                                                              \
  case nc:                                                                                              \
    LL_LAUNCH("rmsnorm_bwd", (rmsnorm_bwd_kernel<T, nc>), dim3((unsigned)blocks), dim3(256), 0, s, d, x, g, rstd, \
              resid, out, dg_part, N, D, a, bout, aux, dot);                                            \
    break;
    LL_NORM_BWD_NC(1) LL_NORM_BWD_NC(2) LL_NORM_BWD_NC(3) LL_NORM_BWD_NC(4)
#undef LL_NORM_BWD_NC
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// out[c] = sum_p part[p][c], in two fixed-order levels: block (x, y) of 16 waves sums the rows
// p = y, y + S, y + 2S, .. of 64 columns (wave w takes every 16th of them, coalesced 256-byte rows)
// into mid[y][c]; then one block per 64 columns adds the S rows of mid in order. Deterministic.
constexpr int kColsumSlabs = 32;
__global__ void __launch_bounds__(1024)
colsum_kernel(const float* __restrict__ part, int64_t P, int64_t stride, int D, float* __restrict__ out,
              int accumulate) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (c < D)
    for (int64_t p = blockIdx.y + (int64_t)w * stride; p < P; p += 16 * stride) s += part[p * D + c];
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < D) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += red[i][lane];
    float* o = out + (int64_t)blockIdx.y * D + c;
    *o = accumulate ? *o + t : t;
  }
}

// scratch: kColsumSlabs * D floats
inline size_t colsum_scratch_floats(int D) { return (size_t)kColsumSlabs * D; }
// out = column sums of part [P, D] (out += with accumulate)
inline hipError_t launch_colsum(const float* part, int64_t P, int D, float* out, float* scratch, hipStream_t s,
                                int accumulate = 0) {
  LL_LAUNCH("colsum", colsum_kernel, dim3((unsigned)cdiv(D, 64), kColsumSlabs), dim3(1024), 0, s, part, P,
            (int64_t)kColsumSlabs, D, scratch, 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LL_LAUNCH("colsum", colsum_kernel, dim3((unsigned)cdiv(D, 64), 1), dim3(1024), 0, s, (const float*)scratch,
            (int64_t)kColsumSlabs, (int64_t)1, D, out, accumulate);
  return hipGetLastError();
}

template <class T>
__global__ void __launch_bounds__(256)
scale_dot_kernel(const T* __restrict__ dy, const T* __restrict__ aux, const float* a, T* __restrict__ out,
                 int64_t n8, float* dot, float* amax) {
  const float av = *a;
  float ds = 0.f, mx = 0.f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float dv[8], xv[8];
    Vec8<T>::load(dy + i * 8, dv);
    Vec8<T>::load(aux + i * 8, xv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ds += dv[k] * xv[k];
      dv[k] = Elem<T>::rnd(av * dv[k]);
      mx = fmaxf(mx, fabsf(dv[k]));
    }
    Vec8<T>::store(out + i * 8, dv);
  }
  block_atomic_add(dot, ds);
  if (amax) block_atomic_max_nonneg(amax, mx);
}
template <class T>
inline hipError_t launch_scale_dot(const T* dy, const T* aux, const float* a, T* out, int64_t n, float* dot,
                                   float* amax, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(cdiv(n8, 256), 2048);
  LL_LAUNCH("scale_dot", (scale_dot_kernel<T>), dim3(blocks), dim3(256), 0, s, dy, aux, a, out, n8, dot, amax);
  return hipGetLastError();
}

// Batched 2-D transpose through a 64 x 64 LDS tile:
//   dst[z][c][r] = src[z][r][c] for r < rows, c < cols;  dst[z][c][r] = 0 for rows <= r < rows_pad.
// Batch z = blockIdx.z splits as (z / zdiv, z % zdiv) with source offset zo*sb_outer + zi*sb_inner
// and destination offset z * sd.
template <class T>
__global__ void __launch_bounds__(256)
transpose_kernel(const T* __restrict__ src, int64_t rows, int cols, int64_t lds, T* __restrict__ dst,
                 int64_t ldd, int64_t rows_pad, int zdiv, int64_t sb_outer, int64_t sb_inner, int64_t sd) {
  __shared__ float tile[64][65];
  const int z = blockIdx.z;
  src += (int64_t)(z / zdiv) * sb_outer + (int64_t)(z % zdiv) * sb_inner;
  dst += (int64_t)z * sd;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    const int c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? Elem<T>::ld(src, r * lds + c) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i;
    const int64_t r = r0 + tx;
    if (c < cols && r < rows_pad) Elem<T>::st(dst, (int64_t)c * ldd + r, tile[tx][i]);
  }
}
// bf16 version with 16-byte accesses on both sides (cols, lds, ldd, rows_pad and the batch strides
// multiples of 8): each thread moves two 8-element row segments into an LDS tile and two 8-element
// column segments out of it.
__global__ void __launch_bounds__(256)
transpose_bf16x8_kernel(const bf16* __restrict__ src, int64_t rows, int cols, int64_t lds, bf16* __restrict__ dst,
                        int64_t ldd, int64_t rows_pad, int zdiv, int64_t sb_outer, int64_t sb_inner, int64_t sd) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int z = blockIdx.z;
  src += (int64_t)(z / zdiv) * sb_outer + (int64_t)(z % zdiv) * sb_inner;
  dst += (int64_t)z * sd;
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int item = threadIdx.x + 256 * k, row = item >> 3, seg = 8 * (item & 7);
    const int64_t r = r0 + row;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (r < rows && c0 + seg < cols) u = *reinterpret_cast<const uint4*>(src + r * lds + c0 + seg);
    *reinterpret_cast<uint4*>(&tile[row][seg]) = u;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int item = threadIdx.x + 256 * k, col = item >> 3, rs = 8 * (item & 7);
    const int64_t r = r0 + rs;
    if (c0 + col >= cols || r >= rows_pad) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[rs + 2 * e][col] | ((uint32_t)tile[rs + 2 * e + 1][col] << 16);
    *reinterpret_cast<uint4*>(dst + (int64_t)(c0 + col) * ldd + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <class T>
inline hipError_t launch_transpose(const T* src, int64_t rows, int cols, int64_t lds, T* dst, int64_t ldd,
                                   int64_t rows_pad, int batch, int zdiv, int64_t sb_outer, int64_t sb_inner,
                                   int64_t sd, hipStream_t s) {
  if (cols <= 0 || rows_pad <= 0 || batch <= 0) return hipSuccess;
  if constexpr (std::is_same<T, bf16>::value) {
    if (cols % 8 == 0 && lds % 8 == 0 && ldd % 8 == 0 && rows_pad % 8 == 0 && sb_outer % 8 == 0 &&
        sb_inner % 8 == 0 && sd % 8 == 0 && aligned16(src) && aligned16(dst)) {
      dim3 grid((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows_pad, 64), (unsigned)batch);
      LL_LAUNCH("transpose", transpose_bf16x8_kernel, grid, dim3(256), 0, s, src, rows, cols, lds, dst, ldd, rows_pad,
                zdiv, sb_outer, sb_inner, sd);
      return hipGetLastError();
    }
  }
  dim3 grid((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows_pad, 64), (unsigned)batch);
  LL_LAUNCH("transpose", (transpose_kernel<T>), grid, dim3(256), 0, s, src, rows, cols, lds, dst, ldd, rows_pad,
                     zdiv, sb_outer, sb_inner, sd);
  return hipGetLastError();
}
template <class T>
inline hipError_t transpose2d(const T* src, int64_t rows, int cols, int64_t lds, T* dst, int64_t ldd,
                              int64_t rows_pad, hipStream_t s) {
  return launch_transpose(src, rows, cols, lds, dst, ldd, rows_pad, 1, 1, 0, 0, 0, s);
}

// fp32 -> storage type conversion (weight gradients accumulated in fp32)
template <class T>
__global__ void convert_kernel(const float* __restrict__ src, T* __restrict__ dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    Elem<T>::st(dst, i, src[i]);
}
template <class T>
inline hipError_t launch_convert(const float* src, T* dst, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 8192);
  LL_LAUNCH("convert", (convert_kernel<T>), dim3(blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace
}  // namespace ll
