// Dynamic tensorwise e4m3fn quantisation (two phases: global amax, then cast), as used by the
// FP8 GEMMs of the MLP [hn.213312.xyz translation, 提升吞吐量 / Increasing throughput: FP8 with
// dynamic scaling on three GEMMs; linlog.top article, 吞吐量优化: torch._scaled_mm, dynamic
// tensorwise scaling].
//   amax      = max |x|                           (order-independent, so bit-reproducible)
//   scale     = 2^floor(log2(fl32(448 / max(amax, 1e-12))))   (power of two: x * scale is exact
//               and a rounding-level change of amax leaves the scale unchanged)
//   inv_scale = 1 / scale                         (exact)
//   q         = e4m3fn_rne(clamp(fl32(x * scale), -448, 448))
// The cast kernel writes the row-major codes and, optionally, the transposed codes (the K-major
// operand of the weight-gradient GEMMs) through a 128 x 128 byte tile in LDS. The transposed
// buffer may have more columns than `rows` (a padded leading dimension); those are zero-filled
// so a GEMM may run its K loop over whole 128-byte tiles.
#pragma once
#include "common.h"

namespace ll {
namespace {

struct QScale {        // per-tensor quantisation state (device memory)
  float amax;
  float scale;
  float inv_scale;
  float pad;
};

__global__ void fill_f32_kernel(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
inline hipError_t fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 4096);
  LL_LAUNCH("fill_f32", fill_f32_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

// amax of x [rows, cols] (ld elements per row); cols % 8 == 0 and ld % 8 == 0.
template <class T>
__global__ void __launch_bounds__(256) amax_kernel(const T* __restrict__ x, int64_t rows, int cols, int64_t ld, float* amax) {
  const int segs = cols / 8;
  float mx = 0.f;
  const int64_t total = rows * segs, stride = (int64_t)gridDim.x * blockDim.x;
  // four independent 16-byte loads in flight per thread and iteration
  for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < total; i0 += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = i0 + u * stride;
      if (i < total) {
        const int64_t r = i / segs;
        Vec8<T>::load(x + r * ld + (int)(i - r * segs) * 8, v[u]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[u][k] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(v[u][k]));
  }
  block_atomic_max_nonneg(amax, mx);
}

template <class T>
inline hipError_t launch_amax(const T* x, int64_t rows, int cols, int64_t ld, float* amax, hipStream_t s) {
  const int64_t total = rows * (cols / 8);
  if (total <= 0) return hipSuccess;
  // 1024 blocks: each ends with one atomic max on the same address, and those atomics serialise
  // (2048 blocks took a third longer on a 75 MB weight); 1024 x 256 threads x 64 bytes still keeps
  // 16 MB of loads in flight
  const int blocks = (int)std::min<int64_t>(cdiv(total, 256), 1024);
  LL_LAUNCH("amax", (amax_kernel<T>), dim3(blocks), dim3(256), 0, s, x, rows, cols, ld, amax);
  return hipGetLastError();
}

__device__ __forceinline__ void scales_from_amax(float amax, float& scale, float& inv) {
  const float ratio = __fdiv_rn(448.0f, fmaxf(amax, 1e-12f));   // normal: in [1.3e-36, 4.5e14]
  scale = __uint_as_float(__float_as_uint(ratio) & 0x7F800000u);  // clear the mantissa
  inv = __fdiv_rn(1.0f, scale);                                   // exact for a power of two
}

// Codes of 4 values: clamp(fl32(x * scale), -448, 448) rounded to e4m3fn; a NaN product (a NaN
// input, or an infinite one times a zero scale) gives the NaN code 0x7F, so that a non-finite
// activation reaches the GEMM as NaN instead of being clamped into a finite code
__device__ __forceinline__ uint32_t quant4(const float* x, float scale) {
  float y[4];
  uint32_t nan_bytes = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float p = __fmul_rn(x[k], scale);
    nan_bytes |= (p != p) ? (0xFFu << (8 * k)) : 0u;
    y[k] = fminf(fmaxf(p, -448.0f), 448.0f);
  }
  const uint32_t c = f32x4_to_e4m3(y[0], y[1], y[2], y[3]);
  return (c & ~nan_bytes) | (0x7F7F7F7Fu & nan_bytes);
}

// Cast of x [rows, cols] with the scale derived from qs->amax. Block = 128 x 128 tile, 256 threads;
// each thread converts 16 consecutive elements of one row in each of four 32-row quarters, so that
// both the codes and the transposed codes leave the block as whole 128-byte rows.
//   q   [rows, ldq] (or null); qt [cols, ldqt] (or null) with ldqt >= rows_pad >= rows;
//   the grid covers rows_pad rows so qt[:, rows:rows_pad] is zero-filled.
// cols % 16 == 0, ld % 8 == 0, ldq % 16 == 0 (any ldqt; 16-byte stores when ldqt % 16 == 0). Block (0,0) thread 0 also writes qs->scale / qs->inv_scale.
// RELU2: the tensor quantised is r = round(relu(x)^2), formed from x on the fly (x = the MLP's
// pre-activation u, so r itself is never stored).
constexpr int kCastTile = 128;
template <class T, bool RELU2 = false>
__global__ void __launch_bounds__(256)
cast_e4m3_kernel(const T* __restrict__ x, int64_t rows, int cols, int64_t ld, QScale* qs,
                 uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt,
                 int64_t rows_pad, float* scale_out, float* inv_out) {
  __shared__ uint32_t tile[kCastTile][kCastTile / 4 + 1];   // 128 rows x 128 bytes (+4 B pad per row)
  float scale, inv;
  scales_from_amax(qs->amax, scale, inv);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    qs->scale = scale;
    qs->inv_scale = inv;
    if (scale_out) *scale_out = scale;
    if (inv_out) *inv_out = inv;
  }
  const int64_t r0 = (int64_t)blockIdx.y * kCastTile;
  const int c0 = blockIdx.x * kCastTile;
  const int tc = (threadIdx.x & 7) * 16;
  const int c = c0 + tc;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int tr = (threadIdx.x >> 3) + 32 * h;
    const int64_t r = r0 + tr;
    uint32_t w[4] = {0, 0, 0, 0};
    if (r < rows && c < cols) {
      float v[16];
      Vec8<T>::load(x + r * ld + c, *reinterpret_cast<float(*)[8]>(v));
      Vec8<T>::load(x + r * ld + c + 8, *reinterpret_cast<float(*)[8]>(v + 8));
      if constexpr (RELU2) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float p = relu_keep_nan(v[k]);
          v[k] = Elem<T>::rnd(p * p);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = quant4(v + 4 * k, scale);
      if (q) *reinterpret_cast<uint4*>(q + r * ldq + c) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (qt) {
#pragma unroll
      for (int k = 0; k < 4; ++k) tile[tr][(tc >> 2) + k] = w[k];
    }
  }
  if (!qt) return;
  __syncthreads();
  // transposed: thread -> output row (source column) cc, 16 source rows rr .. rr + 15; 8 threads
  // write one output row's 128 bytes
  const unsigned char* tb = reinterpret_cast<const unsigned char*>(&tile[0][0]);
  constexpr int RB = (kCastTile / 4 + 1) * 4;               // bytes per LDS tile row
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int cc = (threadIdx.x >> 3) + 32 * h, rr = (threadIdx.x & 7) * 16;
    if (c0 + cc < cols && r0 + rr < rows_pad) {
      uint8_t* dst = qt + (int64_t)(c0 + cc) * ldqt + r0 + rr;
      if ((ldqt & 15) == 0 && r0 + rr + 16 <= rows_pad) {
        uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 16; ++k) o[k >> 2] |= (uint32_t)tb[(rr + k) * RB + cc] << (8 * (k & 3));
        *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        for (int k = 0; k < 16 && r0 + rr + k < rows_pad; ++k) dst[k] = tb[(rr + k) * RB + cc];
      }
    }
  }
}

template <class T, bool RELU2 = false>
inline hipError_t launch_cast_e4m3(const T* x, int64_t rows, int cols, int64_t ld, QScale* qs,
                                   uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, int64_t rows_pad,
                                   float* scale_out, float* inv_out, hipStream_t s) {
  const int64_t rp = qt ? rows_pad : rows;
  const int64_t gy = cdiv(std::max<int64_t>(rp, 1), kCastTile);
  const int gx = (int)cdiv(std::max(cols, 1), kCastTile);
  LL_LAUNCH(RELU2 ? "cast_e4m3_relu2" : "cast_e4m3", (cast_e4m3_kernel<T, RELU2>), dim3(gx, (unsigned)gy), dim3(256), 0,
            s, x, rows, cols, ld, qs, q, ldq, qt, ldqt, rp, scale_out, inv_out);
  return hipGetLastError();
}

}  // namespace
}  // namespace ll
