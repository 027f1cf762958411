// Shared device helpers of the gfx950 kernels: bf16 and e4m3fn conversions, 16-byte vector
// types, wave reductions and small launch utilities. Internal to libll.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

// ------------------------------------------------------------------ element types
struct bf16 { uint16_t u; };          // storage type of bf16 tensors
typedef uint8_t fp8;                   // e4m3fn byte

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round a finite fp32 to the nearest bf16, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two values rounded to bf16 and packed (first in the low half), one instruction
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// Load / store one element of a storage type as fp32; store rounds (RNE) for bf16.
template <class T> struct Elem;
template <> struct Elem<float> {
  static constexpr bool kIsBf16 = false;
  __device__ __forceinline__ static float ld(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void st(float* p, int64_t i, float v) { p[i] = v; }
  __device__ __forceinline__ static float rnd(float v) { return v; }
};
template <> struct Elem<bf16> {
  static constexpr bool kIsBf16 = true;
  __device__ __forceinline__ static float ld(const bf16* p, int64_t i) { return bf2f(p[i].u); }
  __device__ __forceinline__ static void st(bf16* p, int64_t i, float v) { p[i].u = f2bf(v); }
  __device__ __forceinline__ static float rnd(float v) { return round_bf(v); }
};

// 8 consecutive elements <-> 8 floats (16 B for bf16, 32 B for fp32).
template <class T> struct Vec8;
template <> struct Vec8<bf16> {
  __device__ __forceinline__ static void load(const bf16* p, float (&v)[8]) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(w[i] << 16); v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u); }
  }
  __device__ __forceinline__ static void store(bf16* p, const float (&v)[8]) {
    uint4 r;
    r.x = f2bf2(v[0], v[1]);
    r.y = f2bf2(v[2], v[3]);
    r.z = f2bf2(v[4], v[5]);
    r.w = f2bf2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = r;
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// 4 consecutive elements <-> 4 floats (8 B for bf16, 16 B for fp32).
template <class T> struct Vec4;
template <> struct Vec4<bf16> {
  __device__ __forceinline__ static void load(const bf16* p, float (&v)[4]) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xFFFF0000u);
    v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void store(bf16* p, const float (&v)[4]) {
    uint2 r;
    r.x = f2bf2(v[0], v[1]);
    r.y = f2bf2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = r;
  }
};
template <> struct Vec4<float> {
  __device__ __forceinline__ static void load(const float* p, float (&v)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// ------------------------------------------------------------------ e4m3fn
// Round finite fp32 values with |v| <= 448 to the nearest e4m3fn codes, ties to even (OCP E4M3:
// bias 7, 3 mantissa bits, subnormal quantum 2^-9, largest finite 448), four at a time, code k in
// byte k. gfx950's v_cvt_pk_fp8_f32 converts to OCP e4m3fn with round-to-nearest-even and
// subnormals; over every fp32 pattern with |v| <= 448 it gives the same code as rebiasing the
// exponent (-120) and rounding the mantissa from 23 to 3 bits (|v| >= 2^-6), or rounding |v| / 2^-9
// to an integer (|v| < 2^-6), which is how the rule was checked.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float v0, float v1, float v2, float v3) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, lo, true);
}

// relu that passes NaN through (fmaxf(NaN, 0) would return 0); equal to max(v, 0) otherwise
__device__ __forceinline__ float relu_keep_nan(float v) { return v < 0.f ? 0.f : v; }

// Decode an e4m3fn code (finite codes only) to fp32.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80) ? -mag : mag;
}

// ------------------------------------------------------------------ reductions
// Lane movement by DPP (no LDS round trip): CTRL is the dpp_ctrl code (quad_perm 0x00-0xFF,
// row_mirror 0x140, row_half_mirror 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of W consecutive lanes (W = 1, 2, 4, .., 64), in every lane of the group:
// quad swaps (lane ^ 1, lane ^ 2), then the mirrors within 8 and 16 lanes (the quads, then the
// halves, already hold their sums), ds_swizzle for lane ^ 16 and one permute for lane ^ 32.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W is a power of two up to 64");
  if constexpr (W >= 2) v += dpp_move<0xB1>(v);        // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) v += dpp_move<0x4E>(v);        // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) v += dpp_move<0x141>(v);       // row_half_mirror
  if constexpr (W >= 16) v += dpp_move<0x140>(v);      // row_mirror
  if constexpr (W >= 32)                               // bit-mode swizzle: lane ^ 16 within 32
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W is a power of two up to 64");
  if constexpr (W >= 2) v = fmaxf(v, dpp_move<0xB1>(v));
  if constexpr (W >= 4) v = fmaxf(v, dpp_move<0x4E>(v));
  if constexpr (W >= 8) v = fmaxf(v, dpp_move<0x141>(v));
  if constexpr (W >= 16) v = fmaxf(v, dpp_move<0x140>(v));
  if constexpr (W >= 32)
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F)));
  if constexpr (W >= 64) v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Sum (max) of v over the 4 waves of a 256-thread block, added (maxed, v >= 0) into *addr with one
// atomic per block instead of one per wave: thousands of atomics on one address serialise.
// Every thread of the block must call it, at most once per kernel.
__device__ __forceinline__ void block_atomic_add(float* addr, float v) {
  __shared__ float red_add[4];
  v = group_sum<64>(v);
  if ((threadIdx.x & 63) == 0) red_add[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(addr, (red_add[0] + red_add[1]) + (red_add[2] + red_add[3]));
}
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v);
__device__ __forceinline__ void block_atomic_max_nonneg(float* addr, float v) {
  __shared__ float red_max[4];
  v = group_max<64>(v);
  if ((threadIdx.x & 63) == 0) red_max[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) atomic_max_nonneg(addr, fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3])));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// atomic max of a non-negative float through its bit pattern (monotone for v >= 0)
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// ------------------------------------------------------------------ launch tracing (host)
// When tracing is on (llt_trace_begin), every launch is bracketed by two HIP events recorded on
// the launch's own stream, tagged with the kernel's name; llt_trace_get reads the durations.
// Process-wide GEMM block-tile override (0 = automatic), set through llt_set_gemm_config.
int gemm_config_override();

// GEMM launches also record their (M, N, K).
bool trace_on();
int trace_open(const char* tag, hipStream_t s, int64_t m = 0, int64_t n = 0, int64_t k = 0, int gemm_cfg = 0,
               int slices = 0);
void trace_close(int slot, hipStream_t s);

#define LL_LAUNCH_MNK(tag, m, n, k, kern, grid, block, shm, stream, ...)                          \
  do {                                                                                          \
    const int ll_slot_ = ::ll::trace_on() ? ::ll::trace_open((tag), (stream), (m), (n), (k)) : -1; \
    hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                            \
    if (ll_slot_ >= 0) ::ll::trace_close(ll_slot_, (stream));                                   \
  } while (0)
// GEMM launches also record the block configuration that ran and the number of K slices
#define LL_LAUNCH_GEMM(tag, m, n, k, cfg, slices, kern, grid, block, shm, stream, ...)             \
  do {                                                                                          \
    const int ll_slot_ =                                                                        \
        ::ll::trace_on() ? ::ll::trace_open((tag), (stream), (m), (n), (k), (cfg), (slices)) : -1; \
    hipLaunchKernelGGL(kern, grid, block, shm, stream, __VA_ARGS__);                            \
    if (ll_slot_ >= 0) ::ll::trace_close(ll_slot_, (stream));                                   \
  } while (0)
#define LL_LAUNCH(tag, kern, grid, block, shm, stream, ...) \
  LL_LAUNCH_MNK(tag, 0, 0, 0, kern, grid, block, shm, stream, __VA_ARGS__)

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Blocks are dispatched round-robin over the 8 XCDs of MI355X (block b runs on XCD b % 8), each
// XCD with its own L2. Renumber so that consecutive logical tiles land on the same XCD.
__device__ __forceinline__ int xcd_remap(int b, int nb) {
  const int x = b & 7, i = b >> 3, q = nb >> 3, r = nb & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

}  // namespace ll
