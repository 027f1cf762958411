// bf16 causal GQA attention kernels for head_dim 128 (forward, dK/dV, dQ) [hn.213312.xyz
// translation, 设置 / Setup: GQA with 24 query and 8 KV heads, QK-norm, RoPE; youdonthavefriends
// cost analysis, "config appendix": head_dim 128]. Same mathematics as the generic kernels of
// attn.h (online softmax forward saving the log-sum-exp; backward recomputing P from it), laid out
// for gfx950:
//   * every tile moves global -> LDS by direct loads (16 bytes a lane), 2 or 3 stages in flight,
//     one barrier per tile;
//   * one LDS layout serves both operand orientations: a tile is rows of 128 elements (256 bytes)
//     with 16-byte chunks XOR-swizzled by fa_swz(row); a fragment along the head dimension is one
//     16-byte read of a row, and a fragment along the token axis (the transposed operand of
//     dV, dK, dQ and P V) comes from ds_read_b64_tr_b16 over 4 rows x 16 columns, so no
//     transposed copies of Q, K, V or dO exist in memory;
//   * the dK/dV kernel gives each wave 32 keys (K, V and the dK, dV accumulators in registers)
//     so a 64-query tile read from LDS feeds 128 MFMAs per wave.
// MFMA conventions as in gemm.h: mma(acc, first, second) adds first . second^T, a lane of `first`
// holds row (lane & 15) and one of `second` column (lane & 15), each with 8 consecutive k; the
// result leaves lane l with column (l & 15) and rows 4 (l >> 4) + r, r = 0..3.
#pragma once
#include "common.h"
#include "gemm.h"

namespace ll {
namespace {

constexpr float kFaLog2e = 1.4426950408889634f;
constexpr float kFaLn2 = 0.6931471805599453f;

// Chunk swizzle of a 256-byte row (XOR of chunk bits 1..3 with row bits 0..2, and of chunk bit 1
// with row bit 3): the 16-row read at one logical chunk and the 4-row transpose reads (two adjacent
// chunks per row) both run without bank-conflict cycles, as measured with the LDS bank-conflict
// counter (a row bit 3 on chunk bit 0 costs the 16-row read 4 extra cycles).
__device__ __forceinline__ int fa_swz(int row) { return ((row & 7) << 1) ^ ((row >> 2) & 2); }

__device__ __forceinline__ floatx4 fa_mma(floatx4 acc, u32x4 first, u32x4 second) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, first),
                                                 __builtin_bit_cast(bf16x8_t, second), acc, 0, 0, 0);
}

// Issue the direct loads of rows [r0, r0 + R) of a bf16 matrix with 128-element rows at
// src + row * ld (rows at or past rmax repeat row rmax - 1) into an LDS tile; the NW waves of the
// block share the R / 4 one-kilobyte instructions.
template <int R, int NW = 4>
__device__ __forceinline__ void fa_issue(const bf16* src, int64_t ld, int r0, int rmax, unsigned char* lds, int wave,
                                         int lane) {
  static_assert(R % (4 * NW) == 0, "whole instructions per wave");
  constexpr int PW = R / (4 * NW);
  const int phys = lane & 15;
#pragma unroll
  for (int n = 0; n < PW; ++n) {
    const int base = (wave * PW + n) * 1024;
    const int row = (base >> 8) + (lane >> 4);
    const int grow = min(r0 + row, rmax - 1);
    const char* g = reinterpret_cast<const char*>(src + (int64_t)grow * ld) + ((phys ^ fa_swz(row)) << 4);
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)(lds + base), 16, 0, 0);
  }
}

// 8 elements (16 bytes) of tile row `row` at logical chunk `ch` (elements 8 ch .. 8 ch + 7)
__device__ __forceinline__ u32x4 fa_rfrag(const unsigned char* t, int row, int ch) {
  return *reinterpret_cast<const u32x4*>(t + (row * 256 + ((ch ^ fa_swz(row)) << 4)));
}

// Fragment of tile column c0 + (lane & 15) (c0 a multiple of 16) over 8 tile rows,
// k0 + 4g + r and k0 + 16 + 4g + r (r = 0..3, g = lane >> 4, k0 a multiple of 32): the k order
// of an MFMA operand whose other side comes from two 16-row accumulator tiles.
__device__ __forceinline__ u32x4 fa_tfrag(const unsigned char* t, int k0, int c0, int lane) {
  const int li = lane & 15, g = lane >> 4;
  const int row = k0 + 4 * g + (li >> 2);
  const int j = li & 3;
  const int off = row * 256 + ((((c0 >> 3) + (j >> 1)) ^ fa_swz(row)) << 4) + ((j & 1) << 3);
  const u32x2 h0 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (__attribute__((address_space(3))) shortx4*)(t + off)));
  const u32x2 h1 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                  (__attribute__((address_space(3))) shortx4*)(t + (off + 16 * 256))));
  return __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
}

typedef float fa_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 fa_bf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t fa_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(fa_f2{a, b}, fa_bf2));
}
// the 8 values {x[0..3], y[0..3]} of two accumulator tiles as one bf16 MFMA operand
__device__ __forceinline__ u32x4 fa_operand(const floatx4& x, const floatx4& y) {
  return u32x4{fa_pack(x[0], x[1]), fa_pack(x[2], x[3]), fa_pack(y[0], y[1]), fa_pack(y[2], y[3])};
}
// high and low bf16 parts of the same values (x = hi + lo to about 16 significant bits)
__device__ __forceinline__ void fa_operand_split(const floatx4& x, const floatx4& y, u32x4& hi, u32x4& lo) {
  hi = fa_operand(x, y);
  floatx4 xr, yr;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    xr[2 * r] = __uint_as_float(hi[r] << 16);
    xr[2 * r + 1] = __uint_as_float(hi[r] & 0xffff0000u);
    yr[2 * r] = __uint_as_float(hi[2 + r] << 16);
    yr[2 * r + 1] = __uint_as_float(hi[2 + r] & 0xffff0000u);
  }
  lo = fa_operand(x - xr, y - yr);
}

__device__ __forceinline__ void fa_store4(bf16* p, const floatx4& v, float s) {
  *reinterpret_cast<uint2*>(p) = make_uint2(fa_pack(v[0] * s, v[1] * s), fa_pack(v[2] * s, v[3] * s));
}

// Backward of x^ = RoPE(x / rms(x)) (QK-norm without a gain, then the rotation of channel pairs
// (i, i + 64) by the position's angles) for one 128-element head row held by the 4 lanes
// g = 0..3 of one column c16 of an MFMA result: a[t][r] is the gradient of x^ at channel
// 16 t + 4 g + r, before the factor sc. With dr = RoPE^T(sc a) and rr = 1 / rms(x):
// dx = rr dr - x rr^3 mean(x . dr) [hn.213312.xyz translation, 设置 / Setup: QK-norm and RoPE].
// xr: the raw row (bf16), csr: its position's (cos, sin) of pairs 0..63, dst: where dx goes (bf16);
// every lane takes part in the row sum, only lanes with `store` write.
__device__ __forceinline__ void fa_norm_rope_bwd(const floatx4 (&a)[8], float sc, const bf16* __restrict__ xr,
                                                 const float2* __restrict__ csr, float rr, bf16* __restrict__ dst,
                                                 int g, bool store) {
  float t0[4][4], t1[4][4], x0[4][4], x1[4][4];
  float dot = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * t + 4 * g;
    const uint2 u0 = *reinterpret_cast<const uint2*>(xr + i);
    const uint2 u1 = *reinterpret_cast<const uint2*>(xr + i + 64);
    const float4 c01 = *reinterpret_cast<const float4*>(csr + i);
    const float4 c23 = *reinterpret_cast<const float4*>(csr + i + 2);
    const float cv[4] = {c01.x, c01.z, c23.x, c23.z}, sv[4] = {c01.y, c01.w, c23.y, c23.w};
    const uint32_t w0[2] = {u0.x, u0.y}, w1[2] = {u1.x, u1.y};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x0[t][r] = __uint_as_float(r & 1 ? (w0[r >> 1] & 0xffff0000u) : (w0[r >> 1] << 16));
      x1[t][r] = __uint_as_float(r & 1 ? (w1[r >> 1] & 0xffff0000u) : (w1[r >> 1] << 16));
      const float d0 = a[t][r] * sc, d1 = a[t + 4][r] * sc;
      t0[t][r] = d0 * cv[r] + d1 * sv[r];            // rotation by -angle
      t1[t][r] = -d0 * sv[r] + d1 * cv[r];
      dot += x0[t][r] * t0[t][r] + x1[t][r] * t1[t][r];
    }
  }
  dot += __shfl_xor(dot, 16, 64);
  dot += __shfl_xor(dot, 32, 64);
  const float k3 = rr * rr * rr * dot * (1.f / 128.f);
  if (!store) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int i = 16 * t + 4 * g;
    *reinterpret_cast<uint2*>(dst + i) =
        make_uint2(fa_pack(rr * t0[t][0] - x0[t][0] * k3, rr * t0[t][1] - x0[t][1] * k3),
                   fa_pack(rr * t0[t][2] - x0[t][2] * k3, rr * t0[t][3] - x0[t][3] * k3));
    *reinterpret_cast<uint2*>(dst + i + 64) =
        make_uint2(fa_pack(rr * t1[t][0] - x1[t][0] * k3, rr * t1[t][1] - x1[t][1] * k3),
                   fa_pack(rr * t1[t][2] - x1[t][2] * k3, rr * t1[t][3] - x1[t][3] * k3));
  }
}

// Block (4 waves) -> (b, h, query block qb): query blocks with the most key tiles first, and the
// Hq/Hkv heads sharing one K/V head on the same XCD (block indices Hkv * B apart).
struct FaBlock {
  int b, h, hk, blk;
};
__device__ __forceinline__ FaBlock fa_block(int B, int Hq, int Hkv, int nblk) {
  const int bhq = B * Hq, bkv = B * Hkv;
  const int idx = (int)blockIdx.x;
  FaBlock r;
  r.blk = nblk - 1 - idx / bhq;
  const int x = idx % bhq;
  const int hi = x / bkv, gid = x % bkv;
  r.b = gid / Hkv;
  r.hk = gid % Hkv;
  r.h = r.hk * (Hq / Hkv) + hi;
  return r;
}

// ------------------------------------------------------------------ forward
// Block: one (b, h) and 128 queries, wave w the 32 queries q0 + 32 w .. (Q in registers as the
// `second` operand). QK-norm and RoPE of q happen in this load: lane (c16, g) reads elements
// 8 g + 32 c .. + 7 (c = 0..3) of its query's raw head vector from the QKV projection, so the
// rotation pairs (i, i + 64) are chunks c and c + 2 of the same lane and the head's sum of squares
// is the sum over the 4 lanes g = 0..3; the lane rounds q^ = RoPE(q / rms(q)) to bf16 as the MFMA
// operand and writes q^ and 1 / rms(q) for the backward. Per 64-key tile: S^T = K Q^T (lane: query
// column, 4 key rows), online softmax in the exp2 domain, O^T += V^T P^T with P split into bf16
// high and low parts. Writes o [N, Hq*128] and lse [B, Hq, ldl] (natural log; entries of queries
// >= T untouched).
//   qkv [N, ldqkv]: q of head h at columns h * 128 ..; cs [T, 64] (cos, sin) of the RoPE angles;
//   qh [N, Hq * 128] and rq [N, Hq] are written.
template <bool kSplit>
__global__ void __launch_bounds__(256, 2)
fa_fwd_kernel(const bf16* __restrict__ qkv, int64_t ldqkv, const float2* __restrict__ cs, float eps,
              bf16* __restrict__ qh, float* __restrict__ rq, const bf16* __restrict__ kh, const bf16* __restrict__ v,
              int64_t ldv, bf16* __restrict__ o, float* __restrict__ lse, int64_t ldl, int B, int T, int Hq, int Hkv) {
  constexpr int DH = 128, STAGE = 2 * 64 * 256;
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE];
  const int nqb = (T + 127) / 128;
  const FaBlock fb = fa_block(B, Hq, Hkv, nqb);
  const int b = fb.b, h = fb.h, hk = fb.hk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int q0 = fb.blk * 128, qw = q0 + wave * 32;
  const float sl2 = kFaLog2e / sqrtf((float)DH);

  u32x4 qf[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qq = qw + 16 * j + c16, q = min(qq, T - 1);
    const bf16* rowp = qkv + ((int64_t)b * T + q) * ldqkv + (int64_t)h * DH + 8 * g;
    float x[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c) Vec8<bf16>::load(rowp + 32 * c, x[c]);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[c][e] * x[c][e];
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float r = 1.0f / sqrtf(ss / (float)DH + eps);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      // (cos, sin) of pairs i = 32 c + 8 g .. + 7
      const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)q * (DH / 2) + 32 * c + 8 * g);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 cc = c4[u];
        const float cv[2] = {cc.x, cc.z}, sv[2] = {cc.y, cc.w};
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int e = 2 * u + e2;
          const float a0 = x[c][e] * r, a1 = x[c + 2][e] * r;
          x[c][e] = a0 * cv[e2] - a1 * sv[e2];
          x[c + 2][e] = a0 * sv[e2] + a1 * cv[e2];
        }
      }
    }
    bf16* qrow = qh + (((int64_t)b * T + q) * Hq + h) * DH + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[j][c] = u32x4{fa_pack(x[c][0], x[c][1]), fa_pack(x[c][2], x[c][3]), fa_pack(x[c][4], x[c][5]),
                       fa_pack(x[c][6], x[c][7])};
      if (qq < T) *reinterpret_cast<u32x4*>(qrow + 32 * c) = qf[j][c];
    }
    if (qq < T && g == 0) rq[((int64_t)b * T + q) * Hq + h] = r;
  }
  const bf16* kb = kh + ((int64_t)b * T * Hkv + hk) * DH;
  const bf16* vb = v + (int64_t)b * T * ldv + (int64_t)hk * DH;
  const int64_t ldk = (int64_t)Hkv * DH;
  auto issue = [&](int kt, unsigned char* s) __attribute__((always_inline)) {
    fa_issue<64>(kb, ldk, kt * 64, T, s, wave, lane);
    fa_issue<64>(vb, ldv, kt * 64, T, s + 64 * 256, wave, lane);
  };

  floatx4 oacc[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) oacc[t][0] = oacc[t][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  auto compute = [&](const unsigned char* sK, int kt) __attribute__((always_inline)) {
    const unsigned char* sV = sK + 64 * 256;
    const int k0 = kt * 64;
    // a key tile wholly at or below the diagonal of this wave's queries, and inside T, needs no
    // mask (wave-uniform: a scalar branch)
    const bool full = __builtin_amdgcn_readfirstlane((int)(k0 + 63 <= qw && k0 + 64 <= T)) != 0;
    floatx4 s[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i][0] = s[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 ka = fa_rfrag(sK, 16 * i + c16, 4 * c + g);
        s[i][0] = fa_mma(s[i][0], ka, qf[0][c]);
        s[i][1] = fa_mma(s[i][1], ka, qf[1][c]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = qw + 16 * j + c16;
      float tmax = -INFINITY;
      if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = s[i][j][r] * sl2;
            s[i][j][r] = x;
            tmax = fmaxf(tmax, x);
          }
      } else {
        const int lim = min(q, T - 1) - k0 - 4 * g;   // key k0 + 4 g + 16 i + r visible iff 16 i + r <= lim
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = 16 * i + r <= lim ? s[i][j][r] * sl2 : -INFINITY;
            s[i][j][r] = x;
            tmax = fmaxf(tmax, x);
          }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // key 0 is visible to every query, so m is finite from the first tile on
      const float mn = fmaxf(m[j], tmax);
      const float alpha = __builtin_amdgcn_exp2f(m[j] - mn);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[i][j][r] - mn);
          s[i][j][r] = p;
          ps += p;
        }
      l[j] = l[j] * alpha + ps;
      m[j] = mn;
#pragma unroll
      for (int t = 0; t < 8; ++t) oacc[t][j] *= alpha;
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (kSplit) fa_operand_split(s[2 * pr][j], s[2 * pr + 1][j], ph[j], pl[j]);
        else ph[j] = fa_operand(s[2 * pr][j], s[2 * pr + 1][j]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 vt = fa_tfrag(sV, 32 * pr, 16 * t, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          oacc[t][j] = fa_mma(oacc[t][j], vt, ph[j]);
          if constexpr (kSplit) oacc[t][j] = fa_mma(oacc[t][j], vt, pl[j]);
        }
      }
    }
  };

  // tile kt in stage kt % 2; each step waits for its tile, then refills the other stage (read by
  // the previous step, which every wave has finished at the barrier) with tile kt + 1
  const int nkt = min(q0 + 127, T - 1) / 64 + 1;
  auto step = [&](auto si, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(si)::value;
    wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    if constexpr (S == 0) { issue(min(kt + 1, nkt - 1), st1); compute(st0, kt); }
    else { issue(min(kt + 1, nkt - 1), st0); compute(st1, kt); }
  };
  // Straight-line loop body (a conditional step would make the compiler's tracking of the loads
  // in flight conservative at the loop head). A step past the last tile recomputes nothing: its
  // keys lie beyond every query of the block (or beyond T), so the causal mask clears them.
  issue(0, st0);
  for (int kt = 0; kt < nkt; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
  wait_vmcnt<0>();

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float lt = l[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int q = qw + 16 * j + c16;
    if (q >= T) continue;
    const float inv = 1.f / lt;
    bf16* orow = o + (((int64_t)b * T + q) * Hq + h) * DH + 4 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t) fa_store4(orow + 16 * t, oacc[t][j], inv);
    if (g == 0) lse[((int64_t)b * Hq + h) * ldl + q] = (m[j] + log2f(lt)) * kFaLn2;
  }
}

// ------------------------------------------------------------------ backward: dK, dV
// Block: one (b, kv head) and 128 keys, wave w the KPW keys k0 + KPW w .. (K and V rows in
// registers as `second` operands, dK^T and dV^T accumulators): KPW = 32 is 4 waves (one per SIMD),
// KPW = 16 is 8 waves (two per SIMD, each reading the whole query tile from LDS for half the MFMAs). Loops over the Hq/Hkv query heads of the
// group and the 64-query tiles at or after k0, three stages in flight. Per tile: S = Q K^T and
// dP = dO V^T (lane: key column, 4 query rows), P = exp2(S log2e / sqrt(DH) - lse log2e),
// dS = P (dP - Delta); dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transpose reads.
// lse and delta are [B, Hq, ldl] with ldl >= T rounded up to 64 (entries past T may hold anything);
// each lane loads the 16 values of its query rows one tile ahead into registers.
// The epilogue writes dV and, through the backward of the keys' QK-norm and RoPE, dK straight into
// their columns of the QKV-projection gradient: kraw (the raw k columns of the QKV projection), dk
// and dv all have row stride lddv; cs [T, 64] holds the RoPE (cos, sin), rk [N, Hkv] 1 / rms(k).
template <int KPW>
__global__ void __launch_bounds__(64 * (128 / KPW), 1)
fa_dkdv_kernel(const bf16* __restrict__ qh, const bf16* __restrict__ kh, const bf16* __restrict__ v, int64_t ldv,
               const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
               int64_t ldl, const bf16* __restrict__ kraw, const float2* __restrict__ cs, const float* __restrict__ rk,
               bf16* __restrict__ dk, bf16* __restrict__ dv, int64_t lddv, int B, int T, int Hq, int Hkv) {
  constexpr int DH = 128;
  constexpr int TILE = 64 * 256, STAGE = 2 * TILE;
  static_assert(KPW == 16 || KPW == 32, "16 or 32 keys per wave");
  constexpr int NWV = 128 / KPW, JN = KPW / 16;
  constexpr int NIW = 32 / NWV;                         // direct loads per wave per stage (Q and dO)
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[STAGE];
  const int idx = (int)blockIdx.x, bkv = B * Hkv;
  const int kblk = idx / bkv, b = (idx % bkv) / Hkv, hk = idx % Hkv;
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int k0 = kblk * 128, kw = k0 + KPW * wave;
  const float sl2 = kFaLog2e / sqrtf((float)DH);

  u32x4 kf[JN][4], vf[JN][4];
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int key = min(kw + 16 * j + c16, T - 1);
    const bf16* kr = kh + (((int64_t)b * T + key) * Hkv + hk) * DH + 8 * g;
    const bf16* vr = v + ((int64_t)b * T + key) * ldv + (int64_t)hk * DH + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kf[j][c] = *reinterpret_cast<const u32x4*>(kr + 32 * c);
      vf[j][c] = *reinterpret_cast<const u32x4*>(vr + 32 * c);
    }
  }
  floatx4 dka[JN][8], dva[JN][8];
#pragma unroll
  for (int j = 0; j < JN; ++j)
#pragma unroll
    for (int t = 0; t < 8; ++t) dka[j][t] = dva[j][t] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nqt = (T + 63) / 64, qt0 = k0 / 64;
  const int nq = nqt - qt0, niter = G * nq;
  const int64_t ldq = (int64_t)Hq * DH;
  auto issue = [&](int it, unsigned char* s) __attribute__((always_inline)) {
    const int hi = it / nq, q0 = (qt0 + it % nq) * 64;
    const int64_t hoff = ((int64_t)b * T * Hq + hk * G + hi) * DH;
    fa_issue<64, NWV>(qh + hoff, ldq, q0, T, s, wave, lane);
    fa_issue<64, NWV>(dO + hoff, ldq, q0, T, s + TILE, wave, lane);
  };
  // lse and delta of query rows 16 i + 4 g + r of tile it live in buffer it % 3 (one buffer per
  // step of the unrolled loop, so no register copies wait on loads in flight)
  floatx4 lb[3][4], db[3][4];
  auto load_ld = [&](int it, auto bi) __attribute__((always_inline)) {
    constexpr int BI = decltype(bi)::value;
    const int hi = it / nq, q0 = (qt0 + it % nq) * 64;
    const int64_t off = ((int64_t)b * Hq + hk * G + hi) * ldl + q0 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lb[BI][i] = *reinterpret_cast<const floatx4*>(lse + off + 16 * i);
      db[BI][i] = *reinterpret_cast<const floatx4*>(delta + off + 16 * i);
    }
  };
  auto compute = [&](const unsigned char* sQ, int it, const floatx4 (&l4)[4], const floatx4 (&d4)[4])
      __attribute__((always_inline)) {
    const unsigned char* sO = sQ + TILE;
    const bool live = it < niter;
    const int q0 = (qt0 + it % nq) * 64;
    floatx4 s[JN][4], dp[JN][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < JN; ++j) s[j][i] = dp[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 qa = fa_rfrag(sQ, 16 * i + c16, 4 * c + g);
        const u32x4 oa = fa_rfrag(sO, 16 * i + c16, 4 * c + g);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          s[j][i] = fa_mma(s[j][i], qa, kf[j][c]);
          dp[j][i] = fa_mma(dp[j][i], oa, vf[j][c]);
        }
      }
    }
    // a query tile wholly at or past the diagonal of this wave's keys, and inside T, needs no mask
    // (wave-uniform: a scalar branch)
    const bool full = __builtin_amdgcn_readfirstlane((int)(live && q0 >= kw + KPW - 1 && q0 + 64 <= T && kw + KPW <= T)) != 0;
    if (full) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[j][i][r] * sl2 - l4[i][r] * kFaLog2e);
            s[j][i][r] = p;
            dp[j][i][r] = p * (dp[j][i][r] - d4[i][r]);
          }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const int key = kw + 16 * j + c16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int q = q0 + 16 * i + 4 * g + r;
            const bool ok = live && key <= q && q < T && key < T;
            const float p = __builtin_amdgcn_exp2f(s[j][i][r] * sl2 - l4[i][r] * kFaLog2e);
            s[j][i][r] = ok ? p : 0.f;
            dp[j][i][r] = ok ? p * (dp[j][i][r] - d4[i][r]) : 0.f;
          }
        }
      }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      u32x4 pp[JN], ds[JN];
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        pp[j] = fa_operand(s[j][2 * pr], s[j][2 * pr + 1]);
        ds[j] = fa_operand(dp[j][2 * pr], dp[j][2 * pr + 1]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 ot = fa_tfrag(sO, 32 * pr, 16 * t, lane);
        const u32x4 qt = fa_tfrag(sQ, 32 * pr, 16 * t, lane);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          dva[j][t] = fa_mma(dva[j][t], ot, pp[j]);
          dka[j][t] = fa_mma(dka[j][t], qt, ds[j]);
        }
      }
    }
  };
  // Step it: this wave's loads of stage it and of the lse / delta of tile it have landed (only
  // the stage of tile it + 1 may still be loading); after the barrier the stage of tile it - 1 is
  // refilled with tile it + 2. Issue order per step: lse / delta of tile it + 1, then the stage of
  // tile it + 2, so one wait count holds for every step.
  auto step = [&](auto si, int it) __attribute__((always_inline)) {
    constexpr int S = decltype(si)::value;
    wait_vmcnt<NIW>();
    asm volatile("s_barrier" ::: "memory");
    load_ld(min(it + 1, niter - 1), std::integral_constant<int, (S + 1) % 3>{});
    const int nx = min(it + 2, niter - 1);
    if constexpr (S == 0) { issue(nx, st2); compute(st0, it, lb[0], db[0]); }
    else if constexpr (S == 1) { issue(nx, st0); compute(st1, it, lb[1], db[1]); }
    else { issue(nx, st1); compute(st2, it, lb[2], db[2]); }
  };
  issue(0, st0);
  load_ld(0, std::integral_constant<int, 0>{});
  issue(min(1, niter - 1), st1);
  // Straight-line loop body (a conditional step would make the compiler's tracking of the loads
  // in flight conservative at the loop head); the 0-2 steps past the last tile are masked out.
  for (int it = 0; it < niter; it += 3) {
    step(std::integral_constant<int, 0>{}, it);
    step(std::integral_constant<int, 1>{}, it + 1);
    step(std::integral_constant<int, 2>{}, it + 2);
  }
  wait_vmcnt<0>();

  const float sc = 1.f / sqrtf((float)DH);
  // the row indices pass through an empty asm so that the epilogue's addresses and loads are formed
  // here, not hoisted above the query loop where they would hold registers the loop needs
  int kk2[JN];
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    kk2[j] = kw + 16 * j + c16;
    asm volatile("" : "+v"(kk2[j]));
  }
#pragma unroll
  for (int j = 0; j < JN; ++j) {
    const int kk = kk2[j];
    const int key = min(kk, T - 1);
    const int64_t n = (int64_t)b * T + key;
    if (kk < T) {
      bf16* dvr = dv + n * lddv + (int64_t)hk * DH + 4 * g;
#pragma unroll
      for (int t = 0; t < 8; ++t) fa_store4(dvr + 16 * t, dva[j][t], 1.f);
    }
    // dk^ -> dk through the backward of the key's QK-norm and RoPE
    fa_norm_rope_bwd(dka[j], sc, kraw + n * lddv + (int64_t)hk * DH, cs + (int64_t)key * (DH / 2),
                     rk[n * Hkv + hk], dk + n * lddv + (int64_t)hk * DH, g, kk < T);
  }
}

// ------------------------------------------------------------------ backward: dQ
// Block: one (b, h) and 128 queries, wave w the 32 queries q0 + 32 w .. (Q and dO in registers as
// `second` operands). Per 64-key tile up to the diagonal: S^T = K Q^T and dP^T = V dO^T (lane:
// query column, 4 key rows), dS^T = P^T (dP^T - Delta); dQ^T += K^T dS^T with K^T from transpose
// reads. Delta = rowsum(dO * O) of the block's queries is formed here from the dO rows the waves
// hold and the O rows (same layout as dO), used, and written to delta for the dK/dV kernel.
// The epilogue scales dQ^ by 1/sqrt(DH) and takes it through the backward of the queries'
// QK-norm and RoPE: qraw (the raw q columns of the QKV projection) and dq (their columns of its
// gradient) have row stride ldv; cs [T, 64] holds the RoPE (cos, sin), rq [N, Hq] 1 / rms(q).
__global__ void __launch_bounds__(256, 2)
fa_dq_kernel(const bf16* __restrict__ qh, const bf16* __restrict__ kh, const bf16* __restrict__ v, int64_t ldv,
             const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ lse,
             float* __restrict__ delta, int64_t ldl, const bf16* __restrict__ qraw, const float2* __restrict__ cs,
             const float* __restrict__ rq, bf16* __restrict__ dq, int B, int T, int Hq, int Hkv) {
  constexpr int DH = 128, STAGE = 2 * 64 * 256;
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE];
  const int nqb = (T + 127) / 128;
  const FaBlock fb = fa_block(B, Hq, Hkv, nqb);
  const int b = fb.b, h = fb.h, hk = fb.hk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, c16 = lane & 15;
  const int q0 = fb.blk * 128, qw = q0 + wave * 32;
  const float sl2 = kFaLog2e / sqrtf((float)DH);

  u32x4 qf[2][4], of[2][4];
  float l2[2], dl[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = min(qw + 16 * j + c16, T - 1);
    const int64_t off = (((int64_t)b * T + q) * Hq + h) * DH + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qf[j][c] = *reinterpret_cast<const u32x4*>(qh + off + 32 * c);
      of[j][c] = *reinterpret_cast<const u32x4*>(dO + off + 32 * c);
    }
    l2[j] = lse[((int64_t)b * Hq + h) * ldl + q] * kFaLog2e;
    // Delta = rowsum(dO * O) of the query, over the 4 lanes g that hold its row (written for the
    // dK/dV kernel, which runs after this one)
    float dsum = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float o8[8];
      Vec8<bf16>::load(O + off + 32 * c, o8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = of[j][c][w];
        dsum += __uint_as_float(u << 16) * o8[2 * w] + __uint_as_float(u & 0xffff0000u) * o8[2 * w + 1];
      }
    }
    dsum += __shfl_xor(dsum, 16, 64);
    dsum += __shfl_xor(dsum, 32, 64);
    dl[j] = dsum;
    if (g == 0 && qw + 16 * j + c16 < T) delta[((int64_t)b * Hq + h) * ldl + q] = dsum;
  }
  const bf16* kb = kh + ((int64_t)b * T * Hkv + hk) * DH;
  const bf16* vb = v + (int64_t)b * T * ldv + (int64_t)hk * DH;
  const int64_t ldk = (int64_t)Hkv * DH;
  auto issue = [&](int kt, unsigned char* s) __attribute__((always_inline)) {
    fa_issue<64>(kb, ldk, kt * 64, T, s, wave, lane);
    fa_issue<64>(vb, ldv, kt * 64, T, s + 64 * 256, wave, lane);
  };
  floatx4 dqa[8][2];
#pragma unroll
  for (int t = 0; t < 8; ++t) dqa[t][0] = dqa[t][1] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const unsigned char* sK, int kt) __attribute__((always_inline)) {
    const unsigned char* sV = sK + 64 * 256;
    const int k0 = kt * 64;
    floatx4 s[4][2], dp[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i][0] = s[i][1] = dp[i][0] = dp[i][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 ka = fa_rfrag(sK, 16 * i + c16, 4 * c + g);
        const u32x4 va = fa_rfrag(sV, 16 * i + c16, 4 * c + g);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          s[i][j] = fa_mma(s[i][j], ka, qf[j][c]);
          dp[i][j] = fa_mma(dp[i][j], va, of[j][c]);
        }
      }
    }
    // key k0 + 4 g + (16 i + r) is visible to query q iff 16 i + r <= min(q, T - 1) - k0 - 4 g: one
    // compare against a constant per element (a mask-free branch for the tiles below the diagonal,
    // as in the other two kernels, makes this one spill inside the loop at 2 waves per SIMD)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int lim = min(qw + 16 * j + c16, T - 1) - k0 - 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(s[i][j][r] * sl2 - l2[j]);
          dp[i][j][r] = 16 * i + r <= lim ? p * (dp[i][j][r] - dl[j]) : 0.f;
        }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      u32x4 ds[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) ds[j] = fa_operand(dp[2 * pr][j], dp[2 * pr + 1][j]);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x4 kt_ = fa_tfrag(sK, 32 * pr, 16 * t, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) dqa[t][j] = fa_mma(dqa[t][j], kt_, ds[j]);
      }
    }
  };

  // tile kt in stage kt % 2; each step waits for its tile, then refills the other stage (read by
  // the previous step, which every wave has finished at the barrier) with tile kt + 1
  const int nkt = min(q0 + 127, T - 1) / 64 + 1;
  auto step = [&](auto si, int kt) __attribute__((always_inline)) {
    constexpr int S = decltype(si)::value;
    wait_vmcnt<0>();
    asm volatile("s_barrier" ::: "memory");
    if constexpr (S == 0) { issue(min(kt + 1, nkt - 1), st1); compute(st0, kt); }
    else { issue(min(kt + 1, nkt - 1), st0); compute(st1, kt); }
  };
  // Straight-line loop body (a conditional step would make the compiler's tracking of the loads
  // in flight conservative at the loop head). A step past the last tile recomputes nothing: its
  // keys lie beyond every query of the block (or beyond T), so the causal mask clears them.
  issue(0, st0);
  for (int kt = 0; kt < nkt; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    step(std::integral_constant<int, 1>{}, kt + 1);
  }
  wait_vmcnt<0>();

  const float sc = 1.f / sqrtf((float)DH);
  // the row indices pass through an empty asm so that the epilogue's addresses and loads are formed
  // here, not hoisted above the K loop where they would hold registers the loop needs
  int qq2[2] = {qw + c16, qw + 16 + c16};
  asm volatile("" : "+v"(qq2[0]), "+v"(qq2[1]));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qq = qq2[j];
    const int q = min(qq, T - 1);
    const int64_t n = (int64_t)b * T + q;
    floatx4 a[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) a[t] = dqa[t][j];
    // dq^ -> dq through the backward of the query's QK-norm and RoPE
    fa_norm_rope_bwd(a, sc, qraw + n * ldv + (int64_t)h * DH, cs + (int64_t)q * (DH / 2), rq[n * Hq + h],
                     dq + n * ldv + (int64_t)h * DH, g, qq < T);
  }
}

}  // namespace
}  // namespace ll
