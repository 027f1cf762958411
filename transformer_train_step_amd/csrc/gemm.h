// MFMA GEMM for gfx950:  C[m, n] = sum_k A[m, k] * B[n, k]  (both operands K-contiguous, "NT"),
// followed by a fused epilogue on the fp32 accumulator tile.
//
// One kernel template serves the three operand types of the training step:
//   fp32  -> v_mfma_f32_16x16x4_f32                      (tiny fp32 configuration)
//   bf16  -> v_mfma_f32_16x16x32_bf16                    (attention projections, LM head)
//   e4m3  -> v_mfma_scale_f32_16x16x128_f8f6f4, unit scales (the MLP GEMMs)
// The K loop moves 128 bytes of K per tile row whatever the type (64 bf16, 128 e4m3, 32 fp32):
// global -> registers -> LDS (16-byte chunks, XOR-swizzled so the fragment reads of 16 rows hit
// distinct banks), double-buffered with one barrier per K tile. Each lane feeds the MFMA 32
// contiguous bytes of its row per K tile; the MFMA sums over K in a lane order that is the same
// for both operands, so any K permutation inside the tile is harmless.
//
// The MFMA's first operand is the B tile (rows n) and its second the A tile (rows m), so the
// 16x16 fp32 result leaves each lane with 4 consecutive n of one m. The accumulator tile is
// staged through LDS in slabs of 64 rows and the epilogue functor then sees 8 consecutive
// columns of one row per thread (16-byte coalesced stores, row reductions across 16 lanes).
#pragma once
#include <string>

#include "common.h"

namespace ll {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int intx8 __attribute__((ext_vector_type(8)));

template <class ET> struct Mma;
template <> struct Mma<float> {
  __device__ __forceinline__ static void run(floatx4& acc, const uint32_t (&a)[8], const uint32_t (&b)[8]) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[s]), __uint_as_float(b[s]), acc, 0, 0, 0);
  }
};
template <> struct Mma<bf16> {
  __device__ __forceinline__ static void run(floatx4& acc, const uint32_t (&a)[8], const uint32_t (&b)[8]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 ua = make_uint4(a[4 * s], a[4 * s + 1], a[4 * s + 2], a[4 * s + 3]);
      uint4 ub = make_uint4(b[4 * s], b[4 * s + 1], b[4 * s + 2], b[4 * s + 3]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ua),
                                                     __builtin_bit_cast(bf16x8_t, ub), acc, 0, 0, 0);
    }
  }
};
template <> struct Mma<fp8> {
  __device__ __forceinline__ static void run(floatx4& acc, const uint32_t (&a)[8], const uint32_t (&b)[8]) {
    intx8 va, vb;
#pragma unroll
    for (int i = 0; i < 8; ++i) { va[i] = (int)a[i]; vb[i] = (int)b[i]; }
    // format 0 = e4m3 for both operands; E8M0 block scales 127 = 2^0
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
  }
};

enum EpiKind { kEpiPlain = 0, kEpiAmax = 1, kEpiRowLse = 2 };

constexpr int kGemmThreads = 256;
constexpr int kSlabRows = 64;

template <int BM, int BN>
struct GemmSmem {
  static constexpr int kOperand = 2 * (BM + BN) * 128;              // bytes, 2 stages
  static constexpr int kSlab = kSlabRows * (BN + 4) * 4;            // fp32 slab + pad
  static constexpr int kBytes = kOperand > kSlab ? kOperand : kSlab;
};

template <class ET, int BM, int BN, class Epi>
__global__ void __launch_bounds__(kGemmThreads)
gemm_nt_kernel(const ET* __restrict__ A, int64_t lda, const ET* __restrict__ B, int64_t ldb,
               int M, int N, int K, Epi epi) {
  constexpr int WN = 2;                        // 4 waves: 2 x 2
  constexpr int TM = BM / 2, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KE = 128 / (int)sizeof(ET);    // K elements per tile
  constexpr int CA = BM * 8 / kGemmThreads, CB = BN * 8 / kGemmThreads;
  static_assert(CA >= 1 && CB >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) unsigned char smem[GemmSmem<BM, BN>::kBytes];
  uint4* sA = reinterpret_cast<uint4*>(smem);              // [2][BM][8]
  uint4* sB = sA + 2 * BM * 8;                              // [2][BN][8]

  const int nbm = (int)cdiv(M, BM), nbn = (int)cdiv(N, BN);
  const int nb = nbm * nbn;
  int b = xcd_remap(blockIdx.x, nb);
  constexpr int G = 8;                                      // tile rows per L2 group
  const int grp = b / (G * nbn), first = grp * G;
  const int gs = min(nbm - first, G);
  const int bm = first + (b % (G * nbn)) % gs, bn = (b % (G * nbn)) / gs;
  const int m0 = bm * BM, n0 = bn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const char* Ab = reinterpret_cast<const char*>(A);
  const char* Bb = reinterpret_cast<const char*>(B);
  const int64_t ldab = lda * (int64_t)sizeof(ET), ldbb = ldb * (int64_t)sizeof(ET);
  uint4 ra[CA], rb[CB];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * kGemmThreads, row = c >> 3, col = c & 7;
      const int gm = m0 + row;
      ra[i] = gm < M ? *reinterpret_cast<const uint4*>(Ab + gm * ldab + (int64_t)kt * 128 + col * 16)
                     : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * kGemmThreads, row = c >> 3, col = c & 7;
      const int gn = n0 + row;
      rb[i] = gn < N ? *reinterpret_cast<const uint4*>(Bb + gn * ldbb + (int64_t)kt * 128 + col * 16)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * kGemmThreads, row = c >> 3, col = c & 7;
      sA[(st * BM + row) * 8 + (col ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * kGemmThreads, row = c >> 3, col = c & 7;
      sB[(st * BN + row) * 8 + (col ^ (row & 7))] = rb[i];
    }
  };

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / KE;
  const int g = lane >> 4, r16 = lane & 15;
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    uint32_t bf[FN][8];
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int row = wn * TN + i * 16 + r16;
      const uint4 lo = sB[(st * BN + row) * 8 + ((2 * g) ^ (row & 7))];
      const uint4 hi = sB[(st * BN + row) * 8 + ((2 * g + 1) ^ (row & 7))];
      bf[i][0] = lo.x; bf[i][1] = lo.y; bf[i][2] = lo.z; bf[i][3] = lo.w;
      bf[i][4] = hi.x; bf[i][5] = hi.y; bf[i][6] = hi.z; bf[i][7] = hi.w;
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int row = wm * TM + j * 16 + r16;
      const uint4 lo = sA[(st * BM + row) * 8 + ((2 * g) ^ (row & 7))];
      const uint4 hi = sA[(st * BM + row) * 8 + ((2 * g + 1) ^ (row & 7))];
      const uint32_t af[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int i = 0; i < FN; ++i) Mma<ET>::run(acc[i][j], bf[i], af);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue: accumulator -> LDS slab (64 rows) -> functor on row segments
  float* slab = reinterpret_cast<float*>(smem);
  constexpr int LDS_LD = BN + 4;
  constexpr int SEGS = BN / 8;                              // 8-column segments per row
  constexpr int ROWS_PER_PASS = kGemmThreads / SEGS;
  float red_amax = 0.f;
#pragma unroll 1
  for (int s0 = 0; s0 < BM; s0 += kSlabRows) {
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int rloc = wm * TM + j * 16 + r16 - s0;
      if (rloc >= 0 && rloc < kSlabRows) {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          const int c = wn * TN + i * 16 + 4 * g;
          *reinterpret_cast<floatx4*>(slab + rloc * LDS_LD + c) = acc[i][j];
        }
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int p = 0; p < kSlabRows; p += ROWS_PER_PASS) {
      const int rloc = p + tid / SEGS, seg = tid % SEGS;
      const int m = m0 + s0 + rloc, n = n0 + seg * 8;
      float v[8];
      const float4 x0 = *reinterpret_cast<const float4*>(slab + rloc * LDS_LD + seg * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(slab + rloc * LDS_LD + seg * 8 + 4);
      v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w; v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
      const bool ok = (m < M) && (n < N);
      if constexpr (Epi::kKind == kEpiPlain) {
        if (ok) epi.seg(m, n, v);
      } else if constexpr (Epi::kKind == kEpiAmax) {
        if (ok) red_amax = fmaxf(red_amax, epi.seg(m, n, v));
      } else {
        float mx = -INFINITY, se = 0.f;
        if (ok) epi.seg(m, n, v, mx, se);
        // combine the SEGS (<= 16) segments of this row: lanes tid % SEGS are consecutive
#pragma unroll
        for (int o = 1; o < SEGS && o < 64; o <<= 1) {
          const float om = __shfl_xor(mx, o, 64), os = __shfl_xor(se, o, 64);
          const float nm = fmaxf(mx, om);
          se = (nm == -INFINITY) ? 0.f : se * __expf(mx - nm) + os * __expf(om - nm);
          mx = nm;
        }
        if (seg == 0 && m < M) epi.row(m, bn, mx, se);
      }
    }
    __syncthreads();
  }
  if constexpr (Epi::kKind == kEpiAmax) {
    red_amax = wave_max(red_amax);
    if (lane == 0) atomic_max_nonneg(epi.amax, red_amax);
  }
}

// ------------------------------------------------------------------ epilogue functors
// Dequantisation factor of an FP8 GEMM (product of the operands' inverse scales), 1 otherwise.
struct Deq {
  const float* ia;
  const float* ib;
  __device__ __forceinline__ float apply(float acc) const { return ia ? (acc * *ia) * *ib : acc; }
};

// C = round(deq(acc))
template <class OutT> struct EpiStore {
  static constexpr const char* kName = "store";
  static constexpr int kKind = kEpiPlain;
  OutT* C; int64_t ldc; Deq dq;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = dq.apply(v[k]);
    Vec8<OutT>::store(C + (int64_t)m * ldc + n, v);
  }
};

// t = round(deq(acc)); branch[m, n] = t (optional); out = round(x + a * t)
template <class T> struct EpiResidual {
  static constexpr const char* kName = "residual";
  static constexpr int kKind = kEpiPlain;
  T* out; const T* x; T* branch; int64_t ld; const float* a; Deq dq;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
    const int64_t o = (int64_t)m * ld + n;
    float xv[8];
    Vec8<T>::load(x + o, xv);
    const float s = *a;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = Elem<T>::rnd(dq.apply(v[k]));
    if (branch) Vec8<T>::store(branch + o, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = xv[k] + s * v[k];
    Vec8<T>::store(out + o, v);
  }
};

// u = round(deq(acc)); r = round(relu(u)^2); stores u and r; returns max |r|
template <class T> struct EpiRelu2 {
  static constexpr const char* kName = "relu2";
  static constexpr int kKind = kEpiAmax;
  T* u; T* r; int64_t ld; Deq dq; float* amax;
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8]) const {
    const int64_t o = (int64_t)m * ld + n;
    float rr[8], mx = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = Elem<T>::rnd(dq.apply(v[k]));
      const float p = fmaxf(v[k], 0.f);
      rr[k] = Elem<T>::rnd(p * p);
      mx = fmaxf(mx, rr[k]);
    }
    Vec8<T>::store(u + o, v);
    Vec8<T>::store(r + o, rr);
    return mx;
  }
};

// dr = round(deq(acc)); du = round(dr * 2 relu(u)); stores du; returns max |du|
template <class T> struct EpiRelu2Bwd {
  static constexpr const char* kName = "relu2_bwd";
  static constexpr int kKind = kEpiAmax;
  T* du; const T* u; int64_t ld; Deq dq; float* amax;
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8]) const {
    const int64_t o = (int64_t)m * ld + n;
    float uv[8], mx = 0.f;
    Vec8<T>::load(u + o, uv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dr = Elem<T>::rnd(dq.apply(v[k]));
      v[k] = Elem<T>::rnd(dr * (2.f * fmaxf(uv[k], 0.f)));
      mx = fmaxf(mx, fabsf(v[k]));
    }
    Vec8<T>::store(du + o, v);
    return mx;
  }
};

// qkv = round(acc); on the v columns (n >= vcol0) of value-embedding layers:
// v = round(v + table[ids[m], n - vcol0])
template <class T> struct EpiQkv {
  static constexpr const char* kName = "qkv";
  static constexpr int kKind = kEpiPlain;
  T* C; int64_t ldc; const T* table; int64_t ldt; const int32_t* ids; int vcol0;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = Elem<T>::rnd(v[k]);
    if (table && n >= vcol0) {
      float e[8];
      Vec8<T>::load(table + (int64_t)ids[m] * ldt + (n - vcol0), e);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += e[k];
    }
    Vec8<T>::store(C + (int64_t)m * ldc + n, v);
  }
};

// C32 = (accumulate ? C32 : 0) + acc   (fp32 accumulation across calls)
struct EpiAcc32 {
  static constexpr const char* kName = "acc32";
  static constexpr int kKind = kEpiPlain;
  float* C; int64_t ldc; int accumulate;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
    float* p = C + (int64_t)m * ldc + n;
    if (accumulate) {
      float o[8];
      Vec8<float>::load(p, o);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += o[k];
    }
    Vec8<float>::store(p, v);
  }
};

// ------------------------------------------------------------------ launcher
template <class ET> struct OpName;
template <> struct OpName<float> { static constexpr const char* s = "f32"; };
template <> struct OpName<bf16> { static constexpr const char* s = "bf16"; };
template <> struct OpName<fp8> { static constexpr const char* s = "e4m3"; };

// trace tag of a GEMM instantiation: "gemm_<operand type>_<epilogue>"
template <class ET, class Epi>
inline const char* gemm_tag() {
  static const std::string t = std::string("gemm_") + OpName<ET>::s + "_" + Epi::kName;
  return t.c_str();
}

template <class ET, class Epi>
inline hipError_t launch_gemm_nt(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N,
                                 int K, const Epi& epi, hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  if (M <= 0 || N <= 0) return hipSuccess;
  const int64_t nb = cdiv(M, BM) * cdiv(N, BN);
  const char* tag = gemm_tag<ET, Epi>();
  LL_LAUNCH_MNK(tag, M, N, K, (gemm_nt_kernel<ET, BM, BN, Epi>), dim3((unsigned)nb), dim3(kGemmThreads), 0, s,
                     A, lda, B, ldb, M, N, K, epi);
  return hipGetLastError();
}

}  // namespace
}  // namespace ll
