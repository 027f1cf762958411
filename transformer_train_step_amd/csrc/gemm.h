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

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzles. K-major tiles (rows of 128 B): chunk ^ ((row >> 1) & 7) puts the 16
// rows of a fragment read on 16 distinct (bank half, chunk) slots. MN-major tiles (k rows of
// ROWS elements): chunk ^ mn_swz(k) spreads the 4 k-rows of one transpose read over distinct
// chunk pairs, and alternating 16-row k groups over the two halves of the bank window.
__device__ __forceinline__ int kmaj_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int mn_swz(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 4) & 1)); }

// Issue the direct global->LDS loads of one operand tile for K tile kt (this wave's share).
//   K-major: element (r, k) at g[r * ld + k]; tile = ROWS rows x 128 B.
//   MN-major: element (r, k) at g[k * ld + r]; tile = KE k-rows x ROWS elements; k-rows at or
//   beyond kvalid read the zero row instead (the K tail of a token-contracted GEMM).
// Rows/columns past rmax are clamped to valid memory; they only feed outputs that are not stored.
template <class ET, bool KMAJ, int ROWS, int NW>
__device__ __forceinline__ void issue_tile(const char* g, int64_t ldb, int r0, int rmax, int kt, int kvalid,
                                           const char* zrow, unsigned char* lds_op, int wave, int lane) {
  constexpr int TILE = ROWS * 128;
  constexpr int NI = TILE / 1024 / NW;
  static_assert(NI >= 1 && NI * 1024 * NW == TILE, "tile must split evenly over the waves");
  constexpr int KE = 128 / (int)sizeof(ET);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int base = (wave * NI + i) * 1024;
    const char* src;
    if constexpr (KMAJ) {
      const int row = base / 128 + (lane >> 3);
      const int logical = (lane & 7) ^ kmaj_swz(row);
      const int gr = min(r0 + row, rmax - 1);
      src = g + gr * ldb + (int64_t)kt * 128 + logical * 16;
    } else {
      constexpr int CPR = ROWS * (int)sizeof(ET) / 16;
      const int sidx = base / 16 + lane;
      const int krow = sidx / CPR;
      const int logical = (sidx % CPR) ^ mn_swz(krow);
      const int k = kt * KE + krow;
      const int col = min(r0 + logical * (16 / (int)sizeof(ET)), rmax - 16 / (int)sizeof(ET));
      src = k < kvalid ? g + (int64_t)k * ldb + (int64_t)col * (int)sizeof(ET) : zrow;
    }
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds_op + base), 16, 0, 0);
  }
}

// Fragment of 16 rows (K-major) or 16 columns (MN-major) starting at f0: 32 bytes per lane,
// lane (index l & 15, group g = l >> 4) holds K elements [16g, 16g + 16) of the 64 bf16 (or the
// type's equivalent 32 bytes) of this K tile, in the same order for both layouts.
template <bool KMAJ, int ROWS>
__device__ __forceinline__ void read_frag(const unsigned char* t, int f0, int lane, uint32_t (&f)[8]) {
  const int g = lane >> 4;
  if constexpr (KMAJ) {
    const int row = f0 + (lane & 15), sw = kmaj_swz(row);
    const uint4 lo = *reinterpret_cast<const uint4*>(t + row * 128 + ((2 * g) ^ sw) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(t + row * 128 + ((2 * g + 1) ^ sw) * 16);
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w; f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  } else {
    // bf16 only: four ds_read_b64_tr_b16, each giving this lane's column at 4 consecutive k
    constexpr int RB = ROWS * 2;
    const int li = lane & 15, r = li >> 2, j = li & 3;
    const int col = f0 + 4 * j;
    const int chunk = col >> 3, within = (col & 7) * 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {                  // q = 2 * substep + half
      const int k = 16 * g + 4 * q + r;
      const unsigned char* a = t + k * RB + ((chunk ^ mn_swz(k)) * 16) + within;
      const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(a));
      const uint2 u = __builtin_bit_cast(uint2, v);
      f[2 * q] = u.x;
      f[2 * q + 1] = u.y;
    }
  }
}

// C[m, n] = sum_k A(m, k) B(n, k), A(m, k) = AK ? A[m * lda + k] : A[k * lda + m] (likewise B).
// WGM x WGN waves; wave tile (BM/WGM) x (BN/WGN) in 16 x 16 MFMA fragments.
template <class ET, int BM, int BN, int WGM, int WGN, bool AK, bool BK, class Epi>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_kernel(const ET* __restrict__ A, int64_t lda, const ET* __restrict__ B, int64_t ldb, int M, int N, int K,
            const ET* __restrict__ zrow, Epi epi) {
  static_assert((AK && BK) || sizeof(ET) == 2, "MN-major operands are bf16 only");
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int WN = WGN;
  constexpr int TM = BM / WGM, TN = BN / WGN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KE = 128 / (int)sizeof(ET);
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) unsigned char smem[GemmSmem<BM, BN>::kBytes];

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
  const char* zb = reinterpret_cast<const char*>(zrow);
  const int64_t ldab = lda * (int64_t)sizeof(ET), ldbb = ldb * (int64_t)sizeof(ET);

  auto issue = [&](int kt, int st) {
    unsigned char* sa = smem + st * STAGE;
    issue_tile<ET, AK, BM, NW>(Ab, ldab, m0, M, kt, K, zb, sa, wave, lane);
    issue_tile<ET, BK, BN, NW>(Bb, ldbb, n0, N, kt, K, zb, sa + BM * 128, wave, lane);
  };

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)cdiv(K, KE);
  if (nk > 0) issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, st ^ 1);
    const unsigned char* sa = smem + st * STAGE;
    const unsigned char* sb = sa + BM * 128;
    uint32_t bf[FN][8];
#pragma unroll
    for (int i = 0; i < FN; ++i) read_frag<BK, BN>(sb, wn * TN + i * 16, lane, bf[i]);
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      uint32_t af[8];
      read_frag<AK, BM>(sa, wm * TM + j * 16, lane, af);
#pragma unroll
      for (int i = 0; i < FN; ++i) Mma<ET>::run(acc[i][j], bf[i], af);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  const int g = lane >> 4, r16 = lane & 15;
  // ---------------- epilogue: accumulator -> LDS slab (64 rows) -> functor on row segments
  float* slab = reinterpret_cast<float*>(smem);
  constexpr int LDS_LD = BN + 4;
  constexpr int SEGS = BN / 8;                              // 8-column segments per row
  constexpr int ROWS_PER_PASS = NT / SEGS;
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

// Operand layouts of a GEMM call: K-major ("row m holds its K elements contiguously") or MN-major.
struct GemmOps {
  bool a_kmajor = true, b_kmajor = true;
  const void* zrow = nullptr;       // >= 16 zero bytes: K-tail rows of MN-major operands
};

template <class ET, int BM, int BN, int WGM, int WGN, class Epi>
inline hipError_t launch_gemm_cfg(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                  const Epi& epi, const GemmOps& o, hipStream_t s) {
  const int64_t nb = cdiv(M, BM) * cdiv(N, BN);
  const char* tag = gemm_tag<ET, Epi>();
  const ET* z = static_cast<const ET*>(o.zrow);
  constexpr int NT = 64 * WGM * WGN;
  if constexpr (sizeof(ET) == 2) {
    if (!o.a_kmajor && !o.b_kmajor) {
      LL_LAUNCH_MNK(tag, M, N, K, (gemm_kernel<ET, BM, BN, WGM, WGN, false, false, Epi>), dim3((unsigned)nb), dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi);
      return hipGetLastError();
    }
    if (!o.a_kmajor) {
      LL_LAUNCH_MNK(tag, M, N, K, (gemm_kernel<ET, BM, BN, WGM, WGN, false, true, Epi>), dim3((unsigned)nb), dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi);
      return hipGetLastError();
    }
    if (!o.b_kmajor) {
      LL_LAUNCH_MNK(tag, M, N, K, (gemm_kernel<ET, BM, BN, WGM, WGN, true, false, Epi>), dim3((unsigned)nb), dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi);
      return hipGetLastError();
    }
  }
  LL_LAUNCH_MNK(tag, M, N, K, (gemm_kernel<ET, BM, BN, WGM, WGN, true, true, Epi>), dim3((unsigned)nb), dim3(NT), 0, s,
                A, lda, B, ldb, M, N, K, z, epi);
  return hipGetLastError();
}

// Block-tile configurations: 1 = 128 x 128 (4 waves), 2 = 256 x 256 (4 waves), 3 = 256 x 256
// (8 waves, 2 x 4), 4 = 256 x 256 (8 waves, 4 x 2); 0 = automatic (gemm_config_override()).

template <class ET, class Epi>
inline hipError_t launch_gemm_with(int cfg, const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                   const Epi& epi, const GemmOps& o, hipStream_t s) {
  switch (cfg) {
    case 1: return launch_gemm_cfg<ET, 128, 128, 2, 2>(A, lda, B, ldb, M, N, K, epi, o, s);
    case 2: return launch_gemm_cfg<ET, 256, 256, 2, 2>(A, lda, B, ldb, M, N, K, epi, o, s);
    case 3: return launch_gemm_cfg<ET, 256, 256, 2, 4>(A, lda, B, ldb, M, N, K, epi, o, s);
    default: return launch_gemm_cfg<ET, 256, 256, 4, 2>(A, lda, B, ldb, M, N, K, epi, o, s);
  }
}

// Picks the block tile from the wave quantisation on 256 CUs: 256 x 256 with 8 waves (measured
// ~15% faster per FLOP than 128 x 128 on the layer's shapes) unless its last wave of blocks leaves
// so many CUs idle that 128 x 128 finishes first. Requirements (checked by the callers): K a multiple of the K tile for K-major
// operands (64 bf16, 128 e4m3, 32 fp32) or rows zero-padded to it; MN-major operands bf16 with M
// (or N) a multiple of 8 and >= 8, and a zero row for the K tail; N a multiple of 8.
template <class ET, class Epi>
inline hipError_t launch_gemm(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                              const Epi& epi, const GemmOps& o, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  int cfg = gemm_config_override();
  if (cfg == 0) {
    const int64_t t256 = cdiv(M, 256) * cdiv(N, 256), t128 = cdiv(M, 128) * cdiv(N, 128);
    const double e256 = (double)t256 / (double)(cdiv(t256, 256) * 256);
    const double e128 = 0.85 * (double)t128 / (double)(cdiv(t128, 256) * 256);
    cfg = e256 >= e128 ? 3 : 1;
  }
  return launch_gemm_with(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
}

template <class ET, class Epi>
inline hipError_t launch_gemm_nt(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                 const Epi& epi, hipStream_t s) {
  return launch_gemm(A, lda, B, ldb, M, N, K, epi, GemmOps{}, s);
}

}  // namespace
}  // namespace ll
