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
#include <type_traits>

#include "common.h"

namespace ll {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One 16 x 16 output fragment += first . second^T over the NC 16-byte chunks (NC = 1 or 2) of K
// that each lane holds for its row / column. Fragments stay whole 16-byte vectors from the LDS read
// to the MFMA (the vector loads then keep the LDS alias scope of the stage they read).
template <class ET> struct Mma;
template <> struct Mma<float> {
  template <int NC>
  __device__ __forceinline__ static void run(floatx4& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[c][s]), __uint_as_float(b[c][s]), acc, 0, 0, 0);
  }
  template <int NC>
  __device__ __forceinline__ static void run(floatx4& acc, const uint32_t (&a)[8], const uint32_t (&b)[8]) {
#pragma unroll
    for (int s = 0; s < 4 * NC; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[s]), __uint_as_float(b[s]), acc, 0, 0, 0);
  }
};
template <> struct Mma<bf16> {
  template <int NC>
  __device__ __forceinline__ static void run(floatx4& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[c]),
                                                     __builtin_bit_cast(bf16x8_t, b[c]), acc, 0, 0, 0);
  }
  template <int NC>
  __device__ __forceinline__ static void run(floatx4& acc, const uint32_t (&a)[8], const uint32_t (&b)[8]) {
#pragma unroll
    for (int s = 0; s < NC; ++s) {
      u32x4 ua = {a[4 * s], a[4 * s + 1], a[4 * s + 2], a[4 * s + 3]};
      u32x4 ub = {b[4 * s], b[4 * s + 1], b[4 * s + 2], b[4 * s + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ua),
                                                     __builtin_bit_cast(bf16x8_t, ub), acc, 0, 0, 0);
    }
  }
};
template <> struct Mma<fp8> {
  template <int NC>
  __device__ __forceinline__ static void run(floatx4& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
    static_assert(NC == 2, "the e4m3 MFMA takes 32 bytes of K per lane");
    const intx8 va = __builtin_bit_cast(intx8, __builtin_shufflevector(a[0], a[1], 0, 1, 2, 3, 4, 5, 6, 7));
    const intx8 vb = __builtin_bit_cast(intx8, __builtin_shufflevector(b[0], b[1], 0, 1, 2, 3, 4, 5, 6, 7));
    // format 0 = e4m3 for both operands; E8M0 block scales 127 = 2^0
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, acc, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
  }
};

enum EpiKind { kEpiPlain = 0, kEpiAmax = 1, kEpiRowSum = 2 };

constexpr int kGemmThreads = 256;
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));

// 16-byte chunk swizzles. K-major tiles (rows of KB bytes): chosen so that the fragment read of 16
// rows at one logical chunk takes no bank-conflict cycle. MN-major tiles (k rows of ROWS
// elements): chunk ^ mn_swz(k) spreads the 4 k-rows of one transpose read over distinct chunk
// pairs, and alternating 16-row k groups over the two halves of the bank window.
template <int KB>
__device__ __forceinline__ int kmaj_swz(int row) {
  // 128-byte rows: chunk bit 2 from row bit 1, chunk bit 0 from row bit 2. Measured with the LDS
  // bank-conflict counter over every XOR map of the 4 row bits: this map serves a fragment read
  // with no conflict cycle, where a map over row bits 1..3 (one distinct chunk per row pair)
  // costs 4 extra cycles per read.
  // 64-byte rows: chunk bit 1 from row bit 2 (measured the same way over all 256 maps; the former
  // (row >> 2) & 3 cost 4 extra cycles per read)
  if constexpr (KB == 128) return (((row >> 1) & 1) << 2) | ((row >> 2) & 1);
  else return ((row >> 2) & 1) << 1;
}
// 128-byte rows read as 32-row fragments (the 32x32 MFMA: lanes l and l + 32 read the same row at
// chunks two apart, rows r and r + 16 in the same instruction): the 16-row map above with chunk bit 1
// from row bit 4. Measured with the LDS bank-conflict counter to take no conflict cycle.
__device__ __forceinline__ int kmaj_swz32(int row) { return kmaj_swz<128>(row) ^ (((row >> 4) & 1) << 1); }
__device__ __forceinline__ int mn_swz(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 4) & 1)); }

// Issue the direct global->LDS loads of one operand tile for K tile kt (this wave's share).
//   K-major: element (r, k) at g[r * ld + k]; tile = ROWS rows x KB bytes.
//   MN-major: element (r, k) at g[k * ld + r]; tile = KB/es k-rows x ROWS elements; k-rows at or
//   beyond kvalid read the zero row instead (the K tail of a token-contracted GEMM).
// Rows/columns past rmax are clamped to valid memory; they only feed outputs that are not stored.
template <class ET, bool KMAJ, int ROWS, int KB, int NW, bool S32 = false>
__device__ __forceinline__ void issue_tile(const char* g, int64_t ldb, int r0, int rmax, int kt, int kvalid,
                                           const char* zrow, unsigned char* lds_op, int wave, int lane) {
  constexpr int TILE = ROWS * KB;
  constexpr int NI = TILE / 1024 / NW;
  constexpr int KE = KB / (int)sizeof(ET);
  static_assert(NI >= 1 && NI * 1024 * NW == TILE, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int base = (wave * NI + i) * 1024;
    const char* src;
    if constexpr (KMAJ) {
      constexpr int CPR = KB / 16;
      const int row = base / KB + lane / CPR;
      const int logical = (lane % CPR) ^ (S32 ? kmaj_swz32(row) : kmaj_swz<KB>(row));
      const int gr = min(r0 + row, rmax - 1);
      src = g + gr * ldb + (int64_t)kt * KB + logical * 16;
    } else {
      constexpr int CPR = ROWS * (int)sizeof(ET) / 16;
      const int sidx = base / 16 + lane;
      const int krow = sidx / CPR;
      const int logical = (sidx % CPR) ^ mn_swz(krow);
      const int k = kt * KE + krow;
      const int col = min(r0 + logical * (16 / (int)sizeof(ET)), rmax - 16 / (int)sizeof(ET));
      // address formed for every lane (k clamped to a valid row), then a select: no branch
      const char* rowp = g + (int64_t)min(k, kvalid - 1) * ldb + (int64_t)col * (int)sizeof(ET);
      src = k < kvalid ? rowp : zrow;
    }
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds_op + base), 16, 0, 0);
  }
}

// The same loads for a K-major operand with the block's base address in scalar registers:
// `gbase` = row r0 of the block tile at byte kt * KB (wave-uniform), each lane adds a 32-bit offset
// (global_load_lds with an SGPR base), rows clamped to rlast (the last valid row of the block).
// lrow / lchunk: the lane's row within one instruction's rows and its swizzled 16-byte chunk.
// With S32 the chunk map is kmaj_swz32 (32-row fragments), whose row-bit-4 term is the same for all
// lanes of one instruction (RPI = 8 rows), so it is applied as a wave-uniform XOR.
template <int ROWS, int KB, int NW, bool S32 = false>
__device__ __forceinline__ void issue_tile_sbase(const char* gbase, int lrow, int lchunk, int rlast, int ldb,
                                                 unsigned char* lds_op, int wave_s) {
  constexpr int TILE = ROWS * KB;
  constexpr int NI = TILE / 1024 / NW;
  constexpr int RPI = 1024 / KB;                           // rows per load instruction
  static_assert(NI >= 1 && NI * 1024 * NW == TILE, "tile must split evenly over the waves");
  static_assert(!S32 || KB == 128, "32-row map: 128-byte rows");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = min((wave_s * NI + i) * RPI + lrow, rlast);
    const int lc = S32 ? lchunk ^ (((((wave_s * NI + i) * RPI) >> 4) & 1) << 1) : lchunk;
    const char* src = gbase + (uint32_t)(row * ldb + (lc << 4));
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(lds_op + (wave_s * NI + i) * 1024), 16, 0, 0);
  }
}

// Fragment of 16 rows (K-major) or 16 columns (MN-major) starting at f0: KB/4 bytes per lane;
// lane (index l & 15, group g = l >> 4) holds chunks [g * KB/64, (g+1) * KB/64) of 16 bytes of
// the K tile, in the same K order for both layouts. The tile starts at byte off of the stage array
// t; each address is formed as t + (integer offset) so that every LDS read stays a direct
// derivative of its stage array (the compiler then keeps the reads apart from the direct loads
// into the other stages).
template <bool KMAJ, int ROWS, int KB>
__device__ __forceinline__ void read_frag(const unsigned char* t, int off, int f0, int lane, u32x4 (&f)[2]) {
  constexpr int NC = KB / 64;
  const int g = lane >> 4;
  if constexpr (KMAJ) {
    const int row = f0 + (lane & 15), sw = kmaj_swz<KB>(row);
#pragma unroll
    for (int c = 0; c < NC; ++c) f[c] = *reinterpret_cast<const u32x4*>(t + (off + row * KB + ((NC * g + c) ^ sw) * 16));
  } else {
    // bf16 only: ds_read_b64_tr_b16, each giving this lane's column at 4 consecutive k
    constexpr int RB = ROWS * 2;
    const int li = lane & 15, r = li >> 2, j = li & 3;
    const int col = f0 + 4 * j;
    const int chunk = col >> 3, within = (col & 7) * 2;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      u32x2 h[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int k = 8 * NC * g + 8 * c + 4 * q + r;
        const unsigned char* a = t + (off + k * RB + ((chunk ^ mn_swz(k)) * 16) + within);
        h[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                              (__attribute__((address_space(3))) shortx4*)(a)));
      }
      f[c] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3);
    }
  }
}

// Chunk C (16 bytes of K per lane, elements 8 C .. of the lane's 8 NC) of the same fragment:
// one MFMA's operand.
template <bool KMAJ, int ROWS, int KB, int C>
__device__ __forceinline__ u32x4 read_chunk(const unsigned char* t, int off, int f0, int lane) {
  constexpr int NC = KB / 64;
  const int g = lane >> 4;
  if constexpr (KMAJ) {
    const int row = f0 + (lane & 15), sw = kmaj_swz<KB>(row);
    return *reinterpret_cast<const u32x4*>(t + (off + row * KB + ((NC * g + C) ^ sw) * 16));
  } else {
    constexpr int RB = ROWS * 2;
    const int li = lane & 15, r = li >> 2, j = li & 3;
    const int col = f0 + 4 * j;
    const int chunk = col >> 3, within = (col & 7) * 2;
    u32x2 h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 8 * NC * g + 8 * C + 4 * q + r;
      const unsigned char* a = t + (off + k * RB + ((chunk ^ mn_swz(k)) * 16) + within);
      h[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (__attribute__((address_space(3))) shortx4*)(a)));
    }
    return __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3);
  }
}

// 32-row K-major fragment of 128-byte rows for the 32x32x64 e4m3 MFMA: lane l takes row
// f0 + (l & 31) and K bytes [64 C + 32 h, 64 C + 32 h + 32), h = l >> 5, as two 16-byte chunks (the
// MFMA pairs the same lanes of both operands, so only the correspondence of K positions matters).
template <int C>
__device__ __forceinline__ void read_frag32(const unsigned char* t, int off, int f0, int lane, u32x4 (&f)[2]) {
  const int row = f0 + (lane & 31), sw = kmaj_swz32(row), h = lane >> 5;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
    f[cc] = *reinterpret_cast<const u32x4*>(t + (off + row * 128 + (((4 * C + 2 * h + cc) ^ sw) * 16)));
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt fields at their no-wait maxima). Issued through the
// builtin so that the compiler's own wait insertion knows which loads have completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Instruction order of one K step for the machine scheduler (LDS returns in order): the reads
// of A(0) and B(0..2) first; then each further B(i) read three column fragments ahead of its
// MFMAs in row fragment 0, the A(1) read half-way through row fragment 0, and each later A(j + 1)
// read half-way through the MFMAs of row fragment j. MI = MFMAs per fragment pair, RA / RB = LDS
// read instructions per A / B fragment.
template <int FM, int FN, int MI, int RA, int RB>
__device__ __forceinline__ void sched_step() {
  constexpr int kMfma = 0x008, kDsRead = 0x100;
  constexpr int LA = FN < 3 ? FN : 3;
  __builtin_amdgcn_sched_group_barrier(kDsRead, RA + LA * RB, 0);
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, MI, 0);
    if (i + LA < FN) __builtin_amdgcn_sched_group_barrier(kDsRead, RB, 0);
    if (FM > 1 && i == (FN - LA > FN / 2 ? FN - LA : FN / 2)) __builtin_amdgcn_sched_group_barrier(kDsRead, RA, 0);
  }
#pragma unroll
  for (int j = 1; j < FM; ++j) {
    if (j + 1 < FM) {
      __builtin_amdgcn_sched_group_barrier(kMfma, FN * MI / 2, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, RA, 0);
      __builtin_amdgcn_sched_group_barrier(kMfma, FN * MI - FN * MI / 2, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(kMfma, FN * MI, 0);
    }
  }
}

// Instruction order for the machine scheduler: NV0 global loads first, then NRD LDS reads and
// NVM further loads spread evenly over NMF MFMAs (one read and one load per group, the MFMAs
// divided over the groups), so that the reads and loads issue between MFMAs instead of in a burst
// that the MFMAs queue behind.
template <int NMF, int NRD, int NVM, int NV0 = 0>
__device__ __forceinline__ void sched_interleave() {
  constexpr int kMfma = 0x008, kVmem = 0x010, kDsRead = 0x100;
  constexpr int G = NRD > NVM ? NRD : NVM, LO = NMF / G;
  static_assert(G >= 1 && LO >= 1, "at least one MFMA per group");
  if constexpr (NV0 > 0) __builtin_amdgcn_sched_group_barrier(kVmem, NV0, 0);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < NVM) __builtin_amdgcn_sched_group_barrier(kVmem, 1, 0);
    if (g < NRD) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    if ((g + 1) * NMF / G - g * NMF / G == LO) __builtin_amdgcn_sched_group_barrier(kMfma, LO, 0);
    else __builtin_amdgcn_sched_group_barrier(kMfma, LO + 1, 0);
  }
}

// Epilogues that read global memory at the output's position may declare `struct Pf` with
// `Pf load(int m, int n) const` and take it as a fourth argument of seg: the GEMM then issues every
// such load of a pass before staging the pass's accumulators through LDS, so that their latency is
// paid once per pass instead of once per row segment.
// Epilogues with a `prepare()` (reading per-launch scalars such as dequantisation factors into
// registers) get it called once per block before their first segment.
template <class E, class = void> struct HasPrepare : std::false_type {};
template <class E> struct HasPrepare<E, std::void_t<decltype(std::declval<E&>().prepare())>> : std::true_type {};

template <class E, class = void> struct HasPf : std::false_type { using type = char; };
template <class E> struct HasPf<E, std::void_t<typename E::Pf>> : std::true_type { using type = typename E::Pf; };

// Split-K epilogues (static constexpr bool kSplitK = true, int kchunk): block row blockIdx.y of the
// grid takes K elements [blockIdx.y kchunk, min(K, (blockIdx.y + 1) kchunk)) and the epilogue
// stores its partial sums apart from the other slices'.
template <class E, class = void> struct IsSplitK : std::false_type {};
template <class E> struct IsSplitK<E, std::void_t<decltype(E::kSplitK)>> : std::bool_constant<E::kSplitK> {};

// Two-GEMM epilogues (static constexpr bool kPair = true; EpiPair below): the grid's blocks from
// epi.skip on compute a second GEMM, whose operands and shape the epilogue carries.
template <class E, class = void> struct IsPair : std::false_type {};
template <class E> struct IsPair<E, std::void_t<decltype(E::kPair)>> : std::bool_constant<E::kPair> {};

// The same for fewer MFMAs than reads: NV0 loads first, then NMF groups each of a share of the
// NRD reads and NVM loads followed by one MFMA.
template <int NMF, int NRD, int NVM, int NV0 = 0>
__device__ __forceinline__ void sched_interleave_per_mfma() {
  static_assert(NRD <= 3 * NMF && NVM <= 3 * NMF, "at most three reads and three loads per MFMA");
  if constexpr (NV0 > 0) __builtin_amdgcn_sched_group_barrier(0x010, NV0, 0);
#pragma unroll
  for (int g = 0; g < NMF; ++g) {
    const int nv = (g + 1) * NVM / NMF - g * NVM / NMF;
    const int nr = (g + 1) * NRD / NMF - g * NRD / NMF;
    if (nv == 1) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    else if (nv == 2) __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
    else if (nv == 3) __builtin_amdgcn_sched_group_barrier(0x010, 3, 0);
    if (nr == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    else if (nr == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    else if (nr == 3) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
}

// C[m, n] = sum_k A(m, k) B(n, k), A(m, k) = AK ? A[m * lda + k] : A[k * lda + m] (likewise B).
// WGM x WGN waves; wave tile (BM/WGM) x (BN/WGN) in 16 x 16 MFMA fragments. K advances KB bytes
// per tile through an NS-stage LDS ring: tile kt + NS - 1 is in flight while tile kt is multiplied.
template <class ET, int BM, int BN, int WGM, int WGN, int KB, int NS, bool AK, bool BK, class Epi, int MODE = 0>
__global__ void __launch_bounds__(64 * WGM * WGN)
gemm_kernel(const ET* __restrict__ A, int64_t lda, const ET* __restrict__ B, int64_t ldb, int M, int N, int K,
            const ET* __restrict__ zrow, Epi epi, int G) {
  static_assert((AK && BK) || sizeof(ET) == 2, "MN-major operands are bf16 only");
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  constexpr int NW = WGM * WGN, NT = 64 * NW;
  constexpr int WN = WGN;
  constexpr int TM = BM / WGM, TN = BN / WGN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KE = KB / (int)sizeof(ET);
  constexpr int NC = KB / 64;
  constexpr int STAGE = (BM + BN) * KB;
  constexpr int NIW = STAGE / 1024 / NW;                    // load instructions per wave per tile
  // register-prefetch schedule: one wave per SIMD (4 waves, 128 x 128 each), 64-byte K tiles, 3 stages
  constexpr bool RP = (NW == 4 && NS == 3 && KB == 64 && BM == 256 && BN == 256);
  constexpr bool SP = MODE == 1 || MODE == 2;  // split-phase K loop (bf16)
  constexpr bool IL = MODE == 2;   // ... with the reads and half the loads interleaved into the MFMAs
  constexpr int NV0 = NIW / 2;     // loads issued together right after the barrier (IL, SP32)
  constexpr bool SP32 = MODE == 3; // split-phase K loop on the 32x32 MFMAs (x64 e4m3, x16 bf16), interleaved
  constexpr bool PP = MODE == 4;   // ping-pong: two wave groups alternate MFMA-only and LDS/load phases
  constexpr bool PP32 = MODE == 5; // the same on the 32x32x64 e4m3 MFMA
  constexpr bool ACC32 = SP32 || PP32;   // accumulators in the 32 x 32 fragment layout
  static_assert(!PP || (sizeof(ET) == 2 && NS == 2 && KB == 128 && AK && BK && NW == 8),
                "ping-pong loop: bf16, 2 stages, 128-byte K tiles, K-major operands, 8 waves");
  static_assert(!PP32 || (sizeof(ET) == 1 && NS == 2 && KB == 128 && AK && BK && NW == 8 && FM % 2 == 0 && FN % 2 == 0),
                "e4m3 ping-pong loop: 2 stages, 128-byte K tiles, K-major operands, 8 waves");
  static_assert(!SP32 || (sizeof(ET) <= 2 && NS == 2 && KB == 128 && AK && BK && FM % 2 == 0 && FN % 2 == 0),
                "32x32 split-phase loop: e4m3 or bf16, 2 stages, 128-byte K tiles, K-major operands");
  // One LDS array per stage: distinct objects let the compiler see that the direct loads into the
  // next stages do not alias the fragment reads of the current one (a single array indexed by
  // stage makes it wait for every load in flight before the first read of each tile).
  __shared__ __attribute__((aligned(16))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[NS > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) unsigned char st3[NS > 3 ? STAGE : 16];

  int bid = (int)blockIdx.x;
  bool second = false;
  if constexpr (IsPair<Epi>::value) {
    static_assert(!IsSplitK<Epi>::value, "a two-GEMM grid has no K slices");
    // blocks [0, tiles of the first GEMM) take it, [nb0, skip) have nothing to do (skip is a
    // multiple of 8, so block skip + j runs on XCD j % 8 like block j of a grid of its own), the
    // rest take the second GEMM
    if (bid >= (int)(cdiv(M, BM) * cdiv(N, BN))) {
      if (bid < epi.skip) return;
      bid -= epi.skip;
      A = static_cast<const ET*>(epi.a1);
      B = static_cast<const ET*>(epi.b1);
      lda = epi.lda1;
      ldb = epi.ldb1;
      M = epi.m1;
      N = epi.n1;
      K = epi.k1;
      G = epi.g1;
      second = true;
    }
  }
  const int nbm = (int)cdiv(M, BM), nbn = (int)cdiv(N, BN);
  const int nb = nbm * nbn;
  int b = xcd_remap(bid, nb);
  // Each XCD walks its share of the tiles G tile rows at a time (G > 0), or -G tile columns at a
  // time (G < 0)
  int bm, bn;
  if (G > 0) {
    const int grp = b / (G * nbn), first = grp * G;
    const int gs = min(nbm - first, G);
    bm = first + (b % (G * nbn)) % gs;
    bn = (b % (G * nbn)) / gs;
  } else {
    const int gc = -G, grp = b / (gc * nbm), first = grp * gc;
    const int gs = min(nbn - first, gc);
    bn = first + (b % (gc * nbm)) % gs;
    bm = (b % (gc * nbm)) / gs;
  }
  const int m0 = bm * BM, n0 = bn * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const char* Ab = reinterpret_cast<const char*>(A);
  const char* Bb = reinterpret_cast<const char*>(B);
  const char* zb = reinterpret_cast<const char*>(zrow);
  const int64_t ldab = lda * (int64_t)sizeof(ET), ldbb = ldb * (int64_t)sizeof(ET);
  int Kl = K;                                               // K elements of this block
  if constexpr (IsSplitK<Epi>::value) {
    const int k0 = (int)blockIdx.y * epi.kchunk;
    Kl = min(K - k0, epi.kchunk);
    Ab += AK ? (int64_t)k0 * (int64_t)sizeof(ET) : (int64_t)k0 * ldab;
    Bb += BK ? (int64_t)k0 * (int64_t)sizeof(ET) : (int64_t)k0 * ldbb;
  }

  auto stage = [&](auto si) -> unsigned char* {
    constexpr int S = decltype(si)::value;
    if constexpr (S == 0) return st0;
    else if constexpr (S == 1) return st1;
    else if constexpr (S == 2) return st2;
    else return st3;
  };
  auto issue = [&](int kt, unsigned char* sa) {
    issue_tile<ET, AK, BM, KB, NW, SP32>(Ab, ldab, m0, M, kt, Kl, zb, sa, wave, lane);
    issue_tile<ET, BK, BN, KB, NW, SP32>(Bb, ldbb, n0, N, kt, Kl, zb, sa + BM * KB, wave, lane);
  };

  floatx4 acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // SP32: 32 x 32 fragments (lane l: m = l & 31 of fragment j, n = 8 q + 4 (l >> 5) + r of fragment
  // i in element 4 q + r)
  constexpr int FM2 = ACC32 ? FM / 2 : 1, FN2 = ACC32 ? FN / 2 : 1;
  floatx16 acc32[FN2][FM2];
  if constexpr (ACC32) {
#pragma unroll
    for (int i = 0; i < FN2; ++i)
#pragma unroll
      for (int j = 0; j < FM2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc32[i][j][e] = 0.f;
  }

  const int nk = (int)cdiv(Kl, KE);
  // K tile kt lives in stage kt % NS; step<S> handles the tiles with kt % NS == S. Every step
  // issues exactly one tile (NIW loads per wave), so NS - 1 tiles are always in flight and one
  // constant wait count holds in every step: past the last tile, the loads repeat tile nk - 1
  // into stages that are not read again (an L2 hit; the drain below waits for them).
  auto step = [&](auto si, int kt) {
    constexpr int S = decltype(si)::value;
    wait_vmcnt<(NS - 2) * NIW>();                           // tile kt has landed (this wave's part)
    // Barrier without a memory fence: a fence would also wait for the loads of the later tiles.
    // Every wave's part of tile kt has landed once all waves pass it, and the MFMAs of kt - 1
    // have consumed every fragment read of the stage refilled next; the memory clobber keeps the
    // compiler from moving LDS accesses across it.
    asm volatile("s_barrier" ::: "memory");
    issue(min(kt + NS - 1, nk - 1), stage(std::integral_constant<int, (S + NS - 1) % NS>{}));
    const unsigned char* sa = stage(si);
    {
      u32x4 af[2][2], bf[FN][2];
      if constexpr (AK && BK) {
        // K-major operands: every B fragment, then A per row fragment, in the compiler's order
        // (measured faster here than the explicit interleave below)
#pragma unroll
        for (int i = 0; i < FN; ++i) read_frag<BK, BN, KB>(sa, BM * KB, wn * TN + i * 16, lane, bf[i]);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          read_frag<AK, BM, KB>(sa, 0, wm * TM + j * 16, lane, af[0]);
#pragma unroll
          for (int i = 0; i < FN; ++i) Mma<ET>::template run<NC>(acc[i][j], bf[i], af[0]);
        }
      } else {
        // Transpose-read operands: A(0) and B(0..FN-1) first, A(j + 1) ahead of the MFMAs of
        // row fragment j, interleaved with the MFMAs as sched_step lays out (LDS returns in order,
        // so the first MFMAs wait for a few fragments instead of all of them)
        read_frag<AK, BM, KB>(sa, 0, wm * TM, lane, af[0]);
#pragma unroll
        for (int i = 0; i < FN; ++i) read_frag<BK, BN, KB>(sa, BM * KB, wn * TN + i * 16, lane, bf[i]);
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          if (j + 1 < FM) read_frag<AK, BM, KB>(sa, 0, wm * TM + (j + 1) * 16, lane, af[(j + 1) & 1]);
#pragma unroll
          for (int i = 0; i < FN; ++i) Mma<ET>::template run<NC>(acc[i][j], bf[i], af[j & 1]);
        }
        sched_step<FM, FN, NC, (AK ? NC : 2 * NC), (BK ? NC : 2 * NC)>();
      }
    }
  };

  if constexpr (SP) {
    // Split-phase K loop (bf16, 2 stages, 128-byte K tiles): each K tile is two MFMA chunks. The
    // fragments of a chunk are read while the MFMAs of the other chunk run: chunk 1 of tile kt is
    // read ahead of the chunk-0 MFMAs of kt, and after the barrier in the middle of step kt chunk
    // 0 of tile kt + 1 is read ahead of the chunk-1 MFMAs of kt. The barrier also hands the stage
    // of tile kt (fully read by then) to the loads of tile kt + 2.
    static_assert(NS == 2 && KB == 128 && sizeof(ET) == 2, "split-phase loop: bf16, 2 stages, 128-byte K tiles");
    u32x4 fa[2][FM], fb[2][FN];
    auto rd = [&](const unsigned char* sa, auto ci, auto hi) __attribute__((always_inline)) {
      constexpr int C = decltype(ci)::value, H = decltype(hi)::value;
#pragma unroll
      for (int i = 0; i < FN; ++i) fb[H][i] = read_chunk<BK, BN, KB, C>(sa, BM * KB, wn * TN + i * 16, lane);
#pragma unroll
      for (int j = 0; j < FM; ++j) fa[H][j] = read_chunk<AK, BM, KB, C>(sa, 0, wm * TM + j * 16, lane);
    };
    auto mm = [&](auto hi) __attribute__((always_inline)) {
      constexpr int H = decltype(hi)::value;
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int i = 0; i < FN; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[H][i]),
                                                              __builtin_bit_cast(bf16x8_t, fa[H][j]), acc[i][j], 0, 0, 0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    auto half_step = [&](auto si, int kt) __attribute__((always_inline)) {
      constexpr int S = decltype(si)::value;
      unsigned char* sa = stage(std::integral_constant<int, S>{});
      unsigned char* sn = stage(std::integral_constant<int, S ^ 1>{});
      // sched_barrier(0) keeps each group where it is written: the reads ahead of the MFMAs they
      // overlap, the MFMAs ahead of the wait, the loads right after the barrier (the scheduler
      // would otherwise sink them to the next wait, which then waits for them too).
      // The chunk-0 fragments were read during the previous half step and have landed; waiting
      // for them here, before the next reads, keeps the count of LDS reads in flight small enough
      // (the counter holds 15) for the MFMAs below not to wait for the reads issued next.
      // With IL the reads of each phase are spread evenly over its MFMAs; after the barrier half
      // the loads go out at once (the earliest possible start for the next tile) and the other
      // half between the MFMAs. Measured per K tile: ~2,950 clocks per wave instead of ~3,300.
      wait_lgkm0();
      if constexpr (IL) __builtin_amdgcn_sched_barrier(0);
      rd(sa, I1{}, I1{});
      if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
      mm(I0{});
      if constexpr (IL) sched_interleave<FM * FN, FM + FN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lgkm0<0>();              // tile kt + 1 has landed (this wave's part), tile kt is read
      asm volatile("s_barrier" ::: "memory");
      if constexpr (IL) __builtin_amdgcn_sched_barrier(0);
      issue(min(kt + 2, nk - 1), sa);
      if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
      rd(sn, I0{}, I0{});
      if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
      mm(I1{});
      if constexpr (IL) sched_interleave<FM * FN, FM + FN, NIW - NV0, NV0>();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nk > 0) {
      issue(0, st0);
      issue(min(1, nk - 1), st1);
      wait_vmcnt<NIW>();
      asm volatile("s_barrier" ::: "memory");
      rd(st0, I0{}, I0{});
    }
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      half_step(I0{}, kt);
      half_step(I1{}, kt + 1);
    }
    if (kt < nk) half_step(I0{}, kt);
  } else if constexpr (PP || PP32) {
    // Ping-pong K loop. Waves w and w + 4 share SIMD w % 4; group 0 (waves 0-3) runs one phase
    // ahead of group 1 (waves 4-7), and every phase ends at a block barrier:
    //   phase 2t:     group 0 reads tile t's fragments (LDS -> registers); group 1 multiplies t - 1
    //   phase 2t + 1: group 0 multiplies tile t;                          group 1 reads tile t
    // so on each SIMD one wave issues only MFMAs while the other reads, and the MFMA pipe is fed
    // by a single wave from registers. Group 1 takes one extra barrier before its loop and group 0
    // one after it, so both pass the same number of barriers.
    // Each wave loads its eighth of every tile (global -> LDS) in the phase two phases before the
    // tile is first read: group 0 during its read phase of tile t - 1 (phase 2t - 2), group 1
    // during its MFMA phase of tile t - 2 (the same phase), each into the stage of tile t - 2,
    // which both groups finished reading by then; each wave waits for its own loads at the end of
    // the following phase. Past the last tile the loads repeat it into a stage that is not read
    // again.
    // bf16: 16x16x32 MFMAs, fragments [FM or FN][2 chunks of 16 bytes]; e4m3 (PP32): 32x32x64
    // MFMAs, fragments [FM2 or FN2][2 halves of K][2 chunks] (the split-phase e4m3 loop's layout).
    const bool lead = wave < 4;
    constexpr int RA = PP32 ? FM2 : FM, RB = PP32 ? FN2 : FN;
    u32x4 fa[RA][2][2], fb[RB][2][2];
    auto rd = [&](const unsigned char* sa) __attribute__((always_inline)) {
      if constexpr (PP32) {
#pragma unroll
        for (int i = 0; i < FN2; ++i) {
          read_frag32<0>(sa, BM * KB, wn * TN + i * 32, lane, fb[i][0]);
          read_frag32<1>(sa, BM * KB, wn * TN + i * 32, lane, fb[i][1]);
        }
#pragma unroll
        for (int j = 0; j < FM2; ++j) {
          read_frag32<0>(sa, 0, wm * TM + j * 32, lane, fa[j][0]);
          read_frag32<1>(sa, 0, wm * TM + j * 32, lane, fa[j][1]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < FN; ++i) {
          fb[i][0][0] = read_chunk<BK, BN, KB, 0>(sa, BM * KB, wn * TN + i * 16, lane);
          fb[i][1][0] = read_chunk<BK, BN, KB, 1>(sa, BM * KB, wn * TN + i * 16, lane);
        }
#pragma unroll
        for (int j = 0; j < FM; ++j) {
          fa[j][0][0] = read_chunk<AK, BM, KB, 0>(sa, 0, wm * TM + j * 16, lane);
          fa[j][1][0] = read_chunk<AK, BM, KB, 1>(sa, 0, wm * TM + j * 16, lane);
        }
      }
    };
    auto mm = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if constexpr (PP32) {
#pragma unroll
          for (int j = 0; j < FM2; ++j)
#pragma unroll
            for (int i = 0; i < FN2; ++i) {
              const intx8 vb = __builtin_bit_cast(intx8, __builtin_shufflevector(fb[i][c][0], fb[i][c][1], 0, 1, 2, 3, 4, 5, 6, 7));
              const intx8 va = __builtin_bit_cast(intx8, __builtin_shufflevector(fa[j][c][0], fa[j][c][1], 0, 1, 2, 3, 4, 5, 6, 7));
              // format 0 = e4m3 for both operands; E8M0 block scales 127 = 2^0
              acc32[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, va, acc32[i][j], 0, 0, 0, 0x7f7f7f7f, 0,
                                                                             0x7f7f7f7f);
            }
        } else {
#pragma unroll
          for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int i = 0; i < FN; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fb[i][c][0]),
                                                                  __builtin_bit_cast(bf16x8_t, fa[j][c][0]), acc[i][j], 0, 0, 0);
        }
      }
    };
    auto bar = []() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // loads with scalar base addresses (see issue_tile_sbase): the lane's row and chunk are its
    // only per-lane state, which keeps the register budget (128 accumulators + 96 fragment
    // registers) under 256
    const int ldai = (int)ldab, ldbi = (int)ldbb;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform: LDS targets and row offsets in SGPRs
    constexpr int CPR = KB / 16;
    const int lrow = lane / CPR, lchunk = (lane % CPR) ^ kmaj_swz<KB>(lane / CPR);
    const int alast = min(BM, M - m0) - 1, blast = min(BN, N - n0) - 1;
    auto issue = [&](int kt, unsigned char* sa) __attribute__((always_inline)) {
      // opaque copies: the per-instruction offsets are formed at each issue, not held in registers
      int lr = lrow, lc = lchunk;
      asm volatile("" : "+v"(lr), "+v"(lc));
      const int64_t ko = (int64_t)kt * KB;
      issue_tile_sbase<BM, KB, NW, PP32>(Ab + (int64_t)m0 * ldab + ko, lr, lc, alast, ldai, sa, wave_s);
      issue_tile_sbase<BN, KB, NW, PP32>(Bb + (int64_t)n0 * ldbb + ko, lr, lc, blast, ldbi, sa + BM * KB, wave_s);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // One loop per group, each without run-time conditions inside, so that the compiler knows
    // which loads are in flight at every LDS read and inserts no wait of its own.
    auto body_lead = [&](auto si, int t) __attribute__((always_inline)) {
      constexpr int S = decltype(si)::value;
      rd(stage(std::integral_constant<int, S>{}));
      __builtin_amdgcn_sched_barrier(0);
      issue(min(t + 1, nk - 1), stage(std::integral_constant<int, S ^ 1>{}));
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkm0();
      bar();
      mm();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();                                      // this wave's part of tile t + 1
      bar();
    };
    auto body_lag = [&](auto si, int t) __attribute__((always_inline)) {
      constexpr int S = decltype(si)::value;
      rd(stage(std::integral_constant<int, S>{}));
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lgkm0<0>();                                // this wave's part of tile t + 1
      bar();
      issue(min(t + 2, nk - 1), stage(std::integral_constant<int, S>{}));
      __builtin_amdgcn_sched_barrier(0);
      mm();
      __builtin_amdgcn_sched_barrier(0);
      bar();
    };
    if (nk > 0) {
      issue(0, st0);
      if (lead) {
        wait_vmcnt<0>();
        bar();                                              // tile 0 is in LDS
        int t = 0;
        for (; t + 2 <= nk; t += 2) {
          body_lead(I0{}, t);
          body_lead(I1{}, t + 1);
        }
        if (t < nk) body_lead(I0{}, t);
        bar();                                              // group 1's last MFMA phase
      } else {
        issue(min(1, nk - 1), st1);                         // group 1's part of tile 1
        wait_vmcnt<NIW>();
        bar();                                              // tile 0 is in LDS
        bar();                                              // one phase behind group 0
        int t = 0;
        for (; t + 2 <= nk; t += 2) {
          body_lag(I0{}, t);
          body_lag(I1{}, t + 1);
        }
        if (t < nk) body_lag(I0{}, t);
      }
    }
  } else if constexpr (SP32) {
    // The bf16 split-phase structure with e4m3 fragments: half C of a 128-byte K tile is one 32x32x64
    // MFMA step (64 bytes of K), so each half holds FM/2 + FN/2 fragments of 2 x 16 bytes per lane
    // (the 16x16x128 MFMA's fragments are twice as large and do not fit double-buffered).
    u32x4 fa[2][FM2][2], fb[2][FN2][2];
    auto rd = [&](const unsigned char* sa, auto ci, auto hi) __attribute__((always_inline)) {
      constexpr int C = decltype(ci)::value, H = decltype(hi)::value;
#pragma unroll
      for (int i = 0; i < FN2; ++i) read_frag32<C>(sa, BM * KB, wn * TN + i * 32, lane, fb[H][i]);
#pragma unroll
      for (int j = 0; j < FM2; ++j) read_frag32<C>(sa, 0, wm * TM + j * 32, lane, fa[H][j]);
    };
    auto mm = [&](auto hi) __attribute__((always_inline)) {
      constexpr int H = decltype(hi)::value;
#pragma unroll
      for (int j = 0; j < FM2; ++j)
#pragma unroll
        for (int i = 0; i < FN2; ++i) {
          if constexpr (sizeof(ET) == 1) {
            const intx8 vb = __builtin_bit_cast(intx8, __builtin_shufflevector(fb[H][i][0], fb[H][i][1], 0, 1, 2, 3, 4, 5, 6, 7));
            const intx8 va = __builtin_bit_cast(intx8, __builtin_shufflevector(fa[H][j][0], fa[H][j][1], 0, 1, 2, 3, 4, 5, 6, 7));
            // format 0 = e4m3 for both operands; E8M0 block scales 127 = 2^0
            acc32[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, va, acc32[i][j], 0, 0, 0, 0x7f7f7f7f, 0,
                                                                           0x7f7f7f7f);
          } else {
            // two 32x32x16 steps, each on one 16-byte chunk (8 bf16 of K) per lane
#pragma unroll
            for (int c = 0; c < 2; ++c)
              acc32[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fb[H][i][c]),
                                                                    __builtin_bit_cast(bf16x8_t, fa[H][j][c]), acc32[i][j], 0, 0, 0);
          }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    constexpr int NR = 2 * (FM2 + FN2);   // LDS reads per half
    auto half_step = [&](auto si, int kt) __attribute__((always_inline)) {
      constexpr int S = decltype(si)::value;
      unsigned char* sa = stage(std::integral_constant<int, S>{});
      unsigned char* sn = stage(std::integral_constant<int, S ^ 1>{});
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      rd(sa, I1{}, I1{});
      mm(I0{});
      sched_interleave_per_mfma<FM2 * FN2 * (sizeof(ET) == 1 ? 1 : 2), NR, 0>();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lgkm0<0>();              // tile kt + 1 has landed (this wave's part), tile kt is read
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      issue(min(kt + 2, nk - 1), sa);
      rd(sn, I0{}, I0{});
      mm(I1{});
      sched_interleave_per_mfma<FM2 * FN2 * (sizeof(ET) == 1 ? 1 : 2), NR, NIW - NV0, NV0>();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (nk > 0) {
      issue(0, st0);
      issue(min(1, nk - 1), st1);
      wait_vmcnt<NIW>();
      asm volatile("s_barrier" ::: "memory");
      rd(st0, I0{}, I0{});
    }
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      half_step(I0{}, kt);
      half_step(I1{}, kt + 1);
    }
    if (kt < nk) half_step(I0{}, kt);
  } else if constexpr (!RP) {
    if (nk > 0) {
      issue(0, st0);
      if constexpr (NS > 2) issue(min(1, nk - 1), st1);
      if constexpr (NS > 3) issue(min(2, nk - 1), st2);
    }
    for (int kb = 0; kb < nk; kb += NS) {
      step(std::integral_constant<int, 0>{}, kb);
      if (kb + 1 < nk) step(std::integral_constant<int, 1>{}, kb + 1);
      if constexpr (NS > 2) if (kb + 2 < nk) step(std::integral_constant<int, 2>{}, kb + 2);
      if constexpr (NS > 3) if (kb + 3 < nk) step(std::integral_constant<int, 3>{}, kb + 3);
    }
  } else {
    // When step kt starts, the fragments of tile kt are in registers (read during step kt - 1)
    // and tiles kt + 1, kt + 2 are loading. Step kt waits for tile kt + 1, refills the stage of
    // tile kt (its fragments are already in registers) with tile kt + 3, and reads the fragments
    // of tile kt + 1 into the other register set between its MFMAs, so the MFMA pipe does not
    // wait on LDS after the barrier. (Three LDS arrays: the compiler keeps apart the loads and
    // reads of at most three of them.)
    u32x4 fa[2][FM][2], fb[2][FN][2];
    auto stepr = [&](auto si, int kt) {
      constexpr int S = decltype(si)::value, P = S & 1, Q = P ^ 1;
      // this wave's loads of tile kt + 1 have landed and its fragment reads of tile kt are done
      wait_vmcnt_lgkm0<NIW>();
      asm volatile("s_barrier" ::: "memory");
      const unsigned char* sn = stage(std::integral_constant<int, (S + 1) % 3>{});
#pragma unroll
      for (int i = 0; i < FN; ++i) read_frag<BK, BN, KB>(sn, BM * KB, wn * TN + i * 16, lane, fb[Q][i]);
#pragma unroll
      for (int j = 0; j < FM; ++j) read_frag<AK, BM, KB>(sn, 0, wm * TM + j * 16, lane, fa[Q][j]);
      // the reads go out before this step's loads, so no load of this step is in flight behind them
      __builtin_amdgcn_sched_barrier(0);
      issue(min(kt + 3, nk - 1), stage(std::integral_constant<int, S % 3>{}));
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) Mma<ET>::template run<NC>(acc[i][j], fb[P][i], fa[P][j]);
    };
    if (nk > 0) {
      issue(0, st0);
      issue(min(1, nk - 1), st1);
      issue(min(2, nk - 1), st2);
      wait_vmcnt<2 * NIW>();                                // tile 0 has landed
      asm volatile("s_barrier" ::: "memory");
#pragma unroll
      for (int i = 0; i < FN; ++i) read_frag<BK, BN, KB>(st0, BM * KB, wn * TN + i * 16, lane, fb[0][i]);
#pragma unroll
      for (int j = 0; j < FM; ++j) read_frag<AK, BM, KB>(st0, 0, wm * TM + j * 16, lane, fa[0][j]);
    }
    int kb = 0;
    for (; kb + 6 <= nk; kb += 6) {                         // straight-line body: six full steps
      stepr(std::integral_constant<int, 0>{}, kb);
      stepr(std::integral_constant<int, 1>{}, kb + 1);
      stepr(std::integral_constant<int, 2>{}, kb + 2);
      stepr(std::integral_constant<int, 3>{}, kb + 3);
      stepr(std::integral_constant<int, 4>{}, kb + 4);
      stepr(std::integral_constant<int, 5>{}, kb + 5);
    }
    if (kb < nk) stepr(std::integral_constant<int, 0>{}, kb);
    if (kb + 1 < nk) stepr(std::integral_constant<int, 1>{}, kb + 1);
    if (kb + 2 < nk) stepr(std::integral_constant<int, 2>{}, kb + 2);
    if (kb + 3 < nk) stepr(std::integral_constant<int, 3>{}, kb + 3);
    if (kb + 4 < nk) stepr(std::integral_constant<int, 4>{}, kb + 4);
  }
  wait_vmcnt<0>();                                          // drain the repeated tail loads
  __syncthreads();
  Epi ep = epi;                                             // per-launch scalars read once
  if constexpr (IsPair<Epi>::value) ep.sel = second;
  if constexpr (HasPrepare<Epi>::value) ep.prepare();

  const int g = lane >> 4, r16 = lane & 15;
  // ---------------- epilogue: accumulators -> LDS slab -> functor on 8-column segments of rows.
  // A pass covers PR = 2 SR rows, rows [0, SR) in stage array 0 and [SR, 2 SR) in stage array 1
  // (all loads have drained). Slab rows hold BN floats with no padding; 16-byte chunk c of row r
  // sits at chunk c ^ x(r), x(r) = 2 (r & 7) + ((r >> 3) & 1), a bijection over 16 rows, so each
  // fragment write (16 rows x one chunk per 16 lanes) is conflict-free. In the read phase a lane
  // takes the chunk pair (2 s, 2 s + 1) of a row, the lower half of each 8 lanes the even chunk
  // first and the upper half the odd one, so that 16 lanes again hit 16 distinct bank slots.
  constexpr int CPR = BN / 4;                               // 16-byte chunks per slab row
  constexpr int SR = STAGE / (BN * 4) >= 64 ? 64 : STAGE / (BN * 4) >= 32 ? 32 : 16;
  constexpr int PR = 2 * SR;
  constexpr int SPR = CPR / 2;                              // 8-column segments per row
  constexpr int RPI = 64 / SPR;                             // rows per wave instruction
  static_assert(CPR >= 16 && CPR <= 64 && SR >= 16 && SR * BN * 4 <= STAGE, "slab shape");
  static_assert(BM % PR == 0 || PR > BM, "passes must tile the block rows");
  auto slab_row = [&](int r) -> float* {
    return reinterpret_cast<float*>(r < SR ? st0 : st1) + (r < SR ? r : r - SR) * BN;
  };
  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
  float red_amax = 0.f;
  constexpr bool PF = HasPf<Epi>::value;
  constexpr int ITERS = (PR + NW * RPI - 1) / (NW * RPI);   // row groups per wave and pass
  using PfT = typename HasPf<Epi>::type;
#pragma unroll 1
  for (int s0 = 0; s0 < BM; s0 += PR) {
    PfT pf[PF ? ITERS : 1];
    if constexpr (PF) {
      // this pass's global reads, issued before the accumulators go through LDS
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int p = wave * RPI + it * NW * RPI;
        const int m = m0 + s0 + p + lane / SPR, n = n0 + 8 * (lane % SPR);
        if (p < PR && s0 + p < BM && m < M && n < N) pf[it] = ep.load(m, n);
      }
    }
    if constexpr (ACC32) {
#pragma unroll
      for (int j = 0; j < FM2; ++j) {
        const int rloc = wm * TM + j * 32 + (lane & 31) - s0;
        if (rloc >= 0 && rloc < PR) {                       // uniform over each 32-row fragment
          float* row = slab_row(rloc);
          const int x = swz(rloc);
#pragma unroll
          for (int i = 0; i < FN2; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = ((wn * TN + i * 32 + 8 * q) >> 2) + (lane >> 5);
              *reinterpret_cast<floatx4*>(row + ((c ^ x) << 2)) =
                  floatx4{acc32[i][j][4 * q], acc32[i][j][4 * q + 1], acc32[i][j][4 * q + 2], acc32[i][j][4 * q + 3]};
            }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FM; ++j) {
        const int rloc = wm * TM + j * 16 + r16 - s0;
        if (rloc >= 0 && rloc < PR) {                       // uniform over each 16-row fragment
          float* row = slab_row(rloc);
          const int x = swz(rloc);
#pragma unroll
          for (int i = 0; i < FN; ++i) {
            const int c = ((wn * TN + i * 16) >> 2) + g;
            *reinterpret_cast<floatx4*>(row + ((c ^ x) << 2)) = acc[i][j];
          }
        }
      }
    }
    __syncthreads();
    auto emit = [&](int p, const PfT& f) __attribute__((always_inline)) {
      const int rloc = p + lane / SPR, sg = lane % SPR;
      const int m = m0 + s0 + rloc, n = n0 + 8 * sg;
      const float* row = slab_row(rloc);
      const int x = swz(rloc), odd = (sg >> 3) & 1;
      const floatx4 u0 = *reinterpret_cast<const floatx4*>(row + (((2 * sg + odd) ^ x) << 2));
      const floatx4 u1 = *reinterpret_cast<const floatx4*>(row + (((2 * sg + 1 - odd) ^ x) << 2));
      const floatx4 lo = odd ? u1 : u0, hi = odd ? u0 : u1;
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const bool ok = (m < M) && (n < N);
      if constexpr (Epi::kKind == kEpiPlain) {
        if constexpr (PF) {
          if (ok) ep.seg(m, n, v, f);
        } else {
          if (ok) ep.seg(m, n, v);
        }
      } else if constexpr (Epi::kKind == kEpiAmax) {
        if constexpr (PF) {
          if (ok) red_amax = fmaxf(red_amax, ep.seg(m, n, v, f));
        } else {
          if (ok) red_amax = fmaxf(red_amax, ep.seg(m, n, v));
        }
      } else {
        float se = 0.f;
        if (ok) se = ep.seg(m, n, v);
        // add the SPR segment sums of this row (consecutive lanes)
        se = group_sum<SPR>(se);
        if (sg == 0 && m < M) ep.row(m, bn, se);
      }
    };
    if constexpr (PF) {
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const int p = wave * RPI + it * NW * RPI;
        if (p < PR && s0 + p < BM) emit(p, pf[it]);
      }
    } else {
#pragma unroll 1
      for (int p = wave * RPI; p < PR && s0 + p < BM; p += NW * RPI) emit(p, pf[0]);
    }
    __syncthreads();
  }
  if constexpr (Epi::kKind == kEpiAmax) {
    // one atomic per block (one per wave serialises ~60,000 atomics on one address per GEMM)
    __shared__ float red_w[NW];
    red_amax = group_max<64>(red_amax);
    if (lane == 0) red_w[wave] = red_amax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) m = fmaxf(m, red_w[w]);
      atomic_max_nonneg(ep.amax, m);
    }
  }
}

// ------------------------------------------------------------------ epilogue functors
// The raw bytes of one 8-column segment (8 bf16 = 16 B or 8 fp32 = 32 B), loaded ahead of use.
template <class T> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 r{0u, 0u, 0u, 0u};
  __device__ __forceinline__ void load(const bf16* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void to(float (&v)[8]) const {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = __uint_as_float(w[i] << 16); v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u); }
  }
};
template <> struct Raw8<float> {
  float4 a{0.f, 0.f, 0.f, 0.f}, b{0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void to(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Dequantisation factor of an FP8 GEMM (product of the operands' inverse scales), 1 otherwise.
// The factors are read once per block (load(), from the epilogue's prepare()) and kept in
// registers: read through the pointers at each use, they were fetched again for every element,
// each fetch waited for, since the epilogue's stores might alias them.
struct Deq {
  const float* ia;
  const float* ib;
  float a = 1.f, b = 1.f;
  __device__ __forceinline__ void load() {
    if (ia) {
      a = *ia;
      b = *ib;
    }
  }
  __device__ __forceinline__ float apply(float acc) const { return ia ? (acc * a) * b : acc; }
};

// C = round(deq(acc)), or with accumulate C = round(C + deq(acc)) (gradient accumulation over
// micro-batches: one rounding of the sum)
template <class OutT> struct EpiStore {
  static constexpr const char* kName = "store";
  static constexpr int kKind = kEpiPlain;
  OutT* C; int64_t ldc; Deq dq; int accumulate = 0;
  __device__ __forceinline__ void prepare() { dq.load(); }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
    OutT* p = C + (int64_t)m * ldc + n;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = dq.apply(v[k]);
    if (accumulate) {
      float o[8];
      Vec8<OutT>::load(p, o);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += o[k];
    }
    Vec8<OutT>::store(p, v);
  }
};

// out = round(alpha other + beta acc) (other [m, n] read at the output's position; out must not
// alias an operand of the GEMM)
template <class T> struct EpiLin {
  static constexpr const char* kName = "lin";
  static constexpr int kKind = kEpiPlain;
  T* out; const T* other; int64_t ld; float alpha; float beta;
  using Pf = Raw8<T>;
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.load(other + (int64_t)m * ld + n);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    const int64_t o = (int64_t)m * ld + n;
    float x[8];
    f.to(x);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = alpha * x[k] + beta * v[k];
    Vec8<T>::store(out + o, v);
  }
};

// t = round(deq(acc)); branch[m, n] = t (optional); out = round(x + a * t)
template <class T> struct EpiResidual {
  static constexpr const char* kName = "residual";
  static constexpr int kKind = kEpiPlain;
  T* out; const T* x; T* branch; int64_t ld; const float* a; Deq dq;
  float as = 1.f;                                           // *a, read once per block
  __device__ __forceinline__ void prepare() {
    dq.load();
    as = *a;
  }
  using Pf = Raw8<T>;
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.load(x + (int64_t)m * ld + n);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    const int64_t o = (int64_t)m * ld + n;
    float xv[8];
    f.to(xv);
    const float s = as;
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
  __device__ __forceinline__ void prepare() { dq.load(); }
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8]) const {
    const int64_t o = (int64_t)m * ld + n;
    float rr[8], mx = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = Elem<T>::rnd(dq.apply(v[k]));
      const float p = relu_keep_nan(v[k]);
      rr[k] = Elem<T>::rnd(p * p);
      mx = fmaxf(mx, rr[k]);
    }
    Vec8<T>::store(u + o, v);
    Vec8<T>::store(r + o, rr);
    return mx;
  }
};

// u = round(deq(acc)); stores u only; returns max of r = round(relu(u)^2) (the quantiser of r then
// reads u and forms the same r)
template <class T> struct EpiRelu2Amax {
  static constexpr const char* kName = "relu2";
  static constexpr int kKind = kEpiAmax;
  T* u; int64_t ld; Deq dq; float* amax;
  __device__ __forceinline__ void prepare() { dq.load(); }
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8]) const {
    float mx = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = Elem<T>::rnd(dq.apply(v[k]));
      const float p = relu_keep_nan(v[k]);
      mx = fmaxf(mx, Elem<T>::rnd(p * p));
    }
    Vec8<T>::store(u + (int64_t)m * ld + n, v);
    return mx;
  }
};

// dr = round(deq(acc)); du = round(dr * 2 relu(u)); stores du; returns max |du|
template <class T> struct EpiRelu2Bwd {
  static constexpr const char* kName = "relu2_bwd";
  static constexpr int kKind = kEpiAmax;
  T* du; const T* u; int64_t ld; Deq dq; float* amax;
  __device__ __forceinline__ void prepare() { dq.load(); }
  using Pf = Raw8<T>;
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.load(u + (int64_t)m * ld + n);
    return f;
  }
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8], const Pf& f) const {
    const int64_t o = (int64_t)m * ld + n;
    float uv[8], mx = 0.f;
    f.to(uv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dr = Elem<T>::rnd(dq.apply(v[k]));
      v[k] = Elem<T>::rnd(dr * (2.f * relu_keep_nan(uv[k])));
      mx = fmaxf(mx, fabsf(v[k]));
    }
    Vec8<T>::store(du + o, v);
    return mx;
  }
};

// SwiGLU MLP, up projection (the gate half g = round(hn W_gate^T) is already stored at gu[m, n]):
// u = round(acc) is stored at gu[m, F + n] and a = round(silu(g) u) at a[m, n]
template <class T> struct EpiSwigluUp {
  static constexpr const char* kName = "swiglu_up";
  static constexpr int kKind = kEpiPlain;
  T* gu; int64_t ldgu; int F; T* a; int64_t lda;
  using Pf = Raw8<T>;
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.load(gu + (int64_t)m * ldgu + n);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    T* row = gu + (int64_t)m * ldgu;
    float g[8], av[8];
    f.to(g);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[k] = Elem<T>::rnd(v[k]);
      av[k] = g[k] / (1.f + expf(-g[k])) * v[k];
    }
    Vec8<T>::store(row + F + n, v);
    Vec8<T>::store(a + (int64_t)m * lda + n, av);
  }
};

// SwiGLU MLP backward: da = round(acc) (= dm W_proj); with g = gu[m, n], u = gu[m, F + n],
// s = sigmoid(g): dgu[m, n] = round(da u s (1 + g (1 - s))) and dgu[m, F + n] = round(da g s)
template <class T> struct EpiSwigluBwd {
  static constexpr const char* kName = "swiglu_bwd";
  static constexpr int kKind = kEpiPlain;
  T* dgu; const T* gu; int64_t ld; int F;
  struct Pf { Raw8<T> g, u; };
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.g.load(gu + (int64_t)m * ld + n);
    f.u.load(gu + (int64_t)m * ld + n + F);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    const int64_t o = (int64_t)m * ld + n;
    float g[8], u[8], dg[8], du[8];
    f.g.to(g);
    f.u.to(u);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float da = Elem<T>::rnd(v[k]);
      const float sg = 1.f / (1.f + expf(-g[k]));
      dg[k] = da * u[k] * sg * (1.f + g[k] * (1.f - sg));
      du[k] = da * g[k] * sg;
    }
    Vec8<T>::store(dgu + o, dg);
    Vec8<T>::store(dgu + o + F, du);
  }
};

// qkv = round(acc); on the v columns (n >= vcol0) of value-embedding layers:
// v = round(v + table[ids[m], n - vcol0]), nothing added for ids outside [0, rows).
// With kh set (128-wide heads), the k columns [kcol0, vcol0) also leave normalised and rotated
// [hn.213312.xyz translation, 设置 / Setup: QK-norm, RoPE]: k^ = RoPE(k / rms(k)) with
// rms(k) = sqrt(mean(k^2) + eps) over the head, the rotation of channel pairs (i, i + 64) by the
// angles of position m % seq from cs [seq, 64] (cos, sin); k^ goes to kh [M, vcol0 - kcol0] and
// 1 / rms(k) to rk [M, heads]. A head's 16 segments are 16 aligned consecutive lanes of one row (every
// block configuration's N tile is 128 or 256 wide), so the sum of squares is a 16-lane reduction and
// the partner of channel i is 8 lanes away.
template <class T> struct EpiQkv {
  static constexpr const char* kName = "qkv";
  static constexpr int kKind = kEpiPlain;
  T* C; int64_t ldc; const T* table; int64_t ldt; const int32_t* ids; int vcol0; int64_t rows;
  T* kh = nullptr; float* rk = nullptr; const float2* cs = nullptr; int kcol0 = 0; int seq = 1; float eps = 0.f;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = Elem<T>::rnd(v[k]);
    if (kh && n >= kcol0 && n < vcol0) {                    // uniform over the head's 16 lanes
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) ss += v[k] * v[k];
      ss = group_sum<16>(ss);
      const float r = 1.0f / sqrtf(ss / 128.f + eps);
      const int c = (n - kcol0) & 127, i0 = c & 63;
      const bool lo = c < 64;                               // channel i (else i + 64) of pairs i0 ..
      const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)(m % seq) * 64 + i0);
      float y[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 cc = c4[q];                           // (cos, sin) of pairs i0 + 2q, i0 + 2q + 1
        const float cv[2] = {cc.x, cc.z}, sv[2] = {cc.y, cc.w};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int k = 2 * q + e;
          const float own = v[k] * r, oth = dpp_move<0x128>(v[k]) * r;   // row_ror:8, lane ^ 8
          y[k] = lo ? own * cv[e] - oth * sv[e] : oth * sv[e] + own * cv[e];
        }
      }
      Vec8<T>::store(kh + (int64_t)m * (vcol0 - kcol0) + (n - kcol0), y);
      if (c == 0) rk[(int64_t)m * ((vcol0 - kcol0) >> 7) + ((n - kcol0) >> 7)] = r;
    }
    if (table && n >= vcol0) {
      const int32_t id = ids[m];
      if (id >= 0 && id < rows) {
        float e[8];
        Vec8<T>::load(table + (int64_t)id * ldt + (n - vcol0), e);
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] += e[k];
      }
    }
    Vec8<T>::store(C + (int64_t)m * ldc + n, v);
  }
};

// t = (accumulate ? C32 : 0) + acc   (fp32 accumulation across calls), stored to C32
struct EpiAcc32 {
  static constexpr const char* kName = "acc32";
  static constexpr int kKind = kEpiPlain;
  float* C; int64_t ldc; int accumulate;
  using Pf = Raw8<float>;                                   // C32 before the call (accumulate only)
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    if (accumulate) f.load(C + (int64_t)m * ldc + n);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    float* p = C + (int64_t)m * ldc + n;
    if (accumulate) {
      float o[8];
      f.to(o);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += o[k];
    }
    Vec8<float>::store(p, v);
  }
};

// the last call of an fp32 accumulation: out = round(C32 + acc), or with accumulate
// out = round(out + C32 + acc) (C32 is only read)
template <class OutT> struct EpiAcc32Out {
  static constexpr const char* kName = "acc32";
  static constexpr int kKind = kEpiPlain;
  const float* C; OutT* out; int64_t ldc; int accumulate = 0;
  using Pf = Raw8<float>;                                   // C32
  __device__ __forceinline__ Pf load(int m, int n) const {
    Pf f;
    f.load(C + (int64_t)m * ldc + n);
    return f;
  }
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8], const Pf& f) const {
    const int64_t o = (int64_t)m * ldc + n;
    float c[8];
    f.to(c);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += c[k];
    if (accumulate) {
      float p[8];
      Vec8<OutT>::load(out + o, p);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += p[k];
    }
    Vec8<OutT>::store(out + o, v);
  }
};

// Two independent GEMMs in one grid: the kernel's own operands with e0, then (blocks from skip on)
// C1 = A1 B1^T with e1 (operands a1, b1 of the kernel's element type, leading dimensions lda1,
// ldb1, shape m1 x n1 x k1, block order g1). One grid lets the second GEMM's tiles fill the CUs
// that the first one's last wave of blocks leaves idle. Each epilogue is plain or amax-reducing (at
// most one of the two reducing); sel (set by the kernel) picks the one of the block's GEMM, and the
// blocks of a plain one contribute 0 to the other's amax.
template <class E0, class E1> struct EpiPair {
  static constexpr bool kPair = true;
  static constexpr bool kAmax0 = E0::kKind == kEpiAmax, kAmax1 = E1::kKind == kEpiAmax;
  static constexpr int kKind = kAmax0 || kAmax1 ? kEpiAmax : kEpiPlain;
  static_assert((E0::kKind == kEpiPlain || kAmax0) && (E1::kKind == kEpiPlain || kAmax1) && !(kAmax0 && kAmax1),
                "plain epilogues, at most one of them amax-reducing");
  E0 e0; E1 e1;
  const void* a1; int64_t lda1; const void* b1; int64_t ldb1;
  int m1, n1, k1, g1;
  int skip = 0;
  int sel = 0;
  float* amax = nullptr;                                    // the reducing epilogue's (set by the launch)
  struct PfPair {
    typename HasPf<E0>::type p0;
    typename HasPf<E1>::type p1;
  };
  __host__ __device__ void set_amax() {
    if constexpr (kAmax0) amax = e0.amax;
    if constexpr (kAmax1) amax = e1.amax;
  }
  __device__ __forceinline__ void prepare() {
    if (sel) {
      if constexpr (HasPrepare<E1>::value) e1.prepare();
    } else {
      if constexpr (HasPrepare<E0>::value) e0.prepare();
    }
  }
  __device__ __forceinline__ PfPair pf_load(int m, int n) const {
    PfPair f;
    if (sel) {
      if constexpr (HasPf<E1>::value) f.p1 = e1.load(m, n);
    } else {
      if constexpr (HasPf<E0>::value) f.p0 = e0.load(m, n);
    }
    return f;
  }
  template <class E, class F>
  __device__ __forceinline__ static float run(const E& e, int m, int n, float (&v)[8], const F& f) {
    if constexpr (HasPf<E>::value) {
      if constexpr (E::kKind == kEpiAmax) return e.seg(m, n, v, f);
      else e.seg(m, n, v, f);
    } else {
      if constexpr (E::kKind == kEpiAmax) return e.seg(m, n, v);
      else e.seg(m, n, v);
    }
    return 0.f;
  }
  __device__ __forceinline__ float seg_pf(int m, int n, float (&v)[8], const PfPair& f) const {
    return sel ? run(e1, m, n, v, f.p1) : run(e0, m, n, v, f.p0);
  }
};

// EpiPair with the prefetch interface when either epilogue has one
template <class E0, class E1, bool = HasPf<E0>::value || HasPf<E1>::value> struct EpiPairOf : EpiPair<E0, E1> {
  using Pf = typename EpiPair<E0, E1>::PfPair;
  __device__ __forceinline__ Pf load(int m, int n) const { return this->pf_load(m, n); }
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8], const Pf& f) const { return this->seg_pf(m, n, v, f); }
};
template <class E0, class E1> struct EpiPairOf<E0, E1, false> : EpiPair<E0, E1> {
  __device__ __forceinline__ float seg(int m, int n, float (&v)[8]) const {
    return this->seg_pf(m, n, v, typename EpiPair<E0, E1>::PfPair{});
  }
};

// fp32 partial sums of K slice blockIdx.y: C[blockIdx.y slice + m ldc + n] = acc
struct EpiSplitK32 {
  static constexpr const char* kName = "splitk";
  static constexpr int kKind = kEpiPlain;
  static constexpr bool kSplitK = true;
  float* C; int64_t ldc; int64_t slice; int kchunk;
  __device__ __forceinline__ void seg(int m, int n, float (&v)[8]) const {
    Vec8<float>::store(C + (int64_t)blockIdx.y * slice + (int64_t)m * ldc + n, v);
  }
};

// out[m, n] = round(deq(sum over the S slices of part[s slice + m ldp + n])) (+ out[m, n] before the
// rounding with accumulate), 8 columns per thread
template <class T>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int S, int64_t slice,
                                                           int64_t ldp, int M, int N, T* __restrict__ out, int64_t ldo,
                                                           Deq dq, int accumulate) {
  dq.load();
  const int nseg = N / 8;
  const int64_t total = (int64_t)M * nseg;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / nseg), n = (int)(i % nseg) * 8;
    float v[8], t[8];
    Vec8<float>::load(part + (int64_t)m * ldp + n, v);
    for (int sl = 1; sl < S; ++sl) {
      Vec8<float>::load(part + sl * slice + (int64_t)m * ldp + n, t);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += t[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = dq.apply(v[k]);
    if (accumulate) {
      Vec8<T>::load(out + (int64_t)m * ldo + n, t);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += t[k];
    }
    Vec8<T>::store(out + (int64_t)m * ldo + n, v);
  }
}

// ------------------------------------------------------------------ launcher
template <class ET> struct OpName;
template <> struct OpName<float> { static constexpr const char* s = "f32"; };
template <> struct OpName<bf16> { static constexpr const char* s = "bf16"; };
template <> struct OpName<fp8> { static constexpr const char* s = "e4m3"; };

// trace tag of a GEMM instantiation: "gemm_<operand type>_<epilogue>_<layouts>", layouts "k" (K-major)
// or "m" (MN-major) for A then B
template <class ET, class Epi, bool AK, bool BK>
inline const char* gemm_tag() {
  static const std::string t = std::string("gemm_") + OpName<ET>::s + "_" + Epi::kName + "_" + (AK ? "k" : "m") +
                               (BK ? "k" : "m");
  return t.c_str();
}

// Operand layouts of a GEMM call: K-major ("row m holds its K elements contiguously") or MN-major.
struct GemmOps {
  bool a_kmajor = true, b_kmajor = true;
  const void* zrow = nullptr;       // >= 16 zero bytes: K-tail rows of MN-major operands
  int group = 0;                    // block-order group (tile rows or columns); 0 = automatic (2)
};

template <class ET, int BM, int BN, int WGM, int WGN, int KB, int NS, int MODE = 0, class Epi>
inline hipError_t launch_gemm_cfg(int cfg_id, const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                  const Epi& epi, const GemmOps& o, hipStream_t s) {
  const int64_t nbt = cdiv(M, BM) * cdiv(N, BN);
  // Block order: along the longer side of the output, `group` tile rows (or columns) at a time,
  // 2 unless the call site asks otherwise. Measured over groups of 1, 2, 3, 4, 8 on the ping-pong
  // loop: the loss's logits and dH GEMMs run ~1% faster at 4 (their call sites ask for it); the e4m3
  // MLP GEMMs with their own epilogues 1-4% slower at 4 than at 2 in the step (same box), the loss's
  // dW GEMM 2.4% slower.
  const int g = o.group > 0 ? o.group : 2;
  const int G = cdiv(M, BM) >= cdiv(N, BN) ? g : -g;
  unsigned slices = 1;
  if constexpr (IsSplitK<Epi>::value) slices = (unsigned)std::max<int64_t>(1, cdiv(K, epi.kchunk));
  const dim3 nb((unsigned)nbt, slices);
  const ET* z = static_cast<const ET*>(o.zrow);
  constexpr int NT = 64 * WGM * WGN;
  if constexpr (sizeof(ET) == 2 && MODE != 3 && MODE != 4) {   // MODE 3, 4: K-major operands only (the callers check)
    if (!o.a_kmajor && !o.b_kmajor) {
      const char* tag = gemm_tag<ET, Epi, false, false>();
      LL_LAUNCH_GEMM(tag, M, N, K, cfg_id, (int)slices, (gemm_kernel<ET, BM, BN, WGM, WGN, KB, NS, false, false, Epi, MODE>), nb, dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi, G);
      return hipGetLastError();
    }
    if (!o.a_kmajor) {
      const char* tag = gemm_tag<ET, Epi, false, true>();
      LL_LAUNCH_GEMM(tag, M, N, K, cfg_id, (int)slices, (gemm_kernel<ET, BM, BN, WGM, WGN, KB, NS, false, true, Epi, MODE>), nb, dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi, G);
      return hipGetLastError();
    }
    if (!o.b_kmajor) {
      const char* tag = gemm_tag<ET, Epi, true, false>();
      LL_LAUNCH_GEMM(tag, M, N, K, cfg_id, (int)slices, (gemm_kernel<ET, BM, BN, WGM, WGN, KB, NS, true, false, Epi, MODE>), nb, dim3(NT),
                    0, s, A, lda, B, ldb, M, N, K, z, epi, G);
      return hipGetLastError();
    }
  }
  const char* tag = gemm_tag<ET, Epi, true, true>();
  LL_LAUNCH_GEMM(tag, M, N, K, cfg_id, (int)slices, (gemm_kernel<ET, BM, BN, WGM, WGN, KB, NS, true, true, Epi, MODE>), nb, dim3(NT), 0, s,
                A, lda, B, ldb, M, N, K, z, epi, G);
  return hipGetLastError();
}

// Block-tile configurations (block tile, waves, K-tile bytes, LDS stages):
//   1 = 128 x 128, 4 waves, 128 B, 2      2 = 256 x 256, 4 waves (2 x 2), 128 B, 2
//   3 = 256 x 256, 8 waves (2 x 4), 128 B, 2   4 = 256 x 256, 8 waves (4 x 2), 128 B, 2
//   5 = 256 x 256, 8 waves (2 x 4), 64 B, 3    6 = 256 x 256, 8 waves (4 x 2), 64 B, 3
//   7 = 128 x 128, 4 waves, 64 B, 3
//   8 = 256 x 256, 4 waves (2 x 2, one per SIMD), 64 B, 3, fragments of the next K tile prefetched
//       into registers across the barrier
//   9 = 256 x 256, 8 waves (4 x 2), 128 B, 2, split-phase K loop with the LDS reads and half the
//       loads interleaved into the MFMAs (bf16; e4m3 falls back to 4)
//  10 = 256 x 256, 4 waves (2 x 2, one per SIMD), 128 B, 2, split-phase K loop (bf16; e4m3: 4)
//  14 = 256 x 256, 8 waves (4 x 2), 128 B, 2, ping-pong K loop (two wave groups alternating MFMA-only
//       and read/load phases) on the 16x16x32 bf16 MFMA; e4m3 runs it as 15, an MN-major operand as 9
//  15 = the ping-pong loop on the 32x32x64 e4m3 MFMA (bf16 runs it as 14)
//  11 = 256 x 256, 8 waves (4 x 2), 128 B, 2, split-phase K loop on the 32x32 MFMAs (32x32x64 e4m3,
//       32x32x16 bf16) with reads and half the loads interleaved (fp32 runs it as 4; bf16 with an
//       MN-major operand as 9). bf16 measured ~7% slower than 9 on the loss's shapes, so only e4m3
//       takes it automatically.
// e4m3 needs 128-byte K tiles (32 bytes of K per lane per MFMA): 5, 6, 7 fall back to 3, 4, 1.
// 0 = automatic (gemm_config_override()).
template <class ET, class Epi>
inline hipError_t launch_gemm_with(int cfg, const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                   const Epi& epi, const GemmOps& o, hipStream_t s) {
  if constexpr (sizeof(ET) == 1) {
    if (cfg == 5) cfg = 3;
    if (cfg == 6) cfg = 4;
    if (cfg == 7) cfg = 1;
    if (cfg == 8 || cfg == 9 || cfg == 10) cfg = 4;
    if (cfg == 11) return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
  } else if constexpr (sizeof(ET) == 2) {
    if (cfg == 11) {
      if (o.a_kmajor && o.b_kmajor) return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
      cfg = 9;
    }
  } else {
    if (cfg == 9 || cfg == 10 || cfg == 11) cfg = 4;
  }
  if constexpr (sizeof(ET) <= 2) {
    // 12: 256 x 256, 4 waves (2 x 2, one per SIMD, 128 x 128 each), split-phase on the 32x32 MFMAs;
    // 13: the same on the 16x16 MFMAs with interleaved reads (bf16). K-major operands only.
    if ((cfg == 12 || cfg == 13) && o.a_kmajor && o.b_kmajor) {
      if (cfg == 12 || sizeof(ET) == 1) return launch_gemm_cfg<ET, 256, 256, 2, 2, 128, 2, 3>(12, A, lda, B, ldb, M, N, K, epi, o, s);
      if constexpr (sizeof(ET) == 2) return launch_gemm_cfg<ET, 256, 256, 2, 2, 128, 2, 2>(13, A, lda, B, ldb, M, N, K, epi, o, s);
    }
    if (cfg == 12 || cfg == 13) cfg = 9;
  } else {
    if (cfg == 12 || cfg == 13) cfg = 4;
  }
  if constexpr (sizeof(ET) == 2) {
    // 14 (and 15): 256 x 256, 8 waves (4 x 2), 128 B, 2, ping-pong K loop (K-major operands;
    // otherwise 9)
    if (cfg == 14 || cfg == 15) {
      // lane offsets are 32-bit: 256 rows of either operand must span less than 2^31 bytes
      const bool fits = lda < (int64_t(1) << 22) && ldb < (int64_t(1) << 22);
      if (o.a_kmajor && o.b_kmajor && fits)
        return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2, 4>(14, A, lda, B, ldb, M, N, K, epi, o, s);
      cfg = 9;
    }
  } else if constexpr (sizeof(ET) == 1) {
    // 15: 256 x 256, 8 waves (4 x 2), 128 B, 2, ping-pong K loop on the 32x32x64 e4m3 MFMA
    if (cfg == 15 || cfg == 14) {
      const bool fits = lda < (int64_t(1) << 22) && ldb < (int64_t(1) << 22);
      if (fits) return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2, 5>(15, A, lda, B, ldb, M, N, K, epi, o, s);
      cfg = 11;
    }
  } else {
    if (cfg == 14 || cfg == 15) cfg = 4;
  }
  switch (cfg) {
    case 1: return launch_gemm_cfg<ET, 128, 128, 2, 2, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
    case 2: return launch_gemm_cfg<ET, 256, 256, 2, 2, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
    case 3: return launch_gemm_cfg<ET, 256, 256, 2, 4, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
    case 4: return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
    default:
      if constexpr (sizeof(ET) != 1) {
        if (cfg == 5) return launch_gemm_cfg<ET, 256, 256, 2, 4, 64, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        if (cfg == 6) return launch_gemm_cfg<ET, 256, 256, 4, 2, 64, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        if (cfg == 7) return launch_gemm_cfg<ET, 128, 128, 2, 2, 64, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        if (cfg == 8) return launch_gemm_cfg<ET, 256, 256, 2, 2, 64, 3>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        if (cfg == 9) {
          if constexpr (sizeof(ET) == 2) return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
          else return launch_gemm_cfg<ET, 256, 256, 4, 2, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        }
        if (cfg == 10) {
          if constexpr (sizeof(ET) == 2) return launch_gemm_cfg<ET, 256, 256, 2, 2, 128, 2, 1>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
          else return launch_gemm_cfg<ET, 256, 256, 2, 2, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
        }
      }
      return launch_gemm_cfg<ET, 256, 256, 2, 4, 128, 2>(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
  }
}

// Picks the block tile from the wave quantisation on 256 CUs: 256 x 256 with 8 waves (measured
// ~25% faster per FLOP than 128 x 128 on the layer's shapes) unless its last wave of blocks
// leaves so many CUs idle that 128 x 128 finishes first. Requirements (checked by the callers): K a multiple of the K tile for K-major
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
    const double e128 = 0.75 * (double)t128 / (double)(cdiv(t128, 256) * 256);
    // 4 x 2 waves, except 2 x 4 when B is MN-major (measured ~3% faster there); bf16 with both
    // operands K-major takes the ping-pong K loop (measured 1-7% faster than the split-phase loop of
    // configuration 9, which was 2-5% faster than configuration 4), e4m3 the split-phase loop on the
    // 32x32x64 MFMA (6-9% faster than configuration 4 on the MLP shapes)
    const bool kk16 = sizeof(ET) == 2 && o.a_kmajor && o.b_kmajor;
    cfg = e256 >= e128 ? (sizeof(ET) == 1 ? 11 : kk16 ? 14 : o.b_kmajor ? 4 : 3) : 1;
  }
  return launch_gemm_with(cfg, A, lda, B, ldb, M, N, K, epi, o, s);
}

// Whether two GEMMs with K-major operands of these leading dimensions can share one grid
// (launch_gemm_pair): the configuration in force is the automatic one or the pair's own (bf16: the
// ping-pong loop, 14, whose 32-bit lane offsets must reach every row; e4m3: the 32x32x64
// split-phase loop, 11).
template <class ET>
inline bool gemm_pair_ok(int64_t lda0, int64_t ldb0, int64_t lda1, int64_t ldb1) {
  static_assert(sizeof(ET) <= 2, "bf16 or e4m3");
  const int oc = gemm_config_override();
  if constexpr (sizeof(ET) == 1) {
    return oc == 0 || oc == 11;
  } else {
    const int64_t lim = int64_t(1) << 22;
    return (oc == 0 || oc == 14) && lda0 < lim && ldb0 < lim && lda1 < lim && ldb1 < lim;
  }
}

// C0 = A B^T (M x N x K, epilogue epi.e0, block-order group group0) and C1 = A1 B1^T (epi's second
// GEMM, group epi.g1) in one grid: the first GEMM's tiles are dispatched first, then the second's,
// so that with the longer-K GEMM first the shorter tiles fill the CUs the first one's last wave
// leaves idle. 256 x 256 tiles, 8 waves: bf16 on the ping-pong loop (configuration 14), e4m3 on the
// 32x32x64 split-phase loop (11). Both operands of both GEMMs K-major, K a multiple of the K tile
// (64 bf16, 128 e4m3; rows zero-padded), N a multiple of 8; the caller checks gemm_pair_ok. The
// launch trace records the pair's FLOPs as a 1 x 1 x (M N K + M1 N1 K1) GEMM.
template <class ET, class Epi>
inline hipError_t launch_gemm_pair(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                   int group0, Epi epi, hipStream_t s) {
  static_assert(sizeof(ET) <= 2 && IsPair<Epi>::value, "bf16 or e4m3 two-GEMM epilogue");
  if (M <= 0 || N <= 0 || epi.m1 <= 0 || epi.n1 <= 0) return hipErrorInvalidValue;
  const int64_t nb0 = cdiv(M, 256) * cdiv(N, 256), nb1 = cdiv(epi.m1, 256) * cdiv(epi.n1, 256);
  epi.skip = (int)round_up(nb0, 8);
  epi.set_amax();
  const int g0 = cdiv(M, 256) >= cdiv(N, 256) ? group0 : -group0;
  epi.g1 = cdiv(epi.m1, 256) >= cdiv(epi.n1, 256) ? epi.g1 : -epi.g1;
  const int64_t work = (int64_t)M * N * K + (int64_t)epi.m1 * epi.n1 * epi.k1;
  const char* tag = gemm_tag<ET, Epi, true, true>();
  constexpr int kMode = sizeof(ET) == 1 ? 3 : 4;
  LL_LAUNCH_GEMM(tag, 1, 1, work, sizeof(ET) == 1 ? 11 : 14, 1,
                 (gemm_kernel<ET, 256, 256, 4, 2, 128, 2, true, true, Epi, kMode>),
                 dim3((unsigned)(epi.skip + nb1)), dim3(512), 0, s, A, lda, B, ldb, M, N, K,
                 static_cast<const ET*>(nullptr), epi, g0);
  return hipGetLastError();
}

// Number of K slices (1..smax) for a GEMM of `tiles` 256 x 256 output tiles: the one that fills the
// last wave of blocks on 256 CUs best (fewest slices within 2% of the best), each slice at least
// 8 K tiles long.
inline int splitk_slices(int64_t tiles, int64_t K, int ke, int smax) {
  auto eff = [&](int sl) { return (double)(tiles * sl) / (double)(cdiv(tiles * sl, 256) * 256); };
  int best = 1;
  for (int sl = 2; sl <= smax; ++sl)
    if (K >= (int64_t)sl * 8 * ke && eff(sl) > eff(best) + 0.02) best = sl;
  return best;
}

// out = round(deq(A B^T)) (OutT) in `slices` K slices: the GEMM writes each slice's fp32 partial
// sums to scratch [slices, M, N] and a second kernel adds them. For GEMMs with a long K and too few
// output tiles to fill the chip (weight gradients).
template <class ET, class OutT>
inline hipError_t launch_gemm_splitk(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                     int slices, OutT* out, int64_t ldo, float* scratch, const GemmOps& o,
                                     hipStream_t s, Deq dq = Deq{nullptr, nullptr}, int accumulate = 0) {
  if (M <= 0 || N <= 0) return hipSuccess;
  constexpr int KE = 128 / (int)sizeof(ET);
  const int kchunk = (int)std::max<int64_t>(KE, round_up(cdiv(K, slices), KE));
  const int sl = (int)std::max<int64_t>(1, cdiv(K, kchunk));
  EpiSplitK32 e{scratch, (int64_t)N, (int64_t)M * N, kchunk};
  int cfg = gemm_config_override();
  if (cfg == 0) cfg = sizeof(ET) == 1 ? 11 : sizeof(ET) == 2 && o.a_kmajor && o.b_kmajor ? 14 : o.b_kmajor ? 4 : 3;
  hipError_t r = launch_gemm_with(cfg, A, lda, B, ldb, M, N, K, e, o, s);
  if (r != hipSuccess) return r;
  const int64_t work = (int64_t)M * (N / 8);
  LL_LAUNCH("splitk_reduce", splitk_reduce_kernel<OutT>, dim3((unsigned)std::min<int64_t>(cdiv(work, 256), 8192)),
            dim3(256), 0, s, scratch, sl, (int64_t)M * N, (int64_t)N, M, N, out, ldo, dq, accumulate);
  return hipGetLastError();
}

template <class ET, class Epi>
inline hipError_t launch_gemm_nt(const ET* A, int64_t lda, const ET* B, int64_t ldb, int M, int N, int K,
                                 const Epi& epi, hipStream_t s) {
  return launch_gemm(A, lda, B, ldb, M, N, K, epi, GemmOps{}, s);
}

}  // namespace
}  // namespace ll
