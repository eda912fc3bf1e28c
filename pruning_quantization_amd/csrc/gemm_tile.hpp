// MFMA GEMM tile shared by the operator-error and sparse-GEMM calls.
//
// C = A' B'^T for A' [M][Kp] and B [N][K] (both bf16, reduction axis
// contiguous), B'[n][k] = B[n][k % K] (K divides Kp).  A' is either dense
// bf16 rows or a 2:4-compressed operand (kept values [M][Kp/2] in position
// order + 4-bit group metadata [M][Kp/8], the layout of the prune calls),
// which gfx950's sparse MFMA reads as is: v_smfmac_f32_16x16x64_bf16 takes
// per lane 8 kept values of 16 logical k (four groups of four; lane group h
// = lane / 16 holds k 16h .. 16h + 15) and their 2-bit in-group positions
// packed in order, i.e. exactly the 16 metadata bits of those four groups.
// Its dense B operand holds per lane k 8h .. 8h + 7 and 32 + 8h .. 32 + 8h + 7
// (established by an in-bounds lane-layout check of the instruction).
//
// Workgroup tile 256 x 256, eight waves of 128 x 64 (8 x 4 tiles of 16 x 16),
// fp32 accumulation.  k_gemm_dma streams slabs straight into LDS several
// slabs ahead (a register-staged form with 64-deep slabs double-buffered in
// padded LDS rows measured 10-25% slower and was removed).  A lane's k values
// of a fragment are the same positions for A and B, which is all the dense
// product needs.  Strides and depths of GM_FP8 are counted in pairs of codes
// (16-bit units), so a 64-unit slab is 128 codes and every load path is
// shared.  Epilogue: per-row sums of C^2 over the tile's
// columns (EPI_ROWSQ) or C stored as fp32 (EPI_STORE).  GM_FP8 runs the same
// tile on e4m3 codes with v_mfma_f32_16x16x128_f8f6f4 and applies the per-row
// scales of both operands when storing C.
#pragma once

#include "device_common.hpp"

namespace sparq24 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kGM = 256, kGN = 256;
enum GemmEpi : int { EPI_ROWSQ = 0, EPI_STORE = 1 };
// Operand kinds: dense bf16, 2:4-compressed bf16 A (sparse MFMA), dense e4m3
// codes with per-row fp32 scales (C = scale_a[m] * scale_b[n] * sum a b).
enum GemmMode : int { GM_BF16 = 0, GM_SPARSE = 1, GM_FP8 = 2 };
typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct GemmArgs {
  const void* A;     // dense bf16 rows, or the kept values of a compressed operand
  int64_t lda;       // elements between rows of A (Kp, or Kp/2 for compressed values)
  const uint8_t* meta;  // compressed operand: metadata [M][Kp/8] (else null)
  int64_t ldm;       // bytes between metadata rows
  const void* B;
  int64_t ldb;
  int64_t M, N, Kp, K;
  float* out;        // EPI_ROWSQ: part [M][ntiles]; EPI_STORE: C [M][ldc]
  int64_t ld_out;    // EPI_ROWSQ: ntiles; EPI_STORE: elements between rows of C
  const float* scale_a;  // GM_FP8: per-row scales of A [M] and B [N]
  const float* scale_b;
};

// ---------------------------------------------------------------------------
// Multi-stage tile, used for every operand kind: slabs go from global memory
// straight into LDS with global_load_lds (no register staging), S slabs deep, so each slab is requested S - 1 slabs before it is
// consumed and L2 misses stay hidden.
// LDS rows are unpadded; their 16-byte chunks are XOR-swizzled by row so the
// 16 rows a fragment read touches fall in distinct bank groups.  Fragments
// are read in inline-asm blocks that wait for their own results, so the only
// waits on the slab loads are the explicit per-wave vmcnt waits before the
// workgroup barrier that publishes a slab (the barrier is the raw s_barrier:
// __syncthreads would drain every load in flight).  Rows past M or N are
// loaded clamped (their products are never stored; the row-sum epilogue
// masks the columns past N).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int MODE>
struct GemmStages;
template <>
struct GemmStages<GM_BF16> {  // 64-deep slabs (full 128-byte rows): A 32 KB + B 32 KB, 2 stages
  static constexpr int SK = 64, S = 2, ACH = 8, BCH = 8, MB = 0;
};
template <>
struct GemmStages<GM_SPARSE> {  // 64-deep slabs: A 16 KB + B 32 KB + meta 2 KB, 3 stages
  static constexpr int SK = 64, S = 3, ACH = 4, BCH = 8, MB = 2048;
};
template <>
struct GemmStages<GM_FP8> {  // 128-code slabs (64 units): A 32 KB + B 32 KB, 2 stages
  static constexpr int SK = 64, S = 2, ACH = 8, BCH = 8, MB = 0;
};

// chunk slot of chunk c in row r of an LDS slab with NCH 16-byte chunks per row
template <int NCH>
__device__ inline int gemm_swz(int r) {
  return NCH == 8 ? (r & 7) : ((r >> 1) & 3);
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

template <int MODE, int EPI>
__global__ __launch_bounds__(512) void k_gemm_dma(GemmArgs g) {
  using C = GemmStages<MODE>;
  constexpr bool SPARSE = MODE == GM_SPARSE;
  constexpr int BM = kGM, BN = kGN, WTM = 128, WTN = 64, WN = BN / WTN, NT = 512;
  constexpr int TI = WTM / 16, TJ = WTN / 16, TH = TI / 2;
  constexpr int SK = C::SK, S = C::S, ACH = C::ACH, BCH = C::BCH;
  constexpr int A_BYTES = BM * ACH * 16, B_BYTES = BN * BCH * 16;
  constexpr int STAGE = A_BYTES + B_BYTES + C::MB;
  constexpr int QA = BM * ACH / NT, QB = BN * BCH / NT;
  constexpr int QPS = QA + QB + (SPARSE ? 1 : 0);  // slab loads per thread per stage
  static_assert(QA * NT == BM * ACH && QB * NT == BN * BCH, "tile / thread mismatch");
  static_assert(A_BYTES + 3 * (BCH * 256) + 1024 < 65536, "ds_read offsets fit 16 bits");
  static_assert(MODE != GM_FP8 || ACH == BCH, "e4m3 A and B fragments share row offsets");
  __shared__ __attribute__((aligned(16))) uint8_t smem[S * STAGE];
  __shared__ float red[EPI == EPI_ROWSQ ? WN : 1][EPI == EPI_ROWSQ ? BM : 1];
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* B = (const uint16_t*)g.B;
  const int64_t M = g.M, N = g.N, K = g.K;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w / WN, wn = w % WN;
  // XCD-aware tile order: workgroups are dealt to the 8 XCDs round robin, so
  // workgroup p runs on XCD p % 8.  Renumber so that each XCD owns a
  // contiguous range of logical tiles, and walk that range in groups of
  // kGroupM row tiles (row tile fastest): the tiles an XCD runs at once then
  // share a few A row slabs and B column slabs in its L2.
  const int64_t ntn = (N + BN - 1) / BN, ntm = (M + BM - 1) / BM, total = ntm * ntn;
  const int64_t pid = blockIdx.x, per = total / 8;
  const int64_t lid = pid < per * 8 ? (pid % 8) * per + pid / 8 : pid;
  constexpr int64_t kGroupM = 8;
  const int64_t ingroup = kGroupM * ntn, first = (lid / ingroup) * kGroupM;
  const int64_t gsz = ntm - first < kGroupM ? ntm - first : kGroupM;
  const int64_t tm = first + (lid % ingroup) % gsz, tn = (lid % ingroup) / gsz;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  // Slab k0 into stage buffer buf: position p = q * NT + tid of a region is
  // row p / NCH, slot p % NCH; a wave's load writes 64 consecutive positions.
  auto issue = [&](int buf, int64_t k0) {
    uint8_t* st = smem + buf * STAGE;
    const int64_t ak = SPARSE ? k0 / 2 : k0, bk = k0 % K;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int p = q * NT + tid, r = p / ACH, c = (p % ACH) ^ gemm_swz<ACH>(r);
      const int64_t m = m0 + r < M ? m0 + r : M - 1;
      __builtin_amdgcn_global_load_lds(A + m * g.lda + ak + c * 8,
                                       (lds_void_t*)(st + (q * NT + w * 64) * 16), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int p = q * NT + tid, r = p / BCH, c = (p % BCH) ^ gemm_swz<BCH>(r);
      const int64_t n = n0 + r < N ? n0 + r : N - 1;
      __builtin_amdgcn_global_load_lds(B + n * g.ldb + bk + c * 8,
                                       (lds_void_t*)(st + A_BYTES + (q * NT + w * 64) * 16), 16, 0, 0);
    }
    if constexpr (SPARSE) {
      // Metadata (8 bytes per row and slab) laid out per reading lane: 16-byte
      // chunk c = ((wr * 16 + f) * 2 + hp) * 2 + ih holds dword hp of rows
      // wr * 128 + 16 (4 ih + 0..3) + f, i.e. the index halfwords lane f of
      // wave row wr needs for 4 row tiles; chunks sit at c with its low two
      // bits xor (f >> 1) & 3 (8 lanes of one read hit 8 bank groups).
      // Dword p of the region is loaded by thread p.
      const int C = tid >> 2, f = (C >> 2) & 15, c = C ^ ((f >> 1) & 3);
      const int hp = (c >> 1) & 1, i = (c & 1) * 4 + (tid & 3), r = (c >> 6) * WTM + 16 * i + f;
      const int64_t m = m0 + r < M ? m0 + r : M - 1;
      __builtin_amdgcn_global_load_lds(g.meta + m * g.ldm + k0 / 8 + hp * 4,
                                       (lds_void_t*)(st + A_BYTES + B_BYTES + w * 64 * 4), 4, 0, 0);
    }
  };

  // per-lane LDS byte addresses of the fragment reads within stage 0
  const unsigned lds0 = (unsigned)(uintptr_t)(lds_void_t*)smem;
  const int fr = lane & 15, h = lane >> 4;
  const unsigned a_ad = lds0 + (unsigned)(((wm * WTM + fr) * ACH + (h ^ gemm_swz<ACH>(fr))) * 16);
  const unsigned b_ad = lds0 + A_BYTES + (unsigned)(((wn * WTN + fr) * BCH + (h ^ gemm_swz<BCH>(fr))) * 16);
  // sparse: B's second chunk (k 32 + 8h) and the metadata halfword of lane group h
  const unsigned b2_ad = lds0 + A_BYTES + (unsigned)(((wn * WTN + fr) * BCH + ((4 + h) ^ gemm_swz<BCH>(fr))) * 16);
  // the metadata chunk of row tiles 0..3 (that of 4..7 is its neighbour, xor 1)
  const unsigned m_ad =
      lds0 + A_BYTES + B_BYTES + (unsigned)(((((wm * 16 + fr) * 2 + (h >> 1)) * 2) ^ ((fr >> 1) & 3)) * 16);
  const unsigned m_ad2 =
      lds0 + A_BYTES + B_BYTES + (unsigned)(((((wm * 16 + fr) * 2 + (h >> 1)) * 2 + 1) ^ ((fr >> 1) & 3)) * 16);
  const int m_sh = 16 * (h & 1);  // lane group h's halfword of the dword
  constexpr int AR = 16 * ACH * 16, BR = 16 * BCH * 16;  // bytes between 16-row tiles

  f32x4_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t nk = g.Kp / SK;
#pragma unroll
  for (int s = 0; s + 1 < S; ++s) issue(s, (s < nk ? s : nk - 1) * SK);
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt % S);
    wait_vmcnt<(S - 2) * QPS>();  // this wave's loads of slab kt have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave's have, and slab kt - 1 is consumed
    asm volatile("" ::: "memory");
    {
      const int64_t nx = kt + S - 1;
      issue((int)(nx % S), (nx < nk ? nx : nk - 1) * SK);
    }
    const unsigned so = (unsigned)(cur * STAGE);
    if constexpr (SPARSE) {
      const unsigned aa = a_ad + so, ba = b_ad + so, b2 = b2_ad + so, ma = m_ad + so, mb = m_ad2 + so;
      u32x4_t bl[TJ], bh[TJ], af[TH], md;
      // outputs %0..%12; inputs %13 B, %14 B second chunk, %15 A, %16 metadata,
      // %17..%19 B row-tile offsets, %20..%22 A row-tile offsets
      asm volatile(
          "ds_read_b128 %0, %13\n\t"
          "ds_read_b128 %1, %13 offset:%c17\n\t"
          "ds_read_b128 %2, %13 offset:%c18\n\t"
          "ds_read_b128 %3, %13 offset:%c19\n\t"
          "ds_read_b128 %4, %14\n\t"
          "ds_read_b128 %5, %14 offset:%c17\n\t"
          "ds_read_b128 %6, %14 offset:%c18\n\t"
          "ds_read_b128 %7, %14 offset:%c19\n\t"
          "ds_read_b128 %8, %15\n\t"
          "ds_read_b128 %9, %15 offset:%c20\n\t"
          "ds_read_b128 %10, %15 offset:%c21\n\t"
          "ds_read_b128 %11, %15 offset:%c22\n\t"
          "ds_read_b128 %12, %16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(bl[0]), "=&v"(bl[1]), "=&v"(bl[2]), "=&v"(bl[3]), "=&v"(bh[0]), "=&v"(bh[1]),
            "=&v"(bh[2]), "=&v"(bh[3]), "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]),
            "=&v"(md)
          : "v"(ba), "v"(b2), "v"(aa), "v"(ma), "i"(BR), "i"(2 * BR), "i"(3 * BR), "i"(AR),
            "i"(2 * AR), "i"(3 * AR)
          : "memory");
      int ix[TH];
#pragma unroll
      for (int ii = 0; ii < TH; ++ii) ix[ii] = (int)((md[ii] >> m_sh) & 0xFFFFu);
      bf16x16_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bfr[j] = __builtin_shufflevector(__builtin_bit_cast(bf16x8_t, bl[j]), __builtin_bit_cast(bf16x8_t, bh[j]),
                                         0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int ii = 0; ii < TH; ++ii)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[ii][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8_t, af[ii]), bfr[j],
                                                                 acc[ii][j], ix[ii], 0, 0);
      asm volatile(
          "ds_read_b128 %0, %5 offset:%c7\n\t"
          "ds_read_b128 %1, %5 offset:%c8\n\t"
          "ds_read_b128 %2, %5 offset:%c9\n\t"
          "ds_read_b128 %3, %5 offset:%c10\n\t"
          "ds_read_b128 %4, %6\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(md)
          : "v"(aa), "v"(mb), "i"(4 * AR), "i"(5 * AR), "i"(6 * AR), "i"(7 * AR)
          : "memory");
#pragma unroll
      for (int ii = 0; ii < TH; ++ii) ix[ii] = (int)((md[ii] >> m_sh) & 0xFFFFu);
#pragma unroll
      for (int ii = 0; ii < TH; ++ii)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[TH + ii][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
              __builtin_bit_cast(bf16x8_t, af[ii]), bfr[j], acc[TH + ii][j], ix[ii], 0, 0);
    } else if constexpr (MODE == GM_FP8) {
      // a lane's 32 codes of a row are chunks h and 4 + h of the slab (k 16h ..
      // 16h + 15 and 64 + 16h .. 64 + 16h + 15): any split of the 128 k among
      // the lane groups gives the same product as long as A and B use the
      // same one, and this one reads without bank conflicts (chunks 2h and
      // 2h + 1 measured 4 conflict cycles per read); rows in two halves
      // (register budget)
      const unsigned al = lds0 + so + (unsigned)(((wm * WTM + fr) * 8 + (h ^ gemm_swz<8>(fr))) * 16);
      const unsigned ah = lds0 + so + (unsigned)(((wm * WTM + fr) * 8 + ((4 + h) ^ gemm_swz<8>(fr))) * 16);
      const unsigned bl = lds0 + so + A_BYTES + (unsigned)(((wn * WTN + fr) * 8 + (h ^ gemm_swz<8>(fr))) * 16);
      const unsigned bh = lds0 + so + A_BYTES + (unsigned)(((wn * WTN + fr) * 8 + ((4 + h) ^ gemm_swz<8>(fr))) * 16);
      u32x4_t b0[TJ], b1[TJ], x0[TH], x1[TH];
      asm volatile(
          "ds_read_b128 %0, %16\n\t"
          "ds_read_b128 %1, %16 offset:%c20\n\t"
          "ds_read_b128 %2, %16 offset:%c21\n\t"
          "ds_read_b128 %3, %16 offset:%c22\n\t"
          "ds_read_b128 %4, %17\n\t"
          "ds_read_b128 %5, %17 offset:%c20\n\t"
          "ds_read_b128 %6, %17 offset:%c21\n\t"
          "ds_read_b128 %7, %17 offset:%c22\n\t"
          "ds_read_b128 %8, %18\n\t"
          "ds_read_b128 %9, %18 offset:%c20\n\t"
          "ds_read_b128 %10, %18 offset:%c21\n\t"
          "ds_read_b128 %11, %18 offset:%c22\n\t"
          "ds_read_b128 %12, %19\n\t"
          "ds_read_b128 %13, %19 offset:%c20\n\t"
          "ds_read_b128 %14, %19 offset:%c21\n\t"
          "ds_read_b128 %15, %19 offset:%c22\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(b0[0]), "=&v"(b0[1]), "=&v"(b0[2]), "=&v"(b0[3]), "=&v"(b1[0]), "=&v"(b1[1]),
            "=&v"(b1[2]), "=&v"(b1[3]), "=&v"(x0[0]), "=&v"(x0[1]), "=&v"(x0[2]), "=&v"(x0[3]),
            "=&v"(x1[0]), "=&v"(x1[1]), "=&v"(x1[2]), "=&v"(x1[3])
          : "v"(bl), "v"(bh), "v"(al), "v"(ah), "i"(BR), "i"(2 * BR), "i"(3 * BR)
          : "memory");
      i32x8_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        bfr[j] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(b0[j], b1[j], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int ii = 0; ii < TH; ++ii)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[ii][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0[ii], x1[ii], 0, 1, 2, 3, 4, 5, 6, 7)), bfr[j],
              acc[ii][j], 0, 0, 0, 0, 0, 0);
      asm volatile(
          "ds_read_b128 %0, %8 offset:%c10\n\t"
          "ds_read_b128 %1, %8 offset:%c11\n\t"
          "ds_read_b128 %2, %8 offset:%c12\n\t"
          "ds_read_b128 %3, %8 offset:%c13\n\t"
          "ds_read_b128 %4, %9 offset:%c10\n\t"
          "ds_read_b128 %5, %9 offset:%c11\n\t"
          "ds_read_b128 %6, %9 offset:%c12\n\t"
          "ds_read_b128 %7, %9 offset:%c13\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x0[0]), "=&v"(x0[1]), "=&v"(x0[2]), "=&v"(x0[3]), "=&v"(x1[0]), "=&v"(x1[1]),
            "=&v"(x1[2]), "=&v"(x1[3])
          : "v"(al), "v"(ah), "i"(4 * AR), "i"(5 * AR), "i"(6 * AR), "i"(7 * AR)
          : "memory");
#pragma unroll
      for (int ii = 0; ii < TH; ++ii)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[TH + ii][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              __builtin_bit_cast(i32x8_t, __builtin_shufflevector(x0[ii], x1[ii], 0, 1, 2, 3, 4, 5, 6, 7)), bfr[j],
              acc[TH + ii][j], 0, 0, 0, 0, 0, 0);
    } else {
      // two 32-deep steps per slab; lane group h reads chunk 4 st + h of its rows
#pragma unroll
      for (int st = 0; st < SK / 32; ++st) {
        const unsigned aa = lds0 + so + (unsigned)(((wm * WTM + fr) * ACH + ((4 * st + h) ^ gemm_swz<ACH>(fr))) * 16);
        const unsigned ba =
            lds0 + so + A_BYTES + (unsigned)(((wn * WTN + fr) * BCH + ((4 * st + h) ^ gemm_swz<BCH>(fr))) * 16);
        u32x4_t bf[TJ], af[TH];
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:%c10\n\t"
            "ds_read_b128 %2, %8 offset:%c11\n\t"
            "ds_read_b128 %3, %8 offset:%c12\n\t"
            "ds_read_b128 %4, %9\n\t"
            "ds_read_b128 %5, %9 offset:%c13\n\t"
            "ds_read_b128 %6, %9 offset:%c14\n\t"
            "ds_read_b128 %7, %9 offset:%c15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(bf[0]), "=&v"(bf[1]), "=&v"(bf[2]), "=&v"(bf[3]), "=&v"(af[0]), "=&v"(af[1]),
              "=&v"(af[2]), "=&v"(af[3])
            : "v"(ba), "v"(aa), "i"(BR), "i"(2 * BR), "i"(3 * BR), "i"(AR), "i"(2 * AR), "i"(3 * AR)
            : "memory");
#pragma unroll
        for (int ii = 0; ii < TH; ++ii)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[ii]),
                                                                 __builtin_bit_cast(bf16x8_t, bf[j]), acc[ii][j], 0, 0, 0);
        asm volatile(
            "ds_read_b128 %0, %4 offset:%c5\n\t"
            "ds_read_b128 %1, %4 offset:%c6\n\t"
            "ds_read_b128 %2, %4 offset:%c7\n\t"
            "ds_read_b128 %3, %4 offset:%c8\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3])
            : "v"(aa), "i"(4 * AR), "i"(5 * AR), "i"(6 * AR), "i"(7 * AR)
            : "memory");
#pragma unroll
        for (int ii = 0; ii < TH; ++ii)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[TH + ii][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[ii]),
                                                                      __builtin_bit_cast(bf16x8_t, bf[j]),
                                                                      acc[TH + ii][j], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();  // the trailing clamped slab loads land before LDS is reused or released
  asm volatile("" ::: "memory");
  // lane holds C[4 * (lane >> 4) + v][lane & 15] of each 16x16 tile
  if constexpr (EPI == EPI_ROWSQ) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const bool nv = n0 + wn * WTN + j * 16 + (lane & 15) < N;  // clamped B rows past N
          sq = __builtin_fmaf(acc[i][j][v], nv ? acc[i][j][v] : 0.0f, sq);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
        if ((lane & 15) == 0) red[wn][wm * WTM + i * 16 + 4 * (lane >> 4) + v] = sq;
      }
    __syncthreads();
    for (int r = tid; r < BM; r += NT) {
      const int64_t m = m0 + r;
      float a = 0.f;
#pragma unroll
      for (int q = 0; q < WN; ++q) a += red[q][r];
      if (m < M) g.out[m * g.ld_out + tn] = a;
    }
  } else {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + v;
        float sa = 1.0f;
        if constexpr (MODE == GM_FP8) sa = m < M ? g.scale_a[m] : 0.0f;
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int64_t n = n0 + wn * WTN + j * 16 + (lane & 15);
          float c = acc[i][j][v];
          if constexpr (MODE == GM_FP8) c = c * sa * (n < N ? g.scale_b[n] : 0.0f);
          if (m < M && n < N) g.out[m * g.ld_out + n] = c;
        }
      }
  }
}

inline int64_t gemm_tiles(int64_t M, int64_t N) {
  return ((M + kGM - 1) / kGM) * ((N + kGN - 1) / kGN);
}

template <int MODE, int EPI>
inline hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm_dma<MODE, EPI>), dim3((unsigned)gemm_tiles(g.M, g.N)), dim3(512), 0,
                     s, g);
  return hipGetLastError();
}

}  // namespace sparq24
