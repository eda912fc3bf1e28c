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
// 64-deep K slabs double-buffered in LDS with padded rows (the 16 rows a
// fragment read touches fall in distinct banks), fp32 accumulation.  A
// lane's k values of a fragment are the same positions for A and B, which is
// all the dense product needs.  Epilogue: per-row sums of C^2 over the tile's
// columns (EPI_ROWSQ) or C stored as fp32 (EPI_STORE).  GM_FP8 runs the same
// tile on e4m3 codes with v_mfma_f32_16x16x128_f8f6f4 and applies the per-row
// scales of both operands when storing C.
#pragma once

#include "device_common.hpp"

namespace sparq24 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kGK = 64, kGPad = 8;
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

// Strides and depths of GM_FP8 are counted in pairs of codes (16-bit units),
// so a 64-unit slab is 128 codes and every load path is shared.
template <int BM, int BN, int WTM, int WTN, int MODE, int EPI>
__global__ __launch_bounds__((BM / WTM) * (BN / WTN) * 64) void k_gemm(GemmArgs g) {
  constexpr bool SPARSE = MODE == GM_SPARSE;
  constexpr int WN = BN / WTN, NT = (BM / WTM) * WN * 64;
  constexpr int TI = WTM / 16, TJ = WTN / 16;
  constexpr int AW = SPARSE ? kGK / 2 : kGK;           // A elements per row per slab
  constexpr int QA = BM * (AW / 8) / NT, QB = BN * 8 / NT;  // 16-byte chunks per thread
  static_assert(QA * NT == BM * (AW / 8) && QB * NT == BN * 8, "tile / thread mismatch");
  static_assert(!SPARSE || BM <= NT, "one metadata row per thread");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][AW + kGPad];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN][kGK + kGPad];
  __shared__ __attribute__((aligned(16))) uint2 sM[SPARSE ? 2 : 1][SPARSE ? BM : 1];
  __shared__ float red[EPI == EPI_ROWSQ ? WN : 1][BM];
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

  uint4 ra[QA], rb[QB];
  uint2 rm = make_uint2(0, 0);
  // Branch-free slab loads (the loop body stays one scheduling region): rows
  // past the edge read the last row and are zeroed by a select.
  auto gload = [&](int64_t k0) {
    const int64_t kb0 = k0 % K;
    constexpr int CPR = AW / 8;  // 16-byte chunks per A row
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + NT * q, r = c / CPR, cc = c % CPR;
      const int64_t m = m0 + r;
      const int64_t ak = SPARSE ? k0 / 2 : k0;
      const uint4 v = *reinterpret_cast<const uint4*>(A + (m < M ? m : M - 1) * g.lda + ak + cc * 8);
      ra[q] = m < M ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int c = tid + NT * q, r = c >> 3, cc = c & 7;
      const int64_t n = n0 + r;
      const uint4 v = *reinterpret_cast<const uint4*>(B + (n < N ? n : N - 1) * g.ldb + kb0 + cc * 8);
      rb[q] = n < N ? v : make_uint4(0, 0, 0, 0);
    }
    if constexpr (SPARSE) {
      if (tid < BM) {  // 8 metadata bytes = the 16 groups of the slab
        const int64_t m = m0 + tid;
        const uint2 v = *reinterpret_cast<const uint2*>(g.meta + (m < M ? m : M - 1) * g.ldm + k0 / 8);
        rm = m < M ? v : make_uint2(0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
    constexpr int CPR = AW / 8;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + NT * q, r = c / CPR, cc = c % CPR;
      *reinterpret_cast<uint4*>(&sA[buf][r][cc * 8]) = ra[q];
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int c = tid + NT * q, r = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&sB[buf][r][cc * 8]) = rb[q];
    }
    if constexpr (SPARSE) {
      if (tid < BM) sM[buf][tid] = rm;
    }
  };
  f32x4_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t nk = g.Kp / kGK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    // the next slab (the last one again on the final step: harmless, never read)
    gload((kt + 1 < nk ? kt + 1 : kt) * kGK);
    if constexpr (SPARSE) {
      // one 64-deep sparse MFMA per tile: A lane group h = lane / 16 covers
      // logical k 16h .. 16h + 15 (8 kept values, metadata bytes 2h, 2h + 1).
      // Row tiles in two halves keep the live fragments within budget.
      const int h = lane >> 4;
      bf16x16_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        // B: lane group h holds logical k 8h .. 8h + 7 and 32 + 8h .. 32 + 8h + 7
        const uint16_t* br = &sB[cur][wn * WTN + j * 16 + (lane & 15)][0];
        const bf16x8_t lo = *reinterpret_cast<const bf16x8_t*>(br + h * 8);
        const bf16x8_t hi = *reinterpret_cast<const bf16x8_t*>(br + 32 + h * 8);
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
auto do_half = [&]<int half>() {
        constexpr int TH = TI / 2;
        bf16x8_t af[TH];
        int ix[TH];
#pragma unroll
        for (int ii = 0; ii < TH; ++ii) {
          const int r = wm * WTM + (half * TH + ii) * 16 + (lane & 15);
          af[ii] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][r][h * 8]);
          const uint2 mm = sM[cur][r];
          ix[ii] = (int)(((h < 2 ? mm.x : mm.y) >> (16 * (h & 1))) & 0xFFFFu);
        }
#pragma unroll
        for (int ii = 0; ii < TH; ++ii)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[half * TH + ii][j] = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
                af[ii], bfr[j], acc[half * TH + ii][j], ix[ii], 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * TH + (half == 0 ? 2 * TJ : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TH * TJ, 0);
      };
      do_half.template operator()<0>();
      do_half.template operator()<1>();
    } else if constexpr (MODE == GM_FP8) {
      // one 128-deep e4m3 MFMA per tile; a lane's 32 codes are the same k
      // positions for A and B.  Row tiles in two halves (register budget).
      const int h = lane >> 4;
      auto frag = [&](const uint16_t* p) {
        const uint4 x0 = *reinterpret_cast<const uint4*>(p), x1 = *reinterpret_cast<const uint4*>(p + 8);
        return i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      };
      i32x8_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[j] = frag(&sB[cur][wn * WTN + j * 16 + (lane & 15)][h * 16]);
auto do_half = [&]<int half>() {
        constexpr int TH = TI / 2;
        i32x8_t af[TH];
#pragma unroll
        for (int ii = 0; ii < TH; ++ii)
          af[ii] = frag(&sA[cur][wm * WTM + (half * TH + ii) * 16 + (lane & 15)][h * 16]);
#pragma unroll
        for (int ii = 0; ii < TH; ++ii)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[half * TH + ii][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[ii], bfr[j], acc[half * TH + ii][j], 0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * TH + (half == 0 ? 2 * TJ : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TH * TJ, 0);
      };
      do_half.template operator()<0>();
      do_half.template operator()<1>();
    } else {
      bf16x8_t af[TI], bfr[TJ];
#pragma unroll
      for (int st = 0; st < kGK / 32; ++st) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
          af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[cur][wm * WTM + i * 16 + (lane & 15)][st * 32 + (lane >> 4) * 8]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[cur][wn * WTN + j * 16 + (lane & 15)][st * 32 + (lane >> 4) * 8]);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        // all fragment reads of the step issue before its MFMAs (one wait)
        __builtin_amdgcn_sched_group_barrier(0x100, TI + TJ, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TI * TJ, 0);
      }
    }
    sstore(cur ^ 1);
    __syncthreads();
  }
  // lane holds C[4 * (lane >> 4) + v][lane & 15] of each 16x16 tile
  if constexpr (EPI == EPI_ROWSQ) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sq = 0.f;
#pragma unroll
        for (int j = 0; j < TJ; ++j) sq = __builtin_fmaf(acc[i][j][v], acc[i][j][v], sq);
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
  hipLaunchKernelGGL((k_gemm<kGM, kGN, 128, 64, MODE, EPI>), dim3((unsigned)gemm_tiles(g.M, g.N)),
                     dim3(512), 0, s, g);
  return hipGetLastError();
}

}  // namespace sparq24
