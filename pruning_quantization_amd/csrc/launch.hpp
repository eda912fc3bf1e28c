// Internal launcher interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sparq24 {

// Code containers of per-row formats.
enum CodeFmt : int { CF_INT8 = 0, CF_INT16 = 1, CF_FP8 = 2, CF_NONE = 3, CF_MX = 4, CF_NV = 5 };

// One operand as the kernels see it: B x R vectors of K elements.
// Block Hadamard rotation along K applied to an operand as it is loaded:
// n = block size (0 = none, else a power of two in 8..512), c = fp64 1/sqrt(n).
struct Rot {
  int n;
  double c;
};

struct RowDesc {
  const char* x;
  int dtype;            // sparq24_dtype
  int64_t B, R, K;
  int64_t bs, rs, ks;   // strides in BYTES
  bool kcontig;         // ks == element size
  bool flat;            // fully contiguous: bs == R*rs, rs == K*esize
  Rot rot;              // rotation applied on load (n == 0: none)
};

// Sparsity pattern: element-wise 2:4 or pairwise 4:8.
enum Pattern : int { PAT_24 = 0, PAT_48 = 1, PAT_DENSE = 2 };

// One side of an operator-error comparison (the operand as a GEMM would
// consume it): selection pattern, quantizer of what it keeps, NVFP4 tensor
// maximum (given, or reduced from partial maxima).
struct SideParams {
  int pattern;
  int fmt;
  float qmax;
  const float* tamax_in;
  const uint32_t* partials;
  int nparts;
};

constexpr int kMaxQ = 16;

struct QList {
  int n;
  int fmt[kMaxQ];      // CodeFmt (CF_NONE/CF_INT8/CF_INT16/CF_FP8/CF_MX/CF_NV)
  float qmax[kMaxQ];
};

struct EnergyParams {
  QList kept, dense;
  int pairs48;                 // 1: pairwise 4:8 selection instead of 2:4
  // For each kept quantizer, the dense quantizer with the same row format and
  // qmax (INT/FP8), or -1.  Only the bf16 magnitude 2:4 kernel uses it: there
  // the kept maximum is the row maximum, so the twin's codes on the kept
  // positions are the kept-side codes.
  int kept_twin[kMaxQ];
  // INT quantizers (CF_INT8 / CF_INT16) by side, for the bf16 kernel's
  // chunked passes: every kept one, the kept ones without a twin, every
  // dense one (indices into kept / dense)
  int kept_int[kMaxQ], kept_int_solo[kMaxQ], dense_int[kMaxQ];
  int n_kept_int, n_kept_int_solo, n_dense_int;
  const float* nv_tamax;       // device T for NVFP4 (or null -> reduce partials)
  const uint32_t* nv_partials; // fp32 bit patterns of partial maxima
  int n_partials;
  // NVFP4 on kept values: T over the kept values, same protocol
  const float* kept_nv_tamax;
  const uint32_t* kept_nv_partials;
  int n_kept_partials;
  // Dense NVFP4 deferred to launch_energy_nv_dense: its column is written as
  // zero, and each workgroup writes the fp32 bits of the largest |x| of its
  // rows to max_out[workgroup] (the tensor maximum's partials).
  int defer_nv;
  uint32_t* max_out;
};

// Row kernels that hold a whole row in registers support up to this many units.
constexpr int64_t kMaxRowUnits = 4096;  // K <= 32768

hipError_t launch_prune_compress(const RowDesc& d, bool wanda, const float* norm, void* vals,
                                 uint8_t* meta, hipStream_t s);
hipError_t launch_prune_compress_pairs48(const RowDesc& d, void* vals, uint8_t* meta,
                                        hipStream_t s);
hipError_t launch_prune_quantize(const RowDesc& d, int pat, bool wanda, const float* norm,
                                 int cfmt, float qmax, void* codes, uint8_t* meta, float* scales,
                                 hipStream_t s);
// Kept values in MXFP4 / NVFP4 (cfmt CF_MX / CF_NV), either pattern.
hipError_t launch_prune_quant_fp4(const RowDesc& d, int pat, bool wanda, const float* norm,
                                  int cfmt, const float* tamax_in, const uint32_t* partials,
                                  int nparts, void* codes, uint8_t* meta, uint8_t* scales,
                                  float* ts_out, hipStream_t s);
// Partial maxima of |kept| (absmax_partial_count(d) of them).
hipError_t launch_kept_absmax_partials(const RowDesc& d, int pat, bool wanda, const float* norm,
                                       uint32_t* partials, hipStream_t s);
hipError_t launch_quant_rows(const RowDesc& d, int cfmt, float qmax, void* codes, float* scales,
                             hipStream_t s);
int absmax_partial_count(const RowDesc& d);
hipError_t launch_absmax_partials(const RowDesc& d, uint32_t* partials, hipStream_t s);
hipError_t launch_quant_mx(const RowDesc& d, void* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_quant_nv(const RowDesc& d, const float* tamax_in, const uint32_t* partials,
                           int nparts, void* codes, uint8_t* scales, float* ts_out,
                           hipStream_t s);
// Writes per-row partials rowpart[col][row], or (rows_per_block >= rows)
// one partial per team; *nparts receives the partial rows per column.
hipError_t launch_energy_rows(const RowDesc& d, bool wanda, const float* norm,
                              const EnergyParams& p, double* rowpart, int64_t rows_per_block,
                              int64_t* nparts, hipStream_t s, int64_t* grid_out = nullptr);
// The dense NVFP4 error energy of a bf16 operand (no rotation) into partial
// column col of rowpart, in the layout launch_energy_rows used with grid
// workgroups; the tensor maximum from the nparts partial maxima at parts.
hipError_t launch_energy_nv_dense(const RowDesc& d, const uint32_t* parts, int nparts, int col,
                                  double* rowpart, int64_t rows_per_block, int64_t grid,
                                  hipStream_t s);
int64_t energy_partial_rows(int64_t nrows);
int energy_max_workgroups();
// mode 0: out[blk][4] raw sums for pair 0; mode 1: out[blk][npairs][5] E's and R
struct FinalizeParams {
  int ncols;            // 2 + nkept + ndense
  int npairs;
  int kcol[kMaxQ];      // column of the kept error of pair p
  int dcol[kMaxQ];      // column of the dense error of pair p
  int mode;
};
int64_t energy_chunks_per_block(int64_t rows_per_block);
hipError_t launch_energy_finalize(const double* rowpart, int64_t nrows, int64_t rows_per_block,
                                  int64_t nblk, const FinalizeParams& f, double* csum, double* out,
                                  hipStream_t s);
int col_strips(const RowDesc& d);
hipError_t launch_col_l2norm(const RowDesc& d, double* partial, float* norms, hipStream_t s);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// Operator-level error: D = Ahat - A as bf16 hi | lo rows [M][2K]; GEMM with a
// per-row energy epilogue over 128-column tiles; fp64 row sums.
hipError_t launch_side_delta(const RowDesc& d, const SideParams& sp, void* out, hipStream_t s);
int64_t gemm_col_tiles(int64_t N);
hipError_t launch_gemm_rowsq(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                             int64_t N, int64_t Kp, int64_t K, float* part, hipStream_t s);
hipError_t launch_rowsq_final(const float* part, int64_t M, int64_t ntiles, int ncols, double* out,
                              hipStream_t s);
// C [M][N] fp32 (row stride ldc) = A B^T: A 2:4-compressed (values [M][K/2],
// meta [M][K/8]) on the sparse MFMA, or dense bf16 rows (row stride lda).
hipError_t launch_sparse_gemm(const void* values, const uint8_t* meta, int64_t M, int64_t K,
                              const void* B, int64_t ldb, int64_t N, float* C, int64_t ldc,
                              hipStream_t s);
hipError_t launch_dense_gemm(const void* A, int64_t lda, int64_t M, int64_t K, const void* B,
                             int64_t ldb, int64_t N, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_fp8_gemm(const void* A, int64_t lda, const float* sa, int64_t M, int64_t K,
                           const void* B, int64_t ldb, const float* sb, int64_t N, float* C,
                           int64_t ldc, hipStream_t s);
// Rotated copy of a K-contiguous operand (d.rot) into dense [B][R][K] `out`.
hipError_t launch_hadamard(const RowDesc& d, void* out, hipStream_t s);
// Transposed operand -> dense [B][R][K] copy in `out` (B*R*K elements).
hipError_t launch_transpose_rows(const RowDesc& d, void* out, hipStream_t s);

}  // namespace sparq24
