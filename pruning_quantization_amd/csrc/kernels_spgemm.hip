// GEMMs that consume the operands the prune and quantize calls produce
// [PD §3: the 2:4 side runs a sparse GEMM on the pruned and compressed
// operand; its rival a dense GEMM].  The sparse one reads the compressed
// layout (kept values + group metadata) directly with gfx950's sparse MFMA;
// the dense ones are the same tile on uncompressed bf16 rows and on the e4m3
// codes of the dense FP8 rival (per-row scales applied to the output).
// Both write C = A B^T as fp32.  Tile and schedule: gemm_tile.hpp.
#include "dispatch.hpp"
#include "gemm_tile.hpp"

namespace sparq24 {

hipError_t launch_sparse_gemm(const void* values, const uint8_t* meta, int64_t M, int64_t K,
                              const void* B, int64_t ldb, int64_t N, float* C, int64_t ldc,
                              hipStream_t s) {
  const GemmArgs g{values, K / 2, meta, K / 8, B, ldb, M, N, K, K, C, ldc, nullptr, nullptr};
  return launch_gemm<GM_SPARSE, EPI_STORE>(g, s);
}

hipError_t launch_dense_gemm(const void* A, int64_t lda, int64_t M, int64_t K, const void* B,
                             int64_t ldb, int64_t N, float* C, int64_t ldc, hipStream_t s) {
  const GemmArgs g{A, lda, nullptr, 0, B, ldb, M, N, K, K, C, ldc, nullptr, nullptr};
  return launch_gemm<GM_BF16, EPI_STORE>(g, s);
}

// e4m3 codes [M][K] and [N][K] (row strides in bytes), per-row scales.
hipError_t launch_fp8_gemm(const void* A, int64_t lda, const float* sa, int64_t M, int64_t K,
                           const void* B, int64_t ldb, const float* sb, int64_t N, float* C,
                           int64_t ldc, hipStream_t s) {
  const GemmArgs g{A, lda / 2, nullptr, 0, B, ldb / 2, M, N, K / 2, K / 2, C, ldc, sa, sb};
  return launch_gemm<GM_FP8, EPI_STORE>(g, s);
}

}  // namespace sparq24
