// GEMMs that consume the operands the prune and quantize calls produce
// [PD §3: the 2:4 side runs a sparse GEMM on the pruned and compressed
// operand; its rival a dense GEMM].  The sparse one reads the compressed
// layout (kept values + group metadata) directly with gfx950's sparse MFMA;
// the dense one is the same tile on uncompressed rows, for comparison.
// Both write C = A B^T as fp32.  Tile and schedule: gemm_tile.hpp.
#include "dispatch.hpp"
#include "gemm_tile.hpp"

namespace sparq24 {

hipError_t launch_sparse_gemm(const void* values, const uint8_t* meta, int64_t M, int64_t K,
                              const void* B, int64_t ldb, int64_t N, float* C, int64_t ldc,
                              hipStream_t s) {
  const GemmArgs g{values, K / 2, meta, K / 8, B, ldb, M, N, K, K, C, ldc};
  return launch_gemm<true, EPI_STORE>(g, s);
}

hipError_t launch_dense_gemm(const void* A, int64_t lda, int64_t M, int64_t K, const void* B,
                             int64_t ldb, int64_t N, float* C, int64_t ldc, hipStream_t s) {
  const GemmArgs g{A, lda, nullptr, 0, B, ldb, M, N, K, K, C, ldc};
  return launch_gemm<false, EPI_STORE>(g, s);
}

}  // namespace sparq24
