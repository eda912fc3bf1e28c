// Operator-level error of Y = A B^T [PD §2: accuracy is the relative error
// of the operator's output against a full-precision reference output].
//
// For a side (dense, 2:4 or pairwise 4:8, with a quantizer of the values it
// keeps) the output error is Yhat - Y = (Ahat - A) B^T, so no output is ever
// stored: one kernel writes D = Ahat - A of every row as an fp32-exact
// bf16 pair (hi, lo) with D ~= hi + lo, laid out [M][2K] = [hi | lo], and an
// MFMA GEMM of that [M][2K] operand against [B | B] reduces sum_n C[m][n]^2
// per row and 128-column tile.  The reference energy sum_n Y[m][n]^2 is the
// same GEMM on A itself.  A and B are bf16 (the GEMM operand type).
#include "dispatch.hpp"
#include "gemm_tile.hpp"

namespace sparq24 {

// ---------------------------------------------------------------------------
// D = Ahat - A for one side, bf16 rows.  Per element the residual is one fp32
// FMA (code * scale - x, a single rounding; -x where the element is pruned,
// 0 where a kept value is stored as is); hi = bf16(D), lo = bf16(D - hi)
// (D - hi is exact in fp32), so hi + lo is within 2^-17 |D| of D.
// ---------------------------------------------------------------------------
__device__ inline uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Residuals of 4 kept values (one unit) under a block format spanning 4 (NV)
// or 8 (MX) adjacent lanes' units; every lane of the wave must call this.
__device__ inline void kept_block_delta4(bool nv, const float* v, float s_t, float gnv,
                                         float* d) {
  uint32_t am = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t a = __float_as_uint(v[e]) & 0x7FFFFFFFu;
    am = am > a ? am : a;
  }
  uint32_t w = (uint32_t)__shfl_xor((int)am, 1, 64);
  am = am > w ? am : w;
  w = (uint32_t)__shfl_xor((int)am, 2, 64);
  am = am > w ? am : w;
  w = (uint32_t)__shfl_xor((int)am, 4, 64);
  const uint32_t am8 = am > w ? am : w;
  if (nv) {
    const uint32_t bc = enc_e4m3(__uint_as_float(am) * gnv);
    const float bval = dec_e4m3(bc);
    const float dd = bval * s_t;
    const float inv = dd > 0.0f ? 1.0f / dd : 0.0f;
    const uint32_t pk = enc_e2m1_x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = __builtin_fmaf(dec_e2m1((pk >> (4 * e)) & 0xFu) * bval, s_t, -v[e]);
  } else {
    const int ex = mx_exponent(am8);
    const float X = __builtin_ldexpf(1.0f, ex);
    const uint32_t pk = enc_e2m1_x4(__builtin_ldexpf(v[0], -ex), __builtin_ldexpf(v[1], -ex),
                                    __builtin_ldexpf(v[2], -ex), __builtin_ldexpf(v[3], -ex));
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = __builtin_fmaf(dec_e2m1((pk >> (4 * e)) & 0xFu), X, -v[e]);
  }
}

template <int TEAM, int UPL>
SPARQ24_ROW_KERNEL void k_side_delta(RowGeom g, SideParams sp, uint16_t* __restrict__ out) {
  __shared__ uint32_t redu[kBlock / 64];
  float s_t = 0.f, gnv = 0.f;
  if (sp.fmt == CF_NV) nv_tensor_scales(block_tensor_amax(sp.tamax_in, sp.partials, sp.nparts, redu),
                                        s_t, gnv);
  const int64_t K = g.nunits * 8;
  for_each_row<BF16T, TEAM, UPL>(g, [&](Unit<BF16T>(&u)[UPL], int64_t row, int t) {
    uint32_t sel[UPL], km[UPL];
    uint32_t am = 0;  // largest |x| over what the quantizer sees, bf16 bits
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      if (sp.pattern == PAT_24) {
        sel[j] = select16(u[j].w).mb;
        const uint32_t n0 = sel[j] & 0xFu, n1 = sel[j] >> 4;
        km[j] = (1u << (n0 & 3u)) | (1u << (n0 >> 2)) | (16u << (n1 & 3u)) | (16u << (n1 >> 2));
      } else if (sp.pattern == PAT_48) {
        sel[j] = select_pairs48(u[j]);
        km[j] = pairs48_mask(sel[j]);
      } else {
        sel[j] = 0;
        km[j] = 0xFFu;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = ((km[j] >> e) & 1u) ? u[j].absbits(e) : 0u;
        am = am > a ? am : a;
      }
    }
    am = team_max_u32<TEAM>(am, redu);
    const bool perrow = sp.fmt == CF_INT8 || sp.fmt == CF_INT16 || sp.fmt == CF_FP8;
    float s = 0.f, inv = 0.f;
    if (perrow) row_scale(BF16T::to_f32(am), sp.qmax, s, inv);
    uint16_t* hrow = out + row * (2 * K);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = (int64_t)j * TEAM + t;
      float v[8], d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = u[j].f(e);
      if (sp.pattern == PAT_DENSE) {
        if (perrow) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float c[4];
            qdq_row4(sp.fmt, inv, sp.qmax, v + 4 * h, c);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[4 * h + e] = __builtin_fmaf(c[e], s, -v[4 * h + e]);
          }
        } else {  // MX: 32 elements = 4 units; NV: 16 elements = 2 units
          uint32_t bm = unpack_max16(unit_absmax16_packed(u[j].w, 0u)) << 16;  // fp32 bits
          uint32_t w = (uint32_t)__shfl_xor((int)bm, 1, 64);
          bm = bm > w ? bm : w;
          w = (uint32_t)__shfl_xor((int)bm, 2, 64);
          const uint32_t bm4 = bm > w ? bm : w;
          float y[8];
          if (sp.fmt == CF_NV) {
            const uint32_t bc = enc_e4m3(__uint_as_float(bm) * gnv);
            const float bval = dec_e4m3(bc);
            const float dd = bval * s_t;
            const float rinv = dd > 0.0f ? 1.0f / dd : 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = v[e] * rinv;
            const uint32_t pk = enc_e2m1_x8(y);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              d[e] = __builtin_fmaf(dec_e2m1((pk >> (4 * e)) & 0xFu) * bval, s_t, -v[e]);
          } else {
            const int ex = mx_exponent(bm4);
            const float X = __builtin_ldexpf(1.0f, ex);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf(v[e], -ex);
            const uint32_t pk = enc_e2m1_x8(y);
#pragma unroll
            for (int e = 0; e < 8; ++e) d[e] = __builtin_fmaf(dec_e2m1((pk >> (4 * e)) & 0xFu), X, -v[e]);
          }
        }
      } else {
        // kept values in position order, their residuals, then back to positions
        const Kept<BF16T> kp = sp.pattern == PAT_48 ? gather_pairs48(u[j], sel[j]) : gather_kept(u[j], sel[j]);
        const float kv[4] = {kp.f(0), kp.f(1), kp.f(2), kp.f(3)};
        float kd[4] = {0.f, 0.f, 0.f, 0.f};
        if (perrow) {
          float c[4];
          qdq_row4(sp.fmt, inv, sp.qmax, kv, c);
#pragma unroll
          for (int e = 0; e < 4; ++e) kd[e] = __builtin_fmaf(c[e], s, -kv[e]);
        } else if (sp.fmt == CF_MX || sp.fmt == CF_NV) {
          kept_block_delta4(sp.fmt == CF_NV, kv, s_t, gnv, kd);
        }
        uint32_t pos[4];
        if (sp.pattern == PAT_48) {
          const uint32_t p0 = sel[j] & 3u, p1 = sel[j] >> 2;
          pos[0] = 2 * p0; pos[1] = 2 * p0 + 1; pos[2] = 2 * p1; pos[3] = 2 * p1 + 1;
        } else {
          const uint32_t n0 = sel[j] & 0xFu, n1 = sel[j] >> 4;
          pos[0] = n0 & 3u; pos[1] = n0 >> 2; pos[2] = 4 + (n1 & 3u); pos[3] = 4 + (n1 >> 2);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float r = -v[e];  // pruned
#pragma unroll
          for (int q = 0; q < 4; ++q) r = pos[q] == (uint32_t)e ? kd[q] : r;
          d[e] = r;
        }
      }
      if (row < g.nrows && i < g.nunits) {
        uint32_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = bf16_rne(d[e]);
          lo[e] = bf16_rne(d[e] - __uint_as_float(hi[e] << 16));
        }
        st4(hrow + i * 8, hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16),
            hi[6] | (hi[7] << 16));
        st4(hrow + K + i * 8, lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16),
            lo[6] | (lo[7] << 16));
      }
    }
  });
}

// out[m][col] = sum over tiles of part[col][m][tile] in fp64, fixed order.
__global__ __launch_bounds__(kBlock) void k_rowsq_final(const float* __restrict__ part, int64_t M,
                                                        int64_t ntiles, int ncols,
                                                        double* __restrict__ out) {
  // one wave per (column, row): the lanes stride the row's tile partials
  // (contiguous), then a fixed-order wave sum
  const int64_t item = (int64_t)blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (item >= M * ncols) return;  // whole waves
  const int c = (int)(item / M);
  const int64_t m = item % M;
  const float* p = part + ((int64_t)c * M + m) * ntiles;
  double a = 0.0;
  for (int64_t q = lane; q < ntiles; q += 64) a += (double)p[q];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) out[m * ncols + c] = a;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int64_t gemm_col_tiles(int64_t N) { return (N + kGN - 1) / kGN; }

hipError_t launch_side_delta(const RowDesc& d, const SideParams& sp, void* out, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const RowGeom g{d.x, d.R, d.B * d.R, nunits, d.bs, d.rs, d.rot};
  return with_row_variant<0>(nunits, [&]<int TEAM, int UPL>() {
    hipLaunchKernelGGL((k_side_delta<TEAM, UPL>), persistent_grid(g.nrows, TEAM), dim3(kBlock), 0,
                       s, g, sp, (uint16_t*)out);
    return hipGetLastError();
  });
}

hipError_t launch_gemm_rowsq(const void* A, int64_t lda, const void* B, int64_t ldb, int64_t M,
                             int64_t N, int64_t Kp, int64_t K, float* part, hipStream_t s) {
  const GemmArgs g{A, lda, nullptr, 0, B, ldb, M, N, Kp, K, part, gemm_col_tiles(N), nullptr,
                   nullptr};
  return launch_gemm<GM_BF16, EPI_ROWSQ>(g, s);
}

hipError_t launch_rowsq_final(const float* part, int64_t M, int64_t ntiles, int ncols, double* out,
                              hipStream_t s) {
  const int64_t waves = M * ncols, per = kBlock / 64;
  hipLaunchKernelGGL(k_rowsq_final, dim3((unsigned)((waves + per - 1) / per)), dim3(kBlock), 0, s,
                     part, M, ntiles, ncols, out);
  return hipGetLastError();
}

}  // namespace sparq24
