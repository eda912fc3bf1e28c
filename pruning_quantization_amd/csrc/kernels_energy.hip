// Energy reductions that score 2:4 against dense quantization.
//
// Method: Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com English
// summary), [PD §4]: the 2:4 energy loss (dropped sum of squares over the
// total), the error energy of quantizing the kept values, the dense error
// energy at equal bits, their exact additivity once the mask is fixed, and
// the predicted R = sqrt(E_2:4 / E_dense).
//
// One read of the operand per call: a team holds its row in registers,
// selects the 2:4 mask, evaluates every requested quantizer on the fly
// (nothing is written but fp64 per-row partial sums), and a second small
// pass reduces rows per block in a fixed order.
#include "dispatch.hpp"

namespace sparq24 {

__device__ inline float block_tensor_amax_e(const float* tamax_in, const uint32_t* partials,
                                            int nparts, uint32_t* lds) {
  if (tamax_in) return *tamax_in;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += kBlock) m = m > partials[i] ? m : partials[i];
  m = team_max_u32<64>(m, lds);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int i = 1; i < kBlock / 64; ++i) r = r > lds[i] ? r : lds[i];
  return __uint_as_float(r);
}

__device__ inline int mx_exp_e(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  int fl;
  const uint32_t ex = amax_bits >> 23;
  if (ex) fl = (int)ex - 127;
  else fl = (31 - __builtin_clz(amax_bits)) - 149;
  int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// squared fp32 residual accumulated in fp64
__device__ inline void acc_err(double& acc, float xhat_unit, float scale, float v) {
  const float e = __builtin_fmaf(xhat_unit, scale, -v);  // one rounding of code*s - x
  acc = __builtin_fma((double)e, (double)e, acc);
}

template <class DT, int TEAM, int UPL, bool WANDA>
__global__ __launch_bounds__(kBlock) void k_energy_rows(
    const char* __restrict__ x, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    const float* __restrict__ norm, EnergyParams p, double* __restrict__ rowpart,
    int64_t nrows_total) {
  __shared__ uint32_t redu[kBlock / 64];
  __shared__ double redd[kBlock / 64];
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  const bool active = r < R;
  const char* xr = x + b * bs + r * rs;
  const int64_t orow = b * R + r;

  bool any_nv = false;
  for (int q = 0; q < p.dense.n; ++q) any_nv |= (p.dense.fmt[q] == CF_NV);
  float s_t = 0.f, g = 0.f;
  if (any_nv) {
    const float T = block_tensor_amax_e(p.nv_tamax, p.nv_partials, p.n_partials, redu);
    if (T >= 0x1p-64f) { s_t = T / 2688.0f; g = 448.0f / T; }
  }

  Unit<DT> u[UPL];
  uint32_t km[UPL];  // 8-bit kept mask per unit
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int64_t i = (int64_t)j * TEAM + t;
    if (active && i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
    else zero_unit(u[j]);
  }
  double x2 = 0.0, drop = 0.0;
  uint32_t amd = 0, amk = 0;
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int64_t i = (int64_t)j * TEAM + t;
    km[j] = 0;
    if (i < nunits) {
      float n8[8];
      if constexpr (WANDA) {
        const float4* np = reinterpret_cast<const float4*>(norm + i * 8);
        float4 a = np[0], c = np[1];
        n8[0] = a.x; n8[1] = a.y; n8[2] = a.z; n8[3] = a.w;
        n8[4] = c.x; n8[5] = c.y; n8[6] = c.z; n8[7] = c.w;
      }
      const uint32_t n0 = select_group<DT, WANDA>(u[j], 0, n8);
      const uint32_t n1 = select_group<DT, WANDA>(u[j], 1, n8 + 4);
      km[j] = (1u << (n0 & 3u)) | (1u << (n0 >> 2)) | (16u << (n1 & 3u)) | (16u << (n1 >> 2));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = u[j].f(e);
      const double v2 = (double)v * (double)v;  // exact
      x2 += v2;
      const uint32_t a = u[j].absbits(e);
      amd = amd > a ? amd : a;
      if ((km[j] >> e) & 1u) amk = amk > a ? amk : a;
      else drop += v2;
    }
  }
  amd = team_max_u32<TEAM>(amd, redu);
  amk = team_max_u32<TEAM>(amk, redu);
  x2 = team_sum_f64<TEAM>(x2, redd);
  drop = team_sum_f64<TEAM>(drop, redd);
  const int ncols = 2 + p.kept.n + p.dense.n;
  const bool writer = active && t == 0;
  if (writer) {
    rowpart[0 * nrows_total + orow] = x2;
    rowpart[1 * nrows_total + orow] = drop;
  }
  const float famk = DT::to_f32(amk), famd = DT::to_f32(amd);

  // kept-side quantizers (per-row scale from the kept maximum)
  for (int q = 0; q < p.kept.n; ++q) {
    const int fmt = p.kept.fmt[q];
    const float qmax = p.kept.qmax[q];
    double acc = 0.0;
    if (fmt != CF_NONE) {
      float s, inv;
      row_scale(famk, qmax, s, inv);
#pragma unroll
      for (int j = 0; j < UPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((km[j] >> e) & 1u) {
            const float v = u[j].f(e);
            const float y = v * inv;
            const float c = (fmt == CF_FP8) ? dec_e4m3(enc_e4m3(y)) : enc_int(y, qmax);
            acc_err(acc, c, s, v);
          }
    }
    acc = team_sum_f64<TEAM>(acc, redd);
    if (writer) rowpart[(int64_t)(2 + q) * nrows_total + orow] = acc;
  }

  // dense quantizers
  for (int q = 0; q < p.dense.n; ++q) {
    const int fmt = p.dense.fmt[q];
    const float qmax = p.dense.qmax[q];
    double acc = 0.0;
    if (fmt == CF_INT8 || fmt == CF_INT16 || fmt == CF_FP8) {
      float s, inv;
      row_scale(famd, qmax, s, inv);
#pragma unroll
      for (int j = 0; j < UPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = u[j].f(e);
          const float y = v * inv;
          const float c = (fmt == CF_FP8) ? dec_e4m3(enc_e4m3(y)) : enc_int(y, qmax);
          acc_err(acc, c, s, v);
        }
    } else if (fmt == CF_MX || fmt == CF_NV) {
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        uint32_t am = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = u[j].absbits(e);
          am = am > a ? am : a;
        }
        am = __float_as_uint(DT::to_f32(am));
        uint32_t w = (uint32_t)__shfl_xor((int)am, 1, 64);
        am = am > w ? am : w;
        if (fmt == CF_MX) {
          w = (uint32_t)__shfl_xor((int)am, 2, 64);
          am = am > w ? am : w;
          const int ex = mx_exp_e(am);
          const float X = __builtin_ldexpf(1.0f, ex);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = u[j].f(e);
            const float c = dec_e2m1(enc_e2m1(__builtin_ldexpf(v, -ex)));
            acc_err(acc, c, X, v);
          }
        } else {
          const uint32_t bc = enc_e4m3(__uint_as_float(am) * g);
          const float bval = dec_e4m3(bc);
          const float d = bval * s_t;
          const float inv = d > 0.0f ? 1.0f / d : 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = u[j].f(e);
            const float c = dec_e2m1(enc_e2m1(v * inv));
            acc_err(acc, c * bval, s_t, v);
          }
        }
      }
    }
    acc = team_sum_f64<TEAM>(acc, redd);
    if (writer) rowpart[(int64_t)(2 + p.kept.n + q) * nrows_total + orow] = acc;
  }
  (void)ncols;
}

// Sum of rows [blk*rpb, min(nrows, (blk+1)*rpb)) of one column: grid (nblk, ncols).
__global__ __launch_bounds__(kBlock) void k_energy_colsum(const double* __restrict__ rowpart,
                                                          int64_t nrows, int64_t rpb,
                                                          double* __restrict__ sums, int ncols) {
  __shared__ double sh[kBlock];
  const int64_t blk = blockIdx.x;
  const int c = blockIdx.y;
  const int64_t r0 = blk * rpb;
  const int64_t r1 = (r0 + rpb) < nrows ? (r0 + rpb) : nrows;
  const double* col = rowpart + (int64_t)c * nrows;
  double acc = 0.0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kBlock) acc += col[r];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kBlock / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sums[blk * ncols + c] = sh[0];
}

__global__ __launch_bounds__(kBlock) void k_energy_combine(const double* __restrict__ sums,
                                                           int64_t nblk, FinalizeParams f,
                                                           double* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (blk >= nblk) return;
  const double* sb = sums + blk * f.ncols;
  if (f.mode == 0) {
    double* o = out + blk * 4;
    o[0] = sb[0];
    o[1] = sb[1];
    o[2] = sb[f.kcol[0]];
    o[3] = sb[f.dcol[0]];
  } else {
    const double tot = sb[0];
    for (int p = 0; p < f.npairs; ++p) {
      double* o = out + (blk * f.npairs + p) * 5;
      const double ep = sb[1] / tot;
      const double eq = sb[f.kcol[p]] / tot;
      const double e24 = ep + eq;
      const double ed = sb[f.dcol[p]] / tot;
      o[0] = ep;
      o[1] = eq;
      o[2] = e24;
      o[3] = ed;
      o[4] = __builtin_sqrt(e24 / ed);
    }
  }
}

hipError_t launch_energy_rows(const RowDesc& d, bool wanda, const float* norm,
                              const EnergyParams& p, double* rowpart, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const int64_t nrows = d.B * d.R;
  return with_dtype(d.dtype, [&]<class DT>() {
    return with_row_variant(nunits, [&]<int TEAM, int UPL>() {
      if (wanda)
        hipLaunchKernelGGL((k_energy_rows<DT, TEAM, UPL, true>), row_grid(d, TEAM), dim3(kBlock),
                           0, s, d.x, d.R, nunits, d.bs, d.rs, norm, p, rowpart, nrows);
      else
        hipLaunchKernelGGL((k_energy_rows<DT, TEAM, UPL, false>), row_grid(d, TEAM),
                           dim3(kBlock), 0, s, d.x, d.R, nunits, d.bs, d.rs, norm, p, rowpart,
                           nrows);
      return hipGetLastError();
    });
  });
}

hipError_t launch_energy_finalize(const double* rowpart, int64_t nrows, int64_t rows_per_block,
                                  int64_t nblk, const FinalizeParams& f, double* out,
                                  hipStream_t s) {
  // the block sums live right after the row partials in the workspace
  double* sums = const_cast<double*>(rowpart) + (int64_t)f.ncols * nrows;
  hipLaunchKernelGGL(k_energy_colsum, dim3((unsigned)nblk, (unsigned)f.ncols), dim3(kBlock), 0, s,
                     rowpart, nrows, rows_per_block, sums, f.ncols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_energy_combine, dim3((unsigned)((nblk + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, s, sums, nblk, f, out);
  return hipGetLastError();
}

}  // namespace sparq24
