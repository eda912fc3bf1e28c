// Wanda input-channel norms and the plain-copy bandwidth baseline.
//
// Method: Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com English
// summary), [PD §2]: Wanda ranks a weight by its magnitude times the size of
// the activation on its input channel; here that size is the L2 norm of the
// channel over all tokens.
#include <atomic>

#include "dispatch.hpp"

namespace sparq24 {

constexpr int kColStrips = 128;

// Compute units of the current device, cached per device id (relaxed atomics:
// host threads that race on the first query store the same value).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int col_strips(const RowDesc& d) {
  const int64_t rows = d.B * d.R;
  return (int)(rows < kColStrips ? (rows > 0 ? rows : 1) : kColStrips);
}

// Stage 1: partial[strip][k] = sum over the strip's rows of x[row][k]^2 (fp64).
// A thread owns one 8-column unit and walks the rows of its strip in order.
template <class DT>
__global__ __launch_bounds__(kBlock) void k_col_sumsq(const char* __restrict__ x, int64_t R,
                                                      int64_t nunits, int64_t bs, int64_t rs,
                                                      int64_t rows_total, int nstrips,
                                                      double* __restrict__ partial) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int strip = blockIdx.y;
  if (i >= nunits) return;
  const int64_t per = (rows_total + nstrips - 1) / nstrips;
  const int64_t r0 = (int64_t)strip * per;
  const int64_t r1 = (r0 + per) < rows_total ? (r0 + per) : rows_total;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t row = r0; row < r1; ++row) {
    const int64_t b = row / R, r = row % R;
    Unit<DT> u;
    load_unit(u, x + b * bs + r * rs + i * (8 * DT::ESIZE));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double v = (double)u.f(e);
      acc[e] = __builtin_fma(v, v, acc[e]);
    }
  }
  double* o = partial + (int64_t)strip * nunits * 8 + i * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = acc[e];
}

// Stage 2: norms[k] = fp32(sqrt(sum over strips in order)).
__global__ __launch_bounds__(kBlock) void k_col_norm_final(const double* __restrict__ partial,
                                                           int64_t K, int nstrips,
                                                           float* __restrict__ norms) {
  const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (k >= K) return;
  double s = 0.0;
  for (int st = 0; st < nstrips; ++st) s += partial[(int64_t)st * K + k];
  norms[k] = (float)__builtin_sqrt(s);
}

hipError_t launch_col_l2norm(const RowDesc& d, double* partial, float* norms, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const int ns = col_strips(d);
  hipError_t e = with_dtype(d.dtype, [&]<class DT>() {
    hipLaunchKernelGGL((k_col_sumsq<DT>), dim3((unsigned)((nunits + kBlock - 1) / kBlock), ns),
                       dim3(kBlock), 0, s, d.x, d.R, nunits, d.bs, d.rs, d.B * d.R, ns, partial);
    return hipGetLastError();
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_col_norm_final, dim3((unsigned)((d.K + kBlock - 1) / kBlock)), dim3(kBlock),
                     0, s, partial, d.K, ns, norms);
  return hipGetLastError();
}

// Transposed operand (row_stride == 1, reduction axis strided) -> dense
// K-contiguous rows [B][R][K] through a 64x64 LDS tile, so both the reads
// (along R) and the writes (along K) are contiguous.
template <class E>
__global__ __launch_bounds__(kBlock) void k_transpose_rows(const char* __restrict__ x, int64_t R,
                                                           int64_t K, int64_t bs, int64_t ks,
                                                           E* __restrict__ out) {
  // 64 positions x 64 rows per tile.  In: 16-byte chunks along the rows of
  // one position; out: 16-byte chunks along K of one row, each gathered from
  // the tile two rows at a time.
  constexpr int ES = sizeof(E), CE = 16 / ES, LINE = 64 * ES, LCH = LINE / 16;
  __shared__ __align__(16) char tile[64 * LINE];  // [k][r]
  const int64_t k0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64, b = blockIdx.z;
  const int rcount = (int)((R - r0) < 64 ? (R - r0) : 64);
  const int kcount = (int)((K - k0) < 64 ? (K - k0) : 64);  // multiple of 8
  const char* xb = x + b * bs;
  for (int c = threadIdx.x; c < 64 * LCH; c += kBlock) {
    const int kk = c / LCH, r = (c % LCH) * CE;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kk < kcount && r < rcount) {
      const char* p = xb + (k0 + kk) * ks + (r0 + r) * ES;
      if (r + CE <= rcount) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        v = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        E w[CE];
        for (int i = 0; i < CE; ++i) w[i] = i < rcount - r ? reinterpret_cast<const E*>(p)[i] : E(0);
        __builtin_memcpy(&v, w, 16);
      }
    }
    *reinterpret_cast<uint4*>(tile + kk * LINE + r * ES) = v;
  }
  __syncthreads();
  constexpr int OCH = 64 / CE;  // output chunks per row per tile
  for (int item = threadIdx.x; item < 32 * OCH; item += kBlock) {
    const int rp = item % 32, c = item / 32;  // row pair, output chunk
    const int rr = 2 * rp;
    if (rr >= rcount || c * CE >= kcount) continue;
    E a[CE], bb[CE];
#pragma unroll
    for (int i = 0; i < CE; ++i) {
      const E* q = reinterpret_cast<const E*>(tile + (c * CE + i) * LINE + rr * ES);
      a[i] = q[0];
      bb[i] = q[1];
    }
    uint4 va, vb;
    __builtin_memcpy(&va, a, 16);
    __builtin_memcpy(&vb, bb, 16);
    char* o = reinterpret_cast<char*>(out + (b * R + r0 + rr) * K + k0 + c * CE);
    st4(o, va.x, va.y, va.z, va.w);
    if (rr + 1 < rcount) st4(o + K * ES, vb.x, vb.y, vb.z, vb.w);
  }
}

hipError_t launch_transpose_rows(const RowDesc& d, void* out, hipStream_t s) {
  const dim3 grid((unsigned)((d.K + 63) / 64), (unsigned)((d.R + 63) / 64), (unsigned)d.B);
  if (d.dtype == 0)
    hipLaunchKernelGGL((k_transpose_rows<uint32_t>), grid, dim3(kBlock), 0, s, d.x, d.R, d.K, d.bs,
                       d.ks, (uint32_t*)out);
  else
    hipLaunchKernelGGL((k_transpose_rows<uint16_t>), grid, dim3(kBlock), 0, s, d.x, d.R, d.K, d.bs,
                       d.ks, (uint16_t*)out);
  return hipGetLastError();
}

// Read-once / write-once copy of 16-byte vectors (grid-stride), with the same
// nontemporal hints as the prune/quantize kernels, so it is the streaming
// baseline they are compared with.
__global__ __launch_bounds__(kBlock) void k_copy(const uint4* __restrict__ src,
                                                 uint4* __restrict__ dst, int64_t n) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kBlock)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s4 + i), d4 + i);
}

// One 16-byte chunk per thread (the grid covers the buffer; the loop only
// runs again past 2^31 - 1 workgroups).  Over 1 GiB on MI355X this form
// measured 6.59 TB/s (read + write), against 5.1-5.8 TB/s for grids of 2 to
// 16 workgroups per CU and 5.9-6.2 TB/s with 2 to 8 chunks per thread.
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + kBlock - 1) / kBlock;
  if (blocks > 0x7FFFFFFF) blocks = 0x7FFFFFFF;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(kBlock), 0, s, (const uint4*)src,
                     (uint4*)dst, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block Hadamard rotation of a K-contiguous operand into a dense copy
// [PD §4]: load, rotate in registers (hadamard_units), store.
// ---------------------------------------------------------------------------
template <class DT, int TEAM, int UPL, int ROT>
__global__ __launch_bounds__(kBlock) void k_hadamard(const char* __restrict__ x, int64_t R,
                                                     int64_t nunits, int64_t bs, int64_t rs,
                                                     Rot rot, char* __restrict__ out) {
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  const bool active = r < R;
  const char* xr = x + b * bs + (active ? r : 0) * rs;
  char* orow = out + (b * R + r) * nunits * (8 * DT::ESIZE);
  for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
    Unit<DT> u[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (active && i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
      else zero_unit(u[j]);
    }
    hadamard_units<DT, TEAM, UPL, ROT>(u, rot, t);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (active && i < nunits) {
        char* dst = orow + i * (8 * DT::ESIZE);
        st4(dst, u[j].w[0], u[j].w[1], u[j].w[2], u[j].w[3]);
        if constexpr (DT::W == 8) st4(dst + 16, u[j].w[4], u[j].w[5], u[j].w[6], u[j].w[7]);
      }
    }
  }
}

hipError_t launch_hadamard(const RowDesc& d, void* out, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  return with_dtype(d.dtype, [&]<class DT>() {
    auto go = [&]<int TEAM, int UPL, int R>() {
      hipLaunchKernelGGL((k_hadamard<DT, TEAM, UPL, R>), row_grid(d, TEAM), dim3(kBlock), 0, s, d.x,
                         d.R, nunits, d.bs, d.rs, d.rot, (char*)out);
      return hipGetLastError();
    };
    if (d.rot.n > 512)  // blocks over 512 elements, on whole-workgroup teams
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return go.template operator()<TEAM, UPL, 3>();
      });
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      return with_rot<TEAM>(d.rot, [&]<int R>() {
        if constexpr (R == 1) return go.template operator()<TEAM, UPL, 1>();
        else return hipErrorInvalidValue;  // a rotation always has a block; long ones go above
      });
    });
  });
}

}  // namespace sparq24
