// Dense online quantizers, the rivals of 2:4 at equal bits or equal tier.
//
// Method: Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com English
// summary).  [PD §2]: the quantized side pays for online quantization of
// operands produced on the fly.  [PD §3]: INT8 with one scale per row, FP8,
// MXFP4 (one power-of-two scale per 32 elements) and NVFP4 (an FP8 scale per
// 16 elements plus one per tensor).
#include "dispatch.hpp"

namespace sparq24 {

// ---------------------------------------------------------------------------
// Per-row INT-b / FP8: the team holds its row, reduces |x|max, encodes.
// The grid covers every row (one row per team).
// ---------------------------------------------------------------------------
template <class DT>
__device__ inline uint32_t unit_absmax(const Unit<DT>& u) {
  if constexpr (DT::ESIZE == 2) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = u.w[i] & 0x7FFF7FFFu;
      const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
      const uint32_t h = lo > hi ? lo : hi;
      m = m > h ? m : h;
    }
    return m;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = u.w[i] & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
    return m;
  }
}

template <class DT, int TEAM, int UPL, int ROT>
SPARQ24_ROW_KERNEL void k_quant_rows(RowGeom g, int cfmt, float qmax,
                                                       char* __restrict__ codes,
                                                       float* __restrict__ scales) {
  __shared__ uint32_t red[kBlock / 64];
  for_each_row<DT, TEAM, UPL, ROT>(g, [&](Unit<DT>(&u)[UPL], int64_t row, int t) {
    uint32_t am = 0;
    if constexpr (DT::ESIZE == 2) {  // packed 16-bit maxima of |x|, unpacked once
#pragma unroll
      for (int j = 0; j < UPL; ++j) am = unit_absmax16_packed(u[j].w, am);
      am = unpack_max16(am);
    } else {
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const uint32_t a = unit_absmax(u[j]);
        am = am > a ? am : a;
      }
    }
    am = team_max_u32<TEAM>(am, red);
    if (row >= g.nrows) return;
    float s, inv;
    row_scale(DT::to_f32(am), qmax, s, inv);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = (int64_t)j * TEAM + t;
      if (i < g.nunits) {
        const int64_t o = row * g.nunits + i;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = u[j].f(e) * inv;
        if (cfmt == CF_FP8) {
          st2(codes + o * 8, enc_e4m3_x4(y[0], y[1], y[2], y[3]), enc_e4m3_x4(y[4], y[5], y[6], y[7]));
        } else {
          uint32_t r[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = __float_as_uint(int_round_magic(y[e], qmax));
          if (cfmt == CF_INT8) {
            const uint32_t a = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
            const uint32_t b = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
            const uint32_t c = __builtin_amdgcn_perm(r[5], r[4], 0x0c0c0400u);
            const uint32_t d = __builtin_amdgcn_perm(r[7], r[6], 0x0c0c0400u);
            st2(codes + o * 8, __builtin_amdgcn_perm(b, a, 0x05040100u), __builtin_amdgcn_perm(d, c, 0x05040100u));
          } else {  // CF_INT16
            st4(codes + o * 16, __builtin_amdgcn_perm(r[1], r[0], 0x05040100u), __builtin_amdgcn_perm(r[3], r[2], 0x05040100u),
                __builtin_amdgcn_perm(r[5], r[4], 0x05040100u), __builtin_amdgcn_perm(r[7], r[6], 0x05040100u));
          }
        }
      }
    }
    if (t == 0) scales[row] = s;
  });
}

// ---------------------------------------------------------------------------
// Tensor absolute maximum, first stage: one fp32 bit pattern per workgroup
// (a grid-stride walk over rows; max is order-free so the result is exact).
// ---------------------------------------------------------------------------
constexpr int kAbsmaxBlocks = 512;

template <class DT, int TEAM, int UPL, int ROT>
__global__ __launch_bounds__(kBlock) void k_absmax_partial(
    const char* __restrict__ x, int64_t B, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    uint32_t* __restrict__ partials, Rot rot) {
  __shared__ uint32_t red[kBlock / 64];
  const int t = threadIdx.x % TEAM;
  constexpr int RPB = kBlock / TEAM;
  uint32_t am = 0;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TEAM; row < B * R;
       row += (int64_t)gridDim.x * RPB) {
    const int64_t b = row / R, r = row % R;
    const char* xr = x + b * bs + r * rs;
    for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
      Unit<DT> u[UPL];
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const int64_t i = c0 + j * TEAM + t;
        if (i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
        else zero_unit(u[j]);
      }
      if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(u, rot, t);
#pragma unroll
      for (int j = 0; j < UPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = u[j].absbits(e);
          am = am > a ? am : a;
        }
    }
  }
  // to fp32 bits so partials of any storage type compare as fp32
  am = __float_as_uint(DT::to_f32(am));
  am = team_max_u32<64>(am, red);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int i = 1; i < kBlock / 64; ++i) m = m > red[i] ? m : red[i];
    partials[blockIdx.x] = m;
  }
}

int absmax_partial_count(const RowDesc& d) {
  const int64_t rows = d.B * d.R;
  const int64_t want = (rows + 3) / 4;
  return (int)(want < kAbsmaxBlocks ? (want > 0 ? want : 1) : kAbsmaxBlocks);
}

hipError_t launch_absmax_partials(const RowDesc& d, uint32_t* partials, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const int nb = absmax_partial_count(d);
  return with_dtype(d.dtype, [&]<class DT>() {
    auto go = [&]<int TEAM, int UPL, int R>() {
      hipLaunchKernelGGL((k_absmax_partial<DT, TEAM, UPL, R>), dim3(nb), dim3(kBlock), 0, s, d.x,
                         d.B, d.R, nunits, d.bs, d.rs, partials, d.rot);
      return hipGetLastError();
    };
    if (d.rot.n > 512)  // long rotation blocks: whole-workgroup teams
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return go.template operator()<TEAM, UPL, 3>();
      });
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<TEAM, UPL, R>(); });
    });
  });
}

// ---------------------------------------------------------------------------
// MXFP4 / NVFP4.  Lane t owns units t, t+TEAM, ...; an MX block (32
// elements) is 4 adjacent lanes, an NV block (16 elements) 2 adjacent lanes,
// combined with cross-lane xor shuffles.
// ---------------------------------------------------------------------------
template <class DT, int TEAM, int UPL, bool NV, int ROT>
__global__ __launch_bounds__(kBlock) void k_quant_block(
    const char* __restrict__ x, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    const float* __restrict__ tamax_in, const uint32_t* __restrict__ partials, int nparts,
    uint32_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ ts_out,
    Rot rot) {
  __shared__ uint32_t red[kBlock / 64];
  __shared__ float nvinv[NV ? kNvInvEntries : 1];
  float s_t = 0.f, g = 0.f;
  if constexpr (NV) {
    const float T = block_tensor_amax(tamax_in, partials, nparts, red);
    nv_tensor_scales(T, s_t, g);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *ts_out = s_t;
    nv_inv_fill(nvinv, s_t);
    __syncthreads();
  }
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  const bool active = r < R;
  const char* xr = x + b * bs + r * rs;
  const int64_t orow = b * R + r;
  // shuffles below need every lane of the wave, so masked lanes run along
  for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
    Unit<DT> u[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (active && i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
      else zero_unit(u[j]);
    }
    if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(u, rot, t);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      uint32_t am = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = u[j].absbits(e);
        am = am > a ? am : a;
      }
      am = __float_as_uint(DT::to_f32(am));
      uint32_t w = (uint32_t)__shfl_xor((int)am, 1, 64);
      am = am > w ? am : w;
      if constexpr (!NV) {
        w = (uint32_t)__shfl_xor((int)am, 2, 64);
        am = am > w ? am : w;
        const int e = mx_exponent(am);
        float y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = __builtin_ldexpf(u[j].f(q), -e);
        const uint32_t pk = enc_e2m1_x8(y);
        if (active && i < nunits) {
          st(codes + orow * nunits + i, pk);
          if ((i & 3) == 0) st(scales + orow * (nunits / 4) + (i >> 2), (uint8_t)(e + 127));
        }
      } else {
        const uint32_t bc = nv_block_code(__uint_as_float(am), g);
        const float inv = nvinv[bc];
        float y[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) y[q] = u[j].f(q) * inv;
        const uint32_t pk = enc_e2m1_x8(y);
        if (active && i < nunits) {
          st(codes + orow * nunits + i, pk);
          if ((i & 1) == 0) st(scales + orow * (nunits / 2) + (i >> 1), (uint8_t)bc);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prune (2:4 or pairwise 4:8 [PD §6]) and quantize the kept values to MXFP4 /
// NVFP4.  A unit (8 inputs) yields 4 kept values = 4 E2M1 codes (16 bits);
// the compressed row is blocked like a dense one, so an NV block (16 kept)
// is 4 adjacent lanes and an MX block (32 kept) 8.  With NVFP4 the sparse
// operand is Blackwell's sparse FP4 layout of [PD §6].
// ---------------------------------------------------------------------------
template <class DT, int PAT, bool WANDA>
__device__ inline uint32_t select_any(const Unit<DT>& u, const float* norm, int64_t i,
                                      int64_t nunits, Kept<DT>& kp) {
  uint32_t m;
  if constexpr (PAT == PAT_48) {
    m = select_pairs48(u);
    kp = gather_pairs48(u, m);
  } else {
    m = 0;
    if (!WANDA || i < nunits) m = select_unit<DT, WANDA>(u, norm, i * 8);
    kp = gather_kept(u, m);
  }
  return m;
}

template <class DT, int TEAM, int UPL, int PAT, bool WANDA, bool NV, int ROT>
__global__ __launch_bounds__(kBlock) void k_prune_quant_fp4(
    const char* __restrict__ x, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    const float* __restrict__ norm, const float* __restrict__ tamax_in,
    const uint32_t* __restrict__ partials, int nparts, uint16_t* __restrict__ codes,
    uint8_t* __restrict__ meta, uint8_t* __restrict__ scales, float* __restrict__ ts_out,
    Rot rot) {
  __shared__ uint32_t red[kBlock / 64];
  __shared__ float nvinv[NV ? kNvInvEntries : 1];
  float s_t = 0.f, g = 0.f;
  if constexpr (NV) {
    const float T = block_tensor_amax(tamax_in, partials, nparts, red);
    nv_tensor_scales(T, s_t, g);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *ts_out = s_t;
    nv_inv_fill(nvinv, s_t);
    __syncthreads();
  }
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  const bool active = r < R;
  const char* xr = x + b * bs + (active ? r : 0) * rs;
  const int64_t orow = b * R + r;
  // shuffles below need every lane of the wave, so masked lanes run along
  for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
    Unit<DT> u[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (active && i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
      else zero_unit(u[j]);
    }
    if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(u, rot, t);
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      Kept<DT> kp;
      const uint32_t m = select_any<DT, PAT, WANDA>(u[j], norm, i, nunits, kp);
      float v[4];
      uint32_t am = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = kp.f(e);
        const uint32_t a = __float_as_uint(v[e]) & 0x7FFFFFFFu;
        am = am > a ? am : a;
      }
      uint32_t w = (uint32_t)__shfl_xor((int)am, 1, 64);
      am = am > w ? am : w;
      w = (uint32_t)__shfl_xor((int)am, 2, 64);
      am = am > w ? am : w;
      uint32_t sc, pk;
      if constexpr (NV) {
        sc = nv_block_code(__uint_as_float(am), g);
        const float inv = nvinv[sc];
        pk = enc_e2m1_x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
      } else {
        w = (uint32_t)__shfl_xor((int)am, 4, 64);
        am = am > w ? am : w;
        const int e = mx_exponent(am);
        sc = (uint32_t)(e + 127);
        pk = enc_e2m1_x4(__builtin_ldexpf(v[0], -e), __builtin_ldexpf(v[1], -e),
                         __builtin_ldexpf(v[2], -e), __builtin_ldexpf(v[3], -e));
      }
      const uint32_t mo = PAT == PAT_48 ? (uint32_t)__shfl_xor((int)m, 1, 64) : 0u;
      if (active && i < nunits) {
        st(codes + orow * nunits + i, (uint16_t)pk);
        if constexpr (NV) {
          if ((i & 3) == 0) st(scales + orow * (nunits / 4) + (i >> 2), (uint8_t)sc);
        } else {
          if ((i & 7) == 0) st(scales + orow * (nunits / 8) + (i >> 3), (uint8_t)sc);
        }
        if constexpr (PAT == PAT_48) {
          if ((i & 1) == 0) st(meta + orow * (nunits / 2) + (i >> 1), (uint8_t)(m | (mo << 4)));
        } else {
          st(meta + orow * nunits + i, (uint8_t)m);
        }
      }
    }
  }
}

// Partial maxima of the kept values' magnitudes (the NVFP4 tensor maximum of
// a sparse operand whose kept maximum can differ from its plain maximum).
template <class DT, int TEAM, int UPL, int PAT, bool WANDA, int ROT>
__global__ __launch_bounds__(kBlock) void k_kept_absmax_partial(
    const char* __restrict__ x, int64_t B, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    const float* __restrict__ norm, uint32_t* __restrict__ partials, Rot rot) {
  __shared__ uint32_t red[kBlock / 64];
  const int t = threadIdx.x % TEAM;
  constexpr int RPB = kBlock / TEAM;
  uint32_t am = 0;
  for (int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TEAM; row < B * R;
       row += (int64_t)gridDim.x * RPB) {
    const int64_t b = row / R, r = row % R;
    const char* xr = x + b * bs + r * rs;
    for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
      Unit<DT> u[UPL];  // all loads of the chunk in flight before any use
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const int64_t i = c0 + j * TEAM + t;
        if (i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
        else zero_unit(u[j]);
      }
      if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(u, rot, t);
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const int64_t i = c0 + j * TEAM + t;
        Kept<DT> kp;
        select_any<DT, PAT, WANDA>(u[j], norm, i, nunits, kp);  // zero units keep zeros
        const uint32_t a = __float_as_uint(DT::to_f32(kept_absmax(kp)));
        am = am > a ? am : a;
      }
    }
  }
  am = team_max_u32<64>(am, red);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = red[0];
    for (int i = 1; i < kBlock / 64; ++i) m = m > red[i] ? m : red[i];
    partials[blockIdx.x] = m;
  }
}

hipError_t launch_quant_rows(const RowDesc& d, int cfmt, float qmax, void* codes, float* scales,
                             hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const RowGeom g{d.x, d.R, d.B * d.R, nunits, d.bs, d.rs, d.rot};
  return with_dtype(d.dtype, [&]<class DT>() {
    auto go = [&]<int TEAM, int UPL, int R>() {
      hipLaunchKernelGGL((k_quant_rows<DT, TEAM, UPL, R>), stream_grid(g.nrows, TEAM), dim3(kBlock),
                         0, s, g, cfmt, qmax, (char*)codes, scales);
      return hipGetLastError();
    };
    if (d.rot.n > 512)  // rotation blocks over 512 elements, on whole-workgroup teams
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return go.template operator()<TEAM, UPL, 3>();
      });
    return with_row_variant<1>(nunits, [&]<int TEAM, int UPL>() {
      return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<TEAM, UPL, R>(); });
    });
  });
}

template <bool NV>
static hipError_t launch_quant_block(const RowDesc& d, const float* tamax_in,
                                     const uint32_t* partials, int nparts, void* codes,
                                     uint8_t* scales, float* ts_out, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  return with_dtype(d.dtype, [&]<class DT>() {
    auto go = [&]<int TEAM, int UPL, int R>() {
      hipLaunchKernelGGL((k_quant_block<DT, TEAM, UPL, NV, R>), row_grid(d, TEAM), dim3(kBlock), 0,
                         s, d.x, d.R, nunits, d.bs, d.rs, tamax_in, partials, nparts,
                         (uint32_t*)codes, scales, ts_out, d.rot);
      return hipGetLastError();
    };
    if (d.rot.n > 512)  // long rotation blocks: whole-workgroup teams
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return go.template operator()<TEAM, UPL, 3>();
      });
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<TEAM, UPL, R>(); });
    });
  });
}

hipError_t launch_quant_mx(const RowDesc& d, void* codes, uint8_t* scales, hipStream_t s) {
  return launch_quant_block<false>(d, nullptr, nullptr, 0, codes, scales, nullptr, s);
}

hipError_t launch_quant_nv(const RowDesc& d, const float* tamax_in, const uint32_t* partials,
                           int nparts, void* codes, uint8_t* scales, float* ts_out,
                           hipStream_t s) {
  return launch_quant_block<true>(d, tamax_in, partials, nparts, codes, scales, ts_out, s);
}

// Rotation variants exist for magnitude selection only (the rotated calls
// take no Wanda norms).
hipError_t launch_prune_quant_fp4(const RowDesc& d, int pat, bool wanda, const float* norm,
                                  int cfmt, const float* tamax_in, const uint32_t* partials,
                                  int nparts, void* codes, uint8_t* meta, uint8_t* scales,
                                  float* ts_out, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  if (wanda && d.rot.n) return hipErrorInvalidValue;
  const bool nv = cfmt == CF_NV;
  return with_dtype(d.dtype, [&]<class DT>() {
    // LONG: rotation blocks over 512 elements, on whole-workgroup teams
    auto body = [&]<int TEAM, int UPL, bool LONG>() -> hipError_t {
      auto go = [&]<int P, bool W, bool NV, int R>() {
        hipLaunchKernelGGL((k_prune_quant_fp4<DT, TEAM, UPL, P, W, NV, R>), row_grid(d, TEAM),
                           dim3(kBlock), 0, s, d.x, d.R, nunits, d.bs, d.rs, norm, tamax_in,
                           partials, nparts, (uint16_t*)codes, meta, scales, ts_out, d.rot);
        return hipGetLastError();
      };
      auto mag = [&]<int P, bool NV>() {
        if constexpr (LONG) return go.template operator()<P, false, NV, 3>();
        else return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<P, false, NV, R>(); });
      };
      if (pat == PAT_48)
        return nv ? mag.template operator()<PAT_48, true>() : mag.template operator()<PAT_48, false>();
      if constexpr (!LONG) {
        if (wanda)
          return nv ? go.template operator()<PAT_24, true, true, 0>()
                    : go.template operator()<PAT_24, true, false, 0>();
      }
      return nv ? mag.template operator()<PAT_24, true>() : mag.template operator()<PAT_24, false>();
    };
    if (d.rot.n > 512)
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return body.template operator()<TEAM, UPL, true>();
      });
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      return body.template operator()<TEAM, UPL, false>();
    });
  });
}

hipError_t launch_kept_absmax_partials(const RowDesc& d, int pat, bool wanda, const float* norm,
                                       uint32_t* partials, hipStream_t s) {
  if (pat == PAT_24 && !wanda) return launch_absmax_partials(d, partials, s);  // kept max == max
  if (wanda && d.rot.n) return hipErrorInvalidValue;
  const int64_t nunits = d.K / 8;
  const int nb = absmax_partial_count(d);
  return with_dtype(d.dtype, [&]<class DT>() {
    // LONG: rotation blocks over 512 elements, on whole-workgroup teams
    auto body = [&]<int TEAM, int UPL, bool LONG>() -> hipError_t {
      auto go = [&]<int P, bool W, int R>() {
        hipLaunchKernelGGL((k_kept_absmax_partial<DT, TEAM, UPL, P, W, R>), dim3(nb),
                           dim3(kBlock), 0, s, d.x, d.B, d.R, nunits, d.bs, d.rs, norm, partials,
                           d.rot);
        return hipGetLastError();
      };
      if constexpr (LONG) {
        return go.template operator()<PAT_48, false, 3>();  // only pairwise 4:8 gets here rotated
      } else {
        if (pat == PAT_48)
          return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<PAT_48, false, R>(); });
        return go.template operator()<PAT_24, true, 0>();
      }
    };
    if (d.rot.n > 512)
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return body.template operator()<TEAM, UPL, true>();
      });
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      return body.template operator()<TEAM, UPL, false>();
    });
  });
}

}  // namespace sparq24
