// Device building blocks shared by the sparq24 kernels (gfx950, wave64).
//
// Method: Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com English
// summary, cited as [PD §n]).  A "unit" is 8 consecutive elements along the
// reduction axis = two groups of four = one metadata byte.  A "team" is a run
// of TEAM lanes (16..256) that owns one row (one K-vector); lane t of a team
// owns units t, t + TEAM, t + 2*TEAM, ... so that every vector memory
// instruction of a team touches one contiguous span.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparq24 {

constexpr int kBlock = 256;  // threads per workgroup for every row kernel

// ---------------------------------------------------------------------------
// Storage types.  W = dwords per 8-element unit.
// ---------------------------------------------------------------------------
struct BF16T {
  static constexpr int W = 4;
  static constexpr int ESIZE = 2;
  static constexpr uint32_t ABS = 0x7FFFu;
  __device__ static inline float to_f32(uint32_t h) { return __uint_as_float(h << 16); }
};
struct F16T {
  static constexpr int W = 4;
  static constexpr int ESIZE = 2;
  static constexpr uint32_t ABS = 0x7FFFu;
  __device__ static inline float to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
};
struct F32T {
  static constexpr int W = 8;
  static constexpr int ESIZE = 4;
  static constexpr uint32_t ABS = 0x7FFFFFFFu;
  __device__ static inline float to_f32(uint32_t u) { return __uint_as_float(u); }
};

template <class DT>
struct Unit {
  uint32_t w[DT::W];
  // raw storage bits of element i (0..7)
  __device__ inline uint32_t raw(int i) const {
    if constexpr (DT::ESIZE == 2) return (w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
    else return w[i];
  }
  __device__ inline float f(int i) const { return DT::to_f32(raw(i)); }
  __device__ inline uint32_t absbits(int i) const { return raw(i) & DT::ABS; }
};

template <class DT>
__device__ inline void load_unit(Unit<DT>& u, const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < DT::W / 4; ++i) {
    uint4 v = q[i];
    u.w[4 * i + 0] = v.x; u.w[4 * i + 1] = v.y; u.w[4 * i + 2] = v.z; u.w[4 * i + 3] = v.w;
  }
}

template <class DT>
__device__ inline void zero_unit(Unit<DT>& u) {
#pragma unroll
  for (int i = 0; i < DT::W; ++i) u.w[i] = 0;
}

// ---------------------------------------------------------------------------
// Top-2 of 4 with ties to the lower position [PD intro; PD §3].
// Each element gets an integer key whose order is (score, -position): the
// score's bit pattern (non-negative floats order like unsigned integers)
// with (3 - position) in the low bits.  A 7-op max/min network finds the two
// largest keys; their low bits give the positions.
// ---------------------------------------------------------------------------
template <class K>
__device__ inline void top2(K a, K b, K c, K d, K& t1, K& t2) {
  K m1 = a > b ? a : b, n1 = a > b ? b : a;
  K m2 = c > d ? c : d, n2 = c > d ? d : c;
  t1 = m1 > m2 ? m1 : m2;
  K lo = m1 > m2 ? m2 : m1;
  K nn = n1 > n2 ? n1 : n2;
  t2 = lo > nn ? lo : nn;
}

// nibble = i0 | i1 << 2 with i0 < i1, from the low 2 bits (3 - position) of
// the two winning keys: i0 = 3 - max(j), i1 = 3 - min(j).
__device__ inline uint32_t nibble_from_j(uint32_t j1, uint32_t j2) {
  uint32_t jmax = j1 > j2 ? j1 : j2, jmin = j1 > j2 ? j2 : j1;
  return 15u - jmax - 4u * jmin;
}

// Selection for group g (0 or 1) of a unit.
template <class DT, bool WANDA>
__device__ inline uint32_t select_group(const Unit<DT>& u, int g, const float* n4) {
  if constexpr (!WANDA && DT::ESIZE == 2) {
    uint32_t k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = (u.absbits(4 * g + i) << 2) | (3u - i);
    uint32_t t1, t2;
    top2(k[0], k[1], k[2], k[3], t1, t2);
    return nibble_from_j(t1 & 3u, t2 & 3u);
  } else {
    uint64_t k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (WANDA) {
        // exact: <= 24-bit x 24-bit significands fit in fp64's 53, so the low
        // mantissa bits of the product are zero and can carry the position
        double p = (double)__uint_as_float(__float_as_uint(u.f(4 * g + i)) & 0x7FFFFFFFu) *
                   (double)n4[i];
        k[i] = (uint64_t)__double_as_longlong(p) | (uint64_t)(3u - i);
      } else {
        k[i] = ((uint64_t)u.absbits(4 * g + i) << 2) | (uint64_t)(3u - i);
      }
    }
    uint64_t t1, t2;
    top2(k[0], k[1], k[2], k[3], t1, t2);
    return nibble_from_j((uint32_t)t1 & 3u, (uint32_t)t2 & 3u);
  }
}

// Kept raw values of a 16-bit unit given the two nibbles: two dwords, each
// the (i0, i1) pair of one group, gathered with a byte permute.
__device__ inline uint32_t perm_sel(uint32_t nib) {
  uint32_t i0 = nib & 3u, i1 = nib >> 2;
  return 0x01000100u + i0 * 0x0202u + i1 * 0x02020000u;
}

template <class DT>
__device__ inline uint32_t kept_raw(const Unit<DT>& u, int g, uint32_t nib, int which) {
  uint32_t i = which ? (nib >> 2) : (nib & 3u);
  return u.raw(4 * g + (int)i);
}

// ---------------------------------------------------------------------------
// Encoders: exact integer implementations of round-to-nearest-even with
// saturation, sign copied from the input (so -0 keeps its sign bit).
// ---------------------------------------------------------------------------

// OCP e4m3 (bias 7, max 448, subnormal step 2^-9).
__device__ inline uint32_t enc_e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {            // |y| >= 448: saturate
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {      // |y| < 2^-6: multiples of 2^-9 (code 8 = 2^-6)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {                           // keep 3 mantissa bits, RNE on the 20 dropped ones
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);  // rebias 127 -> 7
  }
  return code | sign;
}

__device__ inline float dec_e4m3(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// E2M1 (values 0, .5, 1, 1.5, 2, 3, 4, 6), 4-bit code with sign in bit 3.
__device__ inline uint32_t enc_e2m1(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 28) & 0x8u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x40C00000u) {            // |y| >= 6
    code = 7u;
  } else if (a < 0x3F800000u) {      // |y| < 1: steps of 0.5 (code 2 = 1.0)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
  } else {                           // keep 1 mantissa bit, RNE on 22 dropped bits
    uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
    code = (r >> 22) - (126u << 1);  // rebias 127 -> 1
  }
  return code | sign;
}

__device__ inline float dec_e2m1(uint32_t c) {
  // magnitudes of codes 0..7 in half-units (0,1,2,3,4,6,8,12) as packed nibbles
  float v = (float)((0xC8643210u >> ((c & 7u) * 4u)) & 0xFu) * 0.5f;
  return (c & 8u) ? -v : v;
}

// Symmetric INT code as float (exact integer value), clamp to [-qmax, qmax].
__device__ inline float enc_int(float y, float qmax) {
  float q = __builtin_rintf(y);
  return __builtin_fminf(__builtin_fmaxf(q, -qmax), qmax);
}

// ---------------------------------------------------------------------------
// Team reductions (fixed order -> deterministic).  TEAM <= 64 stays inside a
// wave; larger teams combine their waves through LDS (all threads of the
// block must call these together).
// ---------------------------------------------------------------------------
template <int TEAM>
__device__ inline uint32_t team_max_u32(uint32_t v, uint32_t* lds) {
  if constexpr (TEAM <= 64) {
#pragma unroll
    for (int o = TEAM / 2; o > 0; o >>= 1) {
      uint32_t w = (uint32_t)__shfl_xor((int)v, o, TEAM);
      v = v > w ? v : w;
    }
    return v;
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
      v = v > w ? v : w;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    const int first = (threadIdx.x / TEAM) * (TEAM / 64);
    uint32_t r = lds[first];
#pragma unroll
    for (int i = 1; i < TEAM / 64; ++i) r = r > lds[first + i] ? r : lds[first + i];
    return r;
  }
}

template <int TEAM>
__device__ inline double team_sum_f64(double v, double* lds) {
  if constexpr (TEAM <= 64) {
#pragma unroll
    for (int o = TEAM / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, TEAM);
    return v;
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    const int first = (threadIdx.x / TEAM) * (TEAM / 64);
    double r = lds[first];
#pragma unroll
    for (int i = 1; i < TEAM / 64; ++i) r += lds[first + i];
    return r;
  }
}

// Per-row symmetric scale: s = fp32(amax / qmax), inv = fp32(qmax / amax);
// rows with amax < 2^-64 get s = inv = 0.
__device__ inline void row_scale(float amax, float qmax, float& s, float& inv) {
  if (amax >= 0x1p-64f) {
    s = amax / qmax;
    inv = qmax / amax;
  } else {
    s = 0.0f;
    inv = 0.0f;
  }
}

}  // namespace sparq24
