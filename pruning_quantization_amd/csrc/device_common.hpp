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

#include "launch.hpp"

namespace sparq24 {

constexpr int kBlock = 256;  // threads per workgroup for every row kernel

#define SPARQ24_ROW_KERNEL __global__ __launch_bounds__(kBlock)

// ---------------------------------------------------------------------------
// Storage types.  W = dwords per 8-element unit.
// ---------------------------------------------------------------------------
struct BF16T {
  static constexpr bool IS_BF16 = true;
  static constexpr int W = 4;
  static constexpr int ESIZE = 2;
  static constexpr uint32_t ABS = 0x7FFFu;
  __device__ static inline float to_f32(uint32_t h) { return __uint_as_float(h << 16); }
};
struct F16T {
  static constexpr bool IS_BF16 = false;
  static constexpr int W = 4;
  static constexpr int ESIZE = 2;
  static constexpr uint32_t ABS = 0x7FFFu;
  __device__ static inline float to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
};
struct F32T {
  static constexpr bool IS_BF16 = false;
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

// Streaming hints: operands are read once and outputs written once, so loads
// and stores carry the nontemporal bit (measured 10-20% faster on MI355X).
template <class T>
__device__ inline void st(T* p, T v) {
  __builtin_nontemporal_store(v, p);
}
// 64/128-bit stores as vectors of 32-bit lanes (what the nontemporal builtin takes)
__device__ inline void st2(void* p, uint32_t a, uint32_t b) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v = {a, b};
  st(reinterpret_cast<u32x2*>(p), v);
}
__device__ inline void st4(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v = {a, b, c, d};
  st(reinterpret_cast<u32x4*>(p), v);
}

template <class DT>
__device__ inline void load_unit(Unit<DT>& u, const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < DT::W / 4; ++i) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q) + i);
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
// with (3 - position) in the low bits.  The two largest keys (4 instructions
// for 32-bit keys, a max/min network for 64-bit ones) give the positions in
// their low bits.
// ---------------------------------------------------------------------------
template <class K>
__device__ inline void top2(K a, K b, K c, K d, K& t1, K& t2) {
  if constexpr (sizeof(K) == 4) {
    // M = max(a, b, c), m = median(a, b, c); then t1 = max(M, d) and the
    // second largest of the four is median(m, M, d) (m <= M): 4 instructions
    // (v_max3, v_med3, v_max, v_med3)
    K M, m;
    asm("v_max3_u32 %0, %1, %2, %3" : "=v"(M) : "v"(a), "v"(b), "v"(c));
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(m) : "v"(a), "v"(b), "v"(c));
    t1 = M > d ? M : d;
    asm("v_med3_u32 %0, %1, %2, %3" : "=v"(t2) : "v"(m), "v"(M), "v"(d));
  } else {
    K m1 = a > b ? a : b, n1 = a > b ? b : a;
    K m2 = c > d ? c : d, n2 = c > d ? d : c;
    t1 = m1 > m2 ? m1 : m2;
    K lo = m1 > m2 ? m2 : m1;
    K nn = n1 > n2 ? n1 : n2;
    t2 = lo > nn ? lo : nn;
  }
}

// nibble = i0 | i1 << 2 with i0 < i1, from the low 2 bits (3 - position) of
// the two winning keys: i0 = 3 - max(j), i1 = 3 - min(j).
__device__ inline uint32_t nibble_from_j(uint32_t j1, uint32_t j2) {
  uint32_t jmax = j1 > j2 ? j1 : j2, jmin = j1 > j2 ? j2 : j1;
  return 15u - jmax - 4u * jmin;
}

// fp64 maximum / minimum of finite operands: one instruction each, without
// the quieting of signalling NaNs that the IEEE maxNum / minNum lowering
// adds for operands it cannot prove canonical (keys built with bit
// operations), which no finite value needs.
__device__ inline double max_f64_finite(double a, double b) {
  double r;
  asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline double min_f64_finite(double a, double b) {
  double r;
  asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Selection for group g (0 or 1) of a unit.
template <class DT, bool WANDA>
__device__ inline uint32_t select_group(const Unit<DT>& u, int g, const float* n4) {
  if constexpr (!WANDA && DT::ESIZE == 2) {
    // keys = |x| in bits 16..30, (3 - position) in bits 0..1
    const uint32_t a = u.w[2 * g] & 0x7FFF7FFFu, b = u.w[2 * g + 1] & 0x7FFF7FFFu;
    const uint32_t k0 = (a << 16) | 3u, k1 = (a & 0xFFFF0000u) | 2u;
    const uint32_t k2 = (b << 16) | 1u, k3 = b & 0xFFFF0000u;
    uint32_t t1, t2;
    top2(k0, k1, k2, k3, t1, t2);
    return nibble_from_j(t1 & 3u, t2 & 3u);
  } else if constexpr (WANDA) {
    // exact: <= 24-bit x 24-bit significands fit in fp64's 53, so the low
    // mantissa bits of the product are zero and can carry the position.
    // Non-negative finite doubles (fp64 subnormals are kept) order like their
    // bit patterns, so the fp64 max / min (one instruction each) rank the
    // keys exactly.
    double k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double p = (double)__uint_as_float(__float_as_uint(u.f(4 * g + i)) & 0x7FFFFFFFu) *
                       (double)n4[i];
      k[i] = __longlong_as_double(__double_as_longlong(p) | (long long)(3u - i));
    }
    const double m1 = max_f64_finite(k[0], k[1]), n1 = min_f64_finite(k[0], k[1]);
    const double m2 = max_f64_finite(k[2], k[3]), n2 = min_f64_finite(k[2], k[3]);
    const double t1 = max_f64_finite(m1, m2);
    const double t2 = max_f64_finite(min_f64_finite(m1, m2), max_f64_finite(n1, n2));
    return nibble_from_j((uint32_t)__double_as_longlong(t1) & 3u,
                         (uint32_t)__double_as_longlong(t2) & 3u);
  } else {
    uint64_t k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = ((uint64_t)u.absbits(4 * g + i) << 2) | (uint64_t)(3u - i);
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

// ---------------------------------------------------------------------------
// Packed unsigned 16-bit max of two dwords (v_pk_max_u16).
typedef unsigned short sparq24_u16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(sparq24_u16x2, a),
                                                                __builtin_bit_cast(sparq24_u16x2, b)));
}

// Largest |x| of a 16-bit unit as storage bits, via packed 16-bit max.
__device__ inline uint32_t unit_absmax16_packed(const uint32_t* w, uint32_t acc2) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc2 = pk_max_u16(acc2, w[i] & 0x7FFF7FFFu);
  return acc2;
}
__device__ inline uint32_t unpack_max16(uint32_t acc2) {
  const uint32_t lo = acc2 & 0xFFFFu, hi = acc2 >> 16;
  return lo > hi ? lo : hi;
}

// Magnitude selection for a 16-bit unit, everything in 32-bit lanes:
//  keys  = |x| in bits 16..30, (3 - position) in bits 0..1 (from the pair of
//          elements in one dword: 3 ops per pair);
//  top2  = v_max3 / v_med3 of three keys, then a max and a median with the
//          fourth (4 instructions);
//  i0/i1 = 3 - max(j), 3 - min(j) with j the winners' low bits;
//  kept  = byte permute with selector bytes (2*i0, 2*i0+1, 2*i1, 2*i1+1),
//          i.e. 0x07060706 - (jmax | jmin << 16) * 0x0202;
//  amax  = the top key of each group (its high half is the group's |max|,
//          which magnitude pruning always keeps).
struct Sel16 {
  uint32_t mb;      // metadata byte
  uint32_t k0, k1;  // kept pairs of group 0 and 1 (position order)
  uint32_t topkey;  // max of the two groups' top keys
};

__device__ inline void sel16_group(uint32_t w0, uint32_t w1, uint32_t& nib, uint32_t& kept,
                                   uint32_t& top) {
  const uint32_t a = w0 & 0x7FFF7FFFu, b = w1 & 0x7FFF7FFFu;
  const uint32_t k0 = (a << 16) | 3u, k1 = (a & 0xFFFF0000u) | 2u;
  const uint32_t k2 = (b << 16) | 1u, k3 = b & 0xFFFF0000u;
  uint32_t t1, t2;
  top2(k0, k1, k2, k3, t1, t2);
  const uint32_t j1 = t1 & 3u, j2 = t2 & 3u;
  const uint32_t jmax = j1 > j2 ? j1 : j2, jmin = j1 > j2 ? j2 : j1;
  nib = 15u - jmax - 4u * jmin;
  const uint32_t sel = 0x07060706u - __umul24(jmax | (jmin << 16), 0x0202u);
  kept = __builtin_amdgcn_perm(w1, w0, sel);
  top = t1;
}

__device__ inline Sel16 select16(const uint32_t* w) {
  Sel16 r;
  uint32_t n0, n1, t0, t1;
  sel16_group(w[0], w[1], n0, r.k0, t0);
  sel16_group(w[2], w[3], n1, r.k1, t1);
  r.mb = n0 | (n1 << 4);
  r.topkey = t0 > t1 ? t0 : t1;
  return r;
}

// Selection of a 16-bit unit through a table in LDS.  The keys carry
// 8 * (3 - position) in their low byte, so one byte permute placing the low
// bytes of the two winning keys side by side gives 8 * j1 + 2048 * j2, the
// LDS byte offset of the table entry for that pair of positions.  The entry
// holds the byte-permute selector that gathers the kept pair in position
// order and the group's metadata nibble in both halves of a byte, so the
// unit's metadata byte is one bit-field insert of its two groups' entries.
struct SelLut {
  uint32_t sel, nib;
};
constexpr int kSelLutEntries = 3 + 256 * 3 + 1;

// Every thread of the workgroup calls this; the table is ready after the
// next workgroup barrier.
__device__ inline void sel_lut_fill(SelLut* lut) {
  if (threadIdx.x < 16) {
    const uint32_t j1 = threadIdx.x & 3u, j2 = threadIdx.x >> 2;  // j1 == j2 never occurs
    const uint32_t jmax = j1 > j2 ? j1 : j2, jmin = j1 > j2 ? j2 : j1;
    const uint32_t i0 = 3u - jmax, i1 = 3u - jmin, nib = i0 | (i1 << 2);
    lut[j1 + 256u * j2] = SelLut{0x01000100u + i0 * 0x0202u + i1 * 0x02020000u, nib | (nib << 4)};
  }
}

__device__ inline void sel16_group_lut(uint32_t w0, uint32_t w1, const SelLut* lut, uint32_t& kept,
                                       uint32_t& nib, uint32_t& top) {
  const uint32_t a = w0 & 0x7FFF7FFFu, b = w1 & 0x7FFF7FFFu;
  const uint32_t k0 = (a << 16) | 24u, k1 = (a & 0xFFFF0000u) | 16u;
  const uint32_t k2 = (b << 16) | 8u, k3 = b & 0xFFFF0000u;
  uint32_t t1, t2;
  top2(k0, k1, k2, k3, t1, t2);
  const uint32_t off = __builtin_amdgcn_perm(t2, t1, 0x0c0c0400u);  // 8 * j1 + 2048 * j2
  const SelLut e = *reinterpret_cast<const SelLut*>(reinterpret_cast<const char*>(lut) + off);
  kept = __builtin_amdgcn_perm(w1, w0, e.sel);
  nib = e.nib;
  top = t1;
}

// Kept pairs, metadata byte and the larger top key (its high half is the
// unit's |max|) of a 16-bit unit.
__device__ inline Sel16 select16_lut(const uint32_t* w, const SelLut* lut) {
  Sel16 r;
  uint32_t n0, n1, t0, t1;
  sel16_group_lut(w[0], w[1], lut, r.k0, n0, t0);
  sel16_group_lut(w[2], w[3], lut, r.k1, n1, t1);
  r.mb = (n0 & 0x0Fu) | (n1 & 0xF0u);
  r.topkey = t0 > t1 ? t0 : t1;
  return r;
}

// Wanda selection of a bf16 group from fp32 products.  Rounding to fp32 is
// monotone, so fp32(|w_a| n_a) > fp32(|w_b| n_b) implies the exact products
// order the same way; only equal fp32 values leave the exact order open.  The
// keys are the product's fp32 bits with the low byte replaced by 2 * position
// (a further monotone truncation that keeps the four keys distinct).  When
// the second and third largest keys differ above that byte, the top-2 set is
// exactly the one the exact fp64 products give, ties included (no tie sits at
// the boundary), and the order inside the low byte never decides anything;
// otherwise the group is ambiguous and the caller ranks it exactly.
// a, b: the group's two dwords with sign bits cleared; n: its four norms.
// t1 > t2 > d2 > d1: the four keys in order.  Returns true when ambiguous.
__device__ inline bool wanda_rank_fp32(uint32_t a, uint32_t b, const float* n, uint32_t& t1,
                                       uint32_t& t2, uint32_t& d2, uint32_t& d1) {
  const float p0 = __uint_as_float(a << 16) * n[0], p1 = __uint_as_float(a & 0xFFFF0000u) * n[1];
  const float p2 = __uint_as_float(b << 16) * n[2], p3 = __uint_as_float(b & 0xFFFF0000u) * n[3];
  const uint32_t k0 = __float_as_uint(p0) & 0xFFFFFF00u;
  const uint32_t k1 = (__float_as_uint(p1) & 0xFFFFFF00u) | 2u;
  const uint32_t k2 = (__float_as_uint(p2) & 0xFFFFFF00u) | 4u;
  const uint32_t k3 = (__float_as_uint(p3) & 0xFFFFFF00u) | 6u;
  uint32_t M, m, l;
  asm("v_max3_u32 %0, %1, %2, %3" : "=v"(M) : "v"(k0), "v"(k1), "v"(k2));
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(m) : "v"(k0), "v"(k1), "v"(k2));
  asm("v_min3_u32 %0, %1, %2, %3" : "=v"(l) : "v"(k0), "v"(k1), "v"(k2));
  t1 = M > k3 ? M : k3;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(t2) : "v"(m), "v"(M), "v"(k3));
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(d2) : "v"(l), "v"(m), "v"(k3));
  d1 = l < k3 ? l : k3;
  return (t2 ^ d2) < 256u;
}

// The kept and the dropped |x| of a group as packed bf16 pairs (in rank
// order, not position order).  A key's low byte 2i is the first byte of
// element i in the group's two dwords, so the byte-permute selector that
// gathers a pair is two keys' low bytes placed side by side, plus one.
// Returns true when the group is ambiguous (kept / drop are then not the
// exact selection).
__device__ inline bool wanda_group_fp32(uint32_t a, uint32_t b, const float* n, uint32_t& kept,
                                        uint32_t& drop) {
  uint32_t t1, t2, d2, d1;
  const bool amb = wanda_rank_fp32(a, b, n, t1, t2, d2, d1);
  // selector bytes (2i, 2i + 1, 2j, 2j + 1) for the pair (i, j)
  const uint32_t ks = __builtin_amdgcn_perm(t2, t1, 0x04040000u) + 0x01000100u;
  const uint32_t ds = __builtin_amdgcn_perm(d1, d2, 0x04040000u) + 0x01000100u;
  kept = __builtin_amdgcn_perm(b, a, ks);
  drop = __builtin_amdgcn_perm(b, a, ds);
  return amb;
}

// The metadata nibble i0 | i1 << 2 (i0 < i1) of a group.  Returns true when
// the group is ambiguous (the nibble is then not the exact selection).
__device__ inline bool wanda_nibble_fp32(uint32_t a, uint32_t b, const float* n, uint32_t& nib) {
  uint32_t t1, t2, d2, d1;
  const bool amb = wanda_rank_fp32(a, b, n, t1, t2, d2, d1);
  const uint32_t q1 = t1 & 6u, q2 = t2 & 6u;  // 2 * position
  nib = ((q1 < q2 ? q1 : q2) >> 1) | ((q1 < q2 ? q2 : q1) << 1);
  return amb;
}

// Both group selections of a unit -> metadata byte (group 0 in the low nibble).
// Wanda reads the 8 channel norms of the unit (k0 = its first position).
// ---------------------------------------------------------------------------
template <class DT, bool WANDA>
__device__ inline uint32_t select_unit_norms(const Unit<DT>& u, const float* n8) {
  if constexpr (WANDA && DT::IS_BF16) {
    // fp32 products first; the exact ranking (under a wave-uniform branch,
    // so that it is skipped when no lane needs it) for units with an open
    // group
    uint32_t n0, n1;
    bool amb = wanda_nibble_fp32(u.w[0] & 0x7FFF7FFFu, u.w[1] & 0x7FFF7FFFu, n8, n0);
    amb |= wanda_nibble_fp32(u.w[2] & 0x7FFF7FFFu, u.w[3] & 0x7FFF7FFFu, n8 + 4, n1);
    if (__builtin_amdgcn_ballot_w64(amb)) {
      if (amb) {
        n0 = select_group<DT, true>(u, 0, n8);
        n1 = select_group<DT, true>(u, 1, n8 + 4);
      }
    }
    return n0 | (n1 << 4);
  }
  uint32_t n0 = select_group<DT, WANDA>(u, 0, n8);
  uint32_t n1 = select_group<DT, WANDA>(u, 1, n8 + 4);
  return n0 | (n1 << 4);
}

template <class DT, bool WANDA>
__device__ inline uint32_t select_unit(const Unit<DT>& u, const float* __restrict__ norm,
                                       int64_t k0) {
  float n8[8];
  if constexpr (WANDA) {
    const float4* np = reinterpret_cast<const float4*>(norm + k0);
    float4 a = np[0], b = np[1];
    n8[0] = a.x; n8[1] = a.y; n8[2] = a.z; n8[3] = a.w;
    n8[4] = b.x; n8[5] = b.y; n8[6] = b.z; n8[7] = b.w;
  }
  return select_unit_norms<DT, WANDA>(u, n8);
}

// The four kept elements of a unit (two per group, in position order) as raw
// storage bits.  16-bit types: two dwords, each (kept i0 | kept i1 << 16) of
// one group, gathered with a byte permute.  fp32: four dwords picked with
// selects.  Nothing is indexed at run time, so the unit stays in registers.
template <class DT>
struct Kept {
  uint32_t k[DT::ESIZE == 2 ? 2 : 4];
  __device__ inline uint32_t raw(int e) const {  // e = 0..3, compile-time after unrolling
    if constexpr (DT::ESIZE == 2) return (k[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
    else return k[e];
  }
  __device__ inline float f(int e) const { return DT::to_f32(raw(e)); }
};

__device__ inline uint32_t pick4(uint32_t i, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = (i & 1u) ? b : a;
  const uint32_t hi = (i & 1u) ? d : c;
  return (i & 2u) ? hi : lo;
}

template <class DT>
__device__ inline Kept<DT> gather_kept(const Unit<DT>& u, uint32_t mb) {
  Kept<DT> kp;
  const uint32_t n0 = mb & 0xFu, n1 = (mb >> 4) & 0xFu;
  if constexpr (DT::ESIZE == 2) {
    kp.k[0] = __builtin_amdgcn_perm(u.w[1], u.w[0], perm_sel(n0));
    kp.k[1] = __builtin_amdgcn_perm(u.w[3], u.w[2], perm_sel(n1));
  } else {
    kp.k[0] = pick4(n0 & 3u, u.w[0], u.w[1], u.w[2], u.w[3]);
    kp.k[1] = pick4(n0 >> 2, u.w[0], u.w[1], u.w[2], u.w[3]);
    kp.k[2] = pick4(n1 & 3u, u.w[4], u.w[5], u.w[6], u.w[7]);
    kp.k[3] = pick4(n1 >> 2, u.w[4], u.w[5], u.w[6], u.w[7]);
  }
  return kp;
}

// Largest |kept| of a unit as storage bits (non-negative floats order like
// their bit patterns).
template <class DT>
__device__ inline uint32_t kept_absmax(const Kept<DT>& kp) {
  if constexpr (DT::ESIZE == 2) {
    const uint32_t a = kp.k[0] & 0x7FFF7FFFu, b = kp.k[1] & 0x7FFF7FFFu;
    const uint32_t m = (a & 0xFFFFu) > (b & 0xFFFFu) ? (a & 0xFFFFu) : (b & 0xFFFFu);
    const uint32_t h = (a >> 16) > (b >> 16) ? (a >> 16) : (b >> 16);
    return m > h ? m : h;
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = kp.k[e] & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
    return m;
  }
}

// Pairwise 4:8 [PD §6]: a unit is one group of eight = four adjacent pairs.
// Pair energy e_p = fp64(a^2 + b^2) (exact squares, one rounding, as
// fma(b, b, a*a)); the two pairs with the largest energy are kept, ties to
// the lower pair.  Pair p beats q (p < q) iff e_p >= e_q; with that strict
// total order exactly two pairs win at least two of their three contests.
// Returns the nibble p0 | p1 << 2 (p0 < p1).
template <class DT>
__device__ inline uint32_t select_pairs48(const Unit<DT>& u) {
  double e[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const double a = (double)u.f(2 * p), b = (double)u.f(2 * p + 1);
    e[p] = __builtin_fma(b, b, a * a);
  }
  const uint32_t c01 = e[0] >= e[1], c02 = e[0] >= e[2], c03 = e[0] >= e[3];
  const uint32_t c12 = e[1] >= e[2], c13 = e[1] >= e[3], c23 = e[2] >= e[3];
  const uint32_t w0 = c01 + c02 + c03, w1 = (1u - c01) + c12 + c13;
  const uint32_t w2 = (1u - c02) + (1u - c12) + c23, w3 = (1u - c03) + (1u - c13) + (1u - c23);
  const uint32_t m = (uint32_t)(w0 >= 2) | ((uint32_t)(w1 >= 2) << 1) | ((uint32_t)(w2 >= 2) << 2) |
                     ((uint32_t)(w3 >= 2) << 3);
  const uint32_t p0 = (uint32_t)__builtin_ctz(m), p1 = 31u - (uint32_t)__builtin_clz(m);
  return p0 | (p1 << 2);
}

// 8-bit element mask of a pairwise-4:8 nibble.
__device__ inline uint32_t pairs48_mask(uint32_t nib) {
  return (3u << (2 * (nib & 3u))) | (3u << (2 * (nib >> 2)));
}

// The two kept pairs of a unit as raw storage bits (pair order).
template <class DT>
__device__ inline Kept<DT> gather_pairs48(const Unit<DT>& u, uint32_t nib) {
  Kept<DT> kp;
  const uint32_t p0 = nib & 3u, p1 = nib >> 2;
  if constexpr (DT::ESIZE == 2) {
    kp.k[0] = pick4(p0, u.w[0], u.w[1], u.w[2], u.w[3]);
    kp.k[1] = pick4(p1, u.w[0], u.w[1], u.w[2], u.w[3]);
  } else {
    kp.k[0] = pick4(p0, u.w[0], u.w[2], u.w[4], u.w[6]);
    kp.k[1] = pick4(p0, u.w[1], u.w[3], u.w[5], u.w[7]);
    kp.k[2] = pick4(p1, u.w[0], u.w[2], u.w[4], u.w[6]);
    kp.k[3] = pick4(p1, u.w[1], u.w[3], u.w[5], u.w[7]);
  }
  return kp;
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

// Four e4m3 codes packed little-endian in a dword (element 0 in byte 0), with
// gfx950's v_cvt_pk_fp8_f32 (OCP e4m3, RNE).  Over every finite fp32 with
// |y| < 464 it returns exactly enc_e4m3(y); every caller's |y| is at most
// 448 * (1 + 2^-23), so no clamp is needed.
__device__ inline uint32_t enc_e4m3_x4(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Value of an e4m3 code held in byte SEL of w (gfx950 v_cvt_f32_fp8).
template <int SEL>
__device__ inline float dec_e4m3_hw(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// Values of the two e4m3 codes in 16-bit half H of w, low byte first
// (gfx950 v_cvt_pk_f32_fp8: one instruction for two codes).
template <int H>
__device__ inline f32x2 dec_e4m3_hw_x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, H != 0);
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

// Bit pattern of dec_e2m1(c) (for the conversion check).
__device__ inline uint32_t dec_e2m1_bits(uint32_t c) { return __float_as_uint(dec_e2m1(c)); }


// Values of the two E2M1 codes in byte SEL of w (low nibble -> .x), with
// gfx950's v_cvt_scalef32_pk_f32_fp4 at scale 1; equal to dec_e2m1 on every
// byte and byte position (checked exhaustively by check_converts).
template <int SEL>
__device__ inline f32x2 dec_e2m1_hw_x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Eight E2M1 codes packed two per byte (element 2j in the low nibble of byte
// j) with gfx950's v_cvt_scalef32_pk_fp4_f32 at scale 1; over every finite
// fp32 it returns exactly enc_e2m1 (RNE, saturating at 6, sign copied).
__device__ inline uint32_t enc_e2m1_x8(const float* y) {
  uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], 1.0f, 3);
}

// Four E2M1 codes in bits 0..15 (element j in nibble j), same conversion.
__device__ inline uint32_t enc_e2m1_x4(float a, float b, float c, float d) {
  const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c, d, 1.0f, 1);
}

// Symmetric INT rounding through the fp32 adder: for |y| <= qmax < 2^22,
// fp32(clamp(y) + 1.5 * 2^23) holds round-half-even(clamp(y)) in its low
// mantissa bits (the add rounds to nearest even at unit spacing).  Clamping
// before rounding equals clamping after because qmax is an integer.  The low
// byte / half of the result's bits is the two's-complement code.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23, bit pattern 0x4B400000
__device__ inline float int_round_magic(float y, float qmax) {
  return __builtin_amdgcn_fmed3f(y, -qmax, qmax) + kRoundMagic;
}
// code value as an exact float
__device__ inline float int_code_value(float magic_sum) { return magic_sum - kRoundMagic; }

// Symmetric INT code as float (exact integer value), clamp to [-qmax, qmax].
__device__ inline float enc_int(float y, float qmax) {
  float q = __builtin_rintf(y);
  return __builtin_fminf(__builtin_fmaxf(q, -qmax), qmax);
}

// ---------------------------------------------------------------------------
// Lane exchange and team reductions.
// ---------------------------------------------------------------------------
// Value of lane (lane ^ D) of the wave.  DPP row operations for D <= 8
// (quad_perm [1,0,3,2] and [2,3,0,1]; D = 4 as a quad reverse followed by a
// half-row mirror, i ^ 3 ^ 7 = i ^ 4; row_ror:8 on 16-lane rows), ds_swizzle
// (xor mask 16 within 32 lanes) and ds_bpermute for 32.  Every lane of the
// wave must be active.
template <int CTRL>
__device__ inline uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int D>
__device__ inline uint32_t xor_lane32(uint32_t v) {
  if constexpr (D == 1) return dpp32<0xB1>(v);
  else if constexpr (D == 2) return dpp32<0x4E>(v);
  else if constexpr (D == 4) return dpp32<0x141>(dpp32<0x1B>(v));
  else if constexpr (D == 8) return dpp32<0x128>(v);
  else if constexpr (D == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
  else return (uint32_t)__shfl_xor((int)v, D, 64);
}
template <int D>
__device__ inline double xor_lane(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = xor_lane32<D>((uint32_t)b), hi = xor_lane32<D>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

// Xor butterflies over the TEAM (<= 64) adjacent lanes of a team: DPP row
// operations for distances 1..8, ds_swizzle for 16, and for a whole wave the
// two half-wave results read as scalars.  Every lane ends with the team's
// result, combined in a fixed order (deterministic; commutative + and max give
// all lanes the same bits).  Every lane of the wave must take part.
template <int TEAM>
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  if constexpr (TEAM > 1) { const uint32_t w = xor_lane32<1>(v); v = v > w ? v : w; }
  if constexpr (TEAM > 2) { const uint32_t w = xor_lane32<2>(v); v = v > w ? v : w; }
  if constexpr (TEAM > 4) { const uint32_t w = xor_lane32<4>(v); v = v > w ? v : w; }
  if constexpr (TEAM > 8) { const uint32_t w = xor_lane32<8>(v); v = v > w ? v : w; }
  if constexpr (TEAM > 16) { const uint32_t w = xor_lane32<16>(v); v = v > w ? v : w; }
  if constexpr (TEAM > 32) {
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    v = a > b ? a : b;
  }
  return v;
}

template <int TEAM>
__device__ inline double wave_sum_f64(double v) {
  if constexpr (TEAM > 1) v += xor_lane<1>(v);
  if constexpr (TEAM > 2) v += xor_lane<2>(v);
  if constexpr (TEAM > 4) v += xor_lane<4>(v);
  if constexpr (TEAM > 8) v += xor_lane<8>(v);
  if constexpr (TEAM > 16) v += xor_lane<16>(v);
  if constexpr (TEAM > 32) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t l0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 0);
    const uint32_t h0 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 0);
    const uint32_t l1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, 32);
    const uint32_t h1 = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 32);
    v = __builtin_bit_cast(double, (uint64_t)l0 | ((uint64_t)h0 << 32)) +
        __builtin_bit_cast(double, (uint64_t)l1 | ((uint64_t)h1 << 32));
  }
  return v;
}

// Teams wider than a wave combine their waves through LDS (all threads of the
// block must call these together).
template <int TEAM>
__device__ inline uint32_t team_max_u32(uint32_t v, uint32_t* lds) {
  if constexpr (TEAM <= 64) {
    return wave_max_u32<TEAM>(v);
  } else {
    v = wave_max_u32<64>(v);
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
    return wave_sum_f64<TEAM>(v);
  } else {
    v = wave_sum_f64<64>(v);
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

// ---------------------------------------------------------------------------
// Block Hadamard rotation along K [PD §4: before low-bit quantization the
// operand is multiplied by a rescaled +-1 orthogonal Hadamard matrix].  Each
// aligned block of n elements becomes y = H_n x / sqrt(n) (Sylvester order),
// in the storage type: the sums S are fp64 butterflies (exact whenever the
// block's values span at most 53 - log2(n) bits from the largest magnitude to
// the lowest set bit, so the butterfly order does not matter), a zero sum is
// +0, then fp64(S * c) is rounded to fp32 and to the storage type (RNE).
// A block of n <= 8 * TEAM elements is n/8 units on adjacent lanes of one
// register j (lane t owns units t, t + TEAM, ...), so the butterflies run
// three stages inside a unit and log2(n/8) stages across lanes; longer blocks
// run on whole-workgroup teams (hadamard_team).
// ---------------------------------------------------------------------------
template <class DT>
__device__ inline void unit_store_f32(Unit<DT>& u, const float* f) {
  if constexpr (DT::ESIZE == 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) u.w[e] = __float_as_uint(f[e]);
  } else {
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (DT::IS_BF16) {
        const uint32_t b = __float_as_uint(f[e]);
        h[e] = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;  // RNE, finite values
      } else {
        h[e] = __builtin_bit_cast(uint16_t, (_Float16)f[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) u.w[i] = h[2 * i] | (h[2 * i + 1] << 16);
  }
}

// One butterfly stage across lanes at unit distance D: the lower lane of a
// pair keeps a + b, the upper one a - b (as fma(-1, b, a), exact like the
// subtraction).
template <int D>
__device__ inline void had_xlane(double (&v)[8], int t) {
  const double sgn = (t & D) ? -1.0 : 1.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double p = xor_lane<D>(v[e]);
    v[e] = __builtin_fma(sgn, v[e], p);
  }
}

// The three in-unit butterfly stages and the cross-lane stages of blocks of
// nb units (nb <= 64) on fp64 values.
__device__ inline void had_unit_lanes(double (&v)[8], int nb, int t) {
#pragma unroll
  for (int d = 1; d < 8; d <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!(e & d)) {
        const double a = v[e], b = v[e | d];
        v[e] = a + b;
        v[e | d] = a - b;
      }
  if (nb > 1) had_xlane<1>(v, t);
  if (nb > 2) had_xlane<2>(v, t);
  if (nb > 4) had_xlane<4>(v, t);
  if (nb > 8) had_xlane<8>(v, t);
  if (nb > 16) had_xlane<16>(v, t);
  if (nb > 32) had_xlane<32>(v, t);
}

template <class DT>
__device__ inline void unit_store_rotated(Unit<DT>& u, const double (&v)[8], double c) {
  float f[8];
  // fma(v, c, +0) is (v + 0) * c in one rounding: a zero sum becomes +0, and
  // any other sum is scaled exactly once
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)__builtin_fma(v[e], c, 0.0);
  unit_store_f32(u, f);
}

template <class DT>
__device__ inline void hadamard_unit(Unit<DT>& u, int nb, double c, int t) {
  double v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (double)u.f(e);
  had_unit_lanes(v, nb, t);
  unit_store_rotated(u, v, c);
}

// Blocks of 1024 .. 4096 elements on whole-workgroup teams (TEAM = kBlock =
// 256 lanes; lane t's register j holds unit 256 j + t, so a 4096-element
// block is 16 elements per lane).  After the unit and in-wave lane stages, a
// 4096-element block adds the stage between a lane's registers j and j ^ 1,
// and every block the stages between waves (lane bit 6, and bit 7 from 2048
// elements on), done in one exchange through LDS.  Every thread of the
// workgroup must call this (it holds two workgroup barriers).
template <class DT, int UPL>
__device__ inline void hadamard_team(Unit<DT> (&u)[UPL], const Rot& r, int t) {
  static_assert(UPL <= 4, "rows of up to 8192 elements (32 KB of LDS per 2 registers)");
  typedef double f64x2 __attribute__((ext_vector_type(2)));
  __shared__ f64x2 xw[UPL * 4][kBlock];  // element pairs (e, e + 1): 16-byte LDS accesses
  double v[UPL][8];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = (double)u[j].f(e);
    had_unit_lanes(v[j], 64, t);
  }
  if (r.n == 4096) {
#pragma unroll
    for (int j = 0; j + 1 < UPL; j += 2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double a = v[j][e], b = v[j + 1][e];
        v[j][e] = a + b;
        v[j + 1][e] = a - b;
      }
  }
  __syncthreads();  // the previous row's reads of xw are done
#pragma unroll
  for (int j = 0; j < UPL; ++j)
#pragma unroll
    for (int e = 0; e < 8; e += 2) xw[j * 4 + e / 2][t] = f64x2{v[j][e], v[j][e + 1]};
  __syncthreads();
  const int q = t >> 6, l = t & 63;
#pragma unroll
  for (int j = 0; j < UPL; ++j)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f64x2* col = xw[j * 4 + e / 2];
      if (r.n == 1024) {  // waves 2c, 2c + 1 hold one block: the lower keeps a + b, the upper a - b
        const f64x2 p = col[t ^ 64];
        v[j][e] = (q & 1) ? p.x - v[j][e] : v[j][e] + p.x;
        v[j][e + 1] = (q & 1) ? p.y - v[j][e + 1] : v[j][e + 1] + p.y;
      } else {  // lane bits 6 and 7: the 4-point transform over the four waves
        const f64x2 a0 = col[l], a1 = col[l + 64], a2 = col[l + 128], a3 = col[l + 192];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const double s01 = (q & 1) ? a0[k] - a1[k] : a0[k] + a1[k];
          const double s23 = (q & 1) ? a2[k] - a3[k] : a2[k] + a3[k];
          v[j][e + k] = (q & 2) ? s01 - s23 : s01 + s23;
        }
      }
    }
#pragma unroll
  for (int j = 0; j < UPL; ++j) unit_store_rotated(u[j], v[j], r.c);
}

// ROT = 1: blocks of up to 512 elements (and at most 8 * TEAM), rotated unit
// by unit.  ROT = 3: blocks of 1024 .. 4096 elements on whole-workgroup teams
// (hadamard_team).
template <class DT, int TEAM, int UPL, int ROT>
__device__ inline void hadamard_units(Unit<DT> (&u)[UPL], const Rot& r, int t) {
  static_assert(ROT == 1 || ROT == 3, "rotation variants 1 and 3");
  if constexpr (ROT == 1) {
#pragma unroll
    for (int j = 0; j < UPL; ++j) hadamard_unit(u[j], r.n >> 3, r.c, t);
  } else {
    static_assert(TEAM == kBlock, "whole-workgroup teams only");
    hadamard_team<DT, UPL>(u, r, t);
  }
}

struct RowGeom {
  const char* x;
  int64_t R, nrows, nunits, bs, rs;  // strides in bytes
  Rot rot;                           // rotation on load (n == 0: none)
};

__device__ inline const char* row_ptr(const RowGeom& g, int64_t row) {
  if (g.bs == g.R * g.rs) return g.x + row * g.rs;
  const int64_t b = row / g.R;
  return g.x + b * g.bs + (row - b * g.R) * g.rs;
}

// Every lane issues all UPL loads (a unit past the row's end or a row past
// the last re-reads unit 0 of the operand, which always exists when a kernel
// runs) and zeroes those units afterwards.  With no load under a branch the
// compiler waits for each unit's load just before its first use, so work on
// early units overlaps the arrival of later ones (2-6% on every row kernel).
template <class DT, int TEAM, int UPL>
__device__ inline void load_row(Unit<DT> (&u)[UPL], const RowGeom& g, int64_t row, int t) {
  const bool act = row < g.nrows;
  const char* xr = act ? row_ptr(g, row) : g.x;
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int64_t i = (int64_t)j * TEAM + t;
    const bool ok = act && i < g.nunits;
    load_unit(u[j], ok ? xr + i * (8 * DT::ESIZE) : g.x);
    if (!ok) zero_unit(u[j]);
  }
}

// ---------------------------------------------------------------------------
// Row driver.  Rows are flattened over (b, r); team k of the grid takes rows
// k, k + nteams, k + 2*nteams, ...: one row per team when the grid covers
// every row (the streaming kernels), several for a persistent grid (the
// energy kernels).  The trip count is the same for every team, so team
// reductions that synchronise a workgroup are reached by all of its threads.
// ---------------------------------------------------------------------------
// pre() runs once, after the first row's loads are issued and before they
// are used (set-up such as an LDS table then overlaps the loads' latency);
// every thread of the workgroup calls it.
template <class DT, int TEAM, int UPL, int ROT = 0, class Pre, class Body>
__device__ inline void for_each_row(const RowGeom& g, Pre&& pre, Body&& body) {
  constexpr int TPB = kBlock / TEAM;
  const int t = threadIdx.x % TEAM;
  const int64_t first = (int64_t)blockIdx.x * TPB + threadIdx.x / TEAM;
  const int64_t stride = (int64_t)gridDim.x * TPB;
  const int64_t iters = (g.nrows + stride - 1) / stride;
  for (int64_t it = 0; it < iters; ++it) {
    Unit<DT> A[UPL];
    const int64_t ra = first + it * stride;
    load_row<DT, TEAM, UPL>(A, g, ra, t);
    if (it == 0) pre();
    if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(A, g.rot, t);
    body(A, ra, t);
  }
}
template <class DT, int TEAM, int UPL, int ROT = 0, class Body>
__device__ inline void for_each_row(const RowGeom& g, Body&& body) {
  for_each_row<DT, TEAM, UPL, ROT>(g, [] {}, body);
}

// Same with contiguous rows per team, so the rows a team sums lie in as few
// row blocks as possible.  With q = rows / teams (rounded down), the teams of
// the first workgroups take q + 1 rows each and the others q, just enough
// workgroups taking q + 1 to cover the rows, so a SIMD's teams share the rows
// evenly instead of every team running ceil(rows / teams) iterations.  The
// count is uniform over a workgroup (its team reductions may synchronise the
// workgroup); an iteration past the operand's last row passes row = g.nrows
// and zero units.
struct ContigRows {
  int64_t first, count;
};
template <int TEAM>
__device__ inline ContigRows contig_rows(const RowGeom& g) {
  constexpr int64_t TPB = kBlock / TEAM;
  const int64_t nw = gridDim.x, w = blockIdx.x;
  const int64_t q = g.nrows / (nw * TPB);
  const int64_t rem = g.nrows - q * nw * TPB;
  const int64_t e = (rem + TPB - 1) / TPB;  // workgroups whose teams take q + 1 rows
  const int64_t n = w < e ? q + 1 : q;
  const int64_t base = w < e ? w * TPB * (q + 1) : e * TPB * (q + 1) + (w - e) * TPB * q;
  return ContigRows{base + (int64_t)(threadIdx.x / TEAM) * n, n};
}
template <int TEAM>
__device__ inline int64_t contig_first_row(const RowGeom& g) {
  return contig_rows<TEAM>(g).first;
}
template <class DT, int TEAM, int UPL, int ROT = 0, class Body>
__device__ inline void for_each_row_contig(const RowGeom& g, Body&& body) {
  const int t = threadIdx.x % TEAM;
  const ContigRows cr = contig_rows<TEAM>(g);
  const int64_t rpt = cr.count, r0 = cr.first;
  const int64_t r1 = r0 + rpt < g.nrows ? r0 + rpt : g.nrows;
  for (int64_t it = 0; it < rpt; ++it) {
    Unit<DT> A[UPL];
    const int64_t ra = r0 + it < r1 ? r0 + it : g.nrows;
    load_row<DT, TEAM, UPL>(A, g, ra, t);
    if constexpr (ROT) hadamard_units<DT, TEAM, UPL, ROT>(A, g.rot, t);
    body(A, ra, t);
  }
}

// ---------------------------------------------------------------------------
// Block-format and tensor-scale helpers shared by the quantizer, energy and
// operator-error kernels.
// ---------------------------------------------------------------------------
// Reduce the partial maxima in a workgroup (every thread gets T).
__device__ inline float block_tensor_amax(const float* tamax_in, const uint32_t* partials,
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

// NVFP4 tensor scale and block-scale multiplier from T.
__device__ inline void nv_tensor_scales(float T, float& s_t, float& g) {
  if (T >= 0x1p-64f) {
    s_t = T / 2688.0f;
    g = 448.0f / T;
  } else {
    s_t = 0.0f;
    g = 0.0f;
  }
}

// NVFP4 block scales.  The e4m3 code of a block's scale fp32(am * g) (am >= 0
// the block's absolute maximum, g = fp32(448 / T)) comes from the hardware
// convert of the product clamped to 448, where it equals enc_e4m3 (the
// product can pass 448 when the caller's T is below the operand's maximum,
// and enc_e4m3 saturates).  The
// elements' multiplier fp32(1 / fp32(dec_e4m3(code) * s_t)) (0 for a zero
// scale) comes from a table of the non-negative codes filled once per
// workgroup: the same fp32 operations, done once per code instead of once
// per block.  The table is ready after the next workgroup barrier.
constexpr int kNvInvEntries = 128;
__device__ inline void nv_inv_fill(float* tab, float s_t) {
  for (int c = threadIdx.x; c < kNvInvEntries; c += blockDim.x) {
    const float d = dec_e4m3((uint32_t)c) * s_t;
    tab[c] = d > 0.0f ? 1.0f / d : 0.0f;
  }
}
__device__ inline uint32_t nv_block_code(float am, float g) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fminf(am * g, 448.0f), 0.0f, 0u, false) & 0xFFu;
}

__device__ inline int mx_exponent(uint32_t amax_bits) {
  // floor(log2(amax)) - 2, clamped to [-127, 127]; amax == 0 -> -127
  if (amax_bits == 0) return -127;
  int fl;
  const uint32_t ex = amax_bits >> 23;
  if (ex) fl = (int)ex - 127;
  else fl = (31 - __builtin_clz(amax_bits)) - 149;  // fp32 subnormal
  int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Quantize-dequantize of 4 values with a per-row scale: returns the 4 code
// values (exact floats) in c[].  fmt: CF_FP8 or CF_INT8/CF_INT16.
__device__ inline void qdq_row4(int fmt, float inv, float qmax, const float* v, float* c) {
  if (fmt == CF_FP8) {
    const uint32_t w = enc_e4m3_x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    c[0] = dec_e4m3_hw<0>(w);
    c[1] = dec_e4m3_hw<1>(w);
    c[2] = dec_e4m3_hw<2>(w);
    c[3] = dec_e4m3_hw<3>(w);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = int_code_value(int_round_magic(v[e] * inv, qmax));
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
