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

#ifndef SPARQ24_WIDE_E
#define SPARQ24_WIDE_E 0
#endif
// fp32 / fp16 energy kernel on rows of 2049..4096 elements: two-wave teams
// (TEAM 128, 4 units per lane).  The one-wave form holds 64 elements per lane
// and spills at one wave per SIMD; two-wave teams measured 5-10% faster on
// fp32 and the same on fp16.
#ifndef SPARQ24_WIDE_EG
#define SPARQ24_WIDE_EG 1
#endif

namespace sparq24 {

template <class DT>
__device__ inline uint32_t unit_absmax_e(const Unit<DT>& u) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < DT::W; ++i) {
    if constexpr (DT::ESIZE == 2) {
      const uint32_t a = u.w[i] & 0x7FFF7FFFu;
      const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
      const uint32_t h = lo > hi ? lo : hi;
      m = m > h ? m : h;
    } else {
      const uint32_t a = u.w[i] & 0x7FFFFFFFu;
      m = m > a ? m : a;
    }
  }
  return m;
}

// ---------------------------------------------------------------------------
// bf16 + magnitude fast path.  The top-2 network already orders each group's
// keys; a key's high half is the element's bf16 magnitude, i.e. the fp32 bit
// pattern of |x|.  So the two kept and the two dropped magnitudes fall out of
// the network (two extra mins), and because every quantizer here is
// symmetric in sign (RNE integers, sign-magnitude e4m3/e2m1 with the sign
// copied), each error energy depends on |x| only.  The group maximum is
// always kept, so the kept row maximum is also the plain row maximum.
// Per unit the 8 magnitudes are held as kept (0..3) then dropped (4..7);
// block quantizers only need a unit's membership, not the order inside it.
// Squared residuals are summed pairwise in fp32 over a unit (at most three
// roundings after the single-rounded fp32 residual, < 3.6e-7 relative) and
// accumulated in fp64.
// ---------------------------------------------------------------------------
// Kept and dropped magnitudes of one group as packed bf16 pairs: bits 0..15
// and 16..31 each hold a |x| bf16 pattern.
// The four keys in order, t1 > t2 > d2 > d1: with M, m and n the max, median
// and min of k0..k2, t1 = max(M, k3), t2 = median(m, M, k3), d2 = median(n,
// m, k3), d1 = min(n, k3) (7 instructions instead of a 10-instruction
// network).
__device__ inline uint32_t u32_max3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_max3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline uint32_t u32_min3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_min3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline uint32_t u32_med3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline void sort4_keys(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3, uint32_t& t1,
                                  uint32_t& t2, uint32_t& d2, uint32_t& d1) {
  const uint32_t M = u32_max3(k0, k1, k2), m = u32_med3(k0, k1, k2), n = u32_min3(k0, k1, k2);
  t1 = M > k3 ? M : k3;
  t2 = u32_med3(m, M, k3);
  d2 = u32_med3(n, m, k3);
  d1 = n < k3 ? n : k3;
}

__device__ inline void sel16_mags_packed(uint32_t w0, uint32_t w1, uint32_t& kept, uint32_t& drop,
                                         uint32_t& top) {
  const uint32_t a = w0 & 0x7FFF7FFFu, b = w1 & 0x7FFF7FFFu;
  const uint32_t k0 = (a << 16) | 3u, k1 = (a & 0xFFFF0000u) | 2u;
  const uint32_t k2 = (b << 16) | 1u, k3 = b & 0xFFFF0000u;
  uint32_t t1, t2, d2, d1;
  sort4_keys(k0, k1, k2, k3, t1, t2, d2, d1);
  kept = __builtin_amdgcn_perm(t2, t1, 0x07060302u);  // t1 high half low, t2 high half high
  drop = __builtin_amdgcn_perm(d2, d1, 0x07060302u);
  top = t1;
}
__device__ inline float mag_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ inline float mag_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

__device__ inline void sel16_mags(uint32_t w0, uint32_t w1, float* kept2, float* drop2,
                                  uint32_t& top) {
  const uint32_t a = w0 & 0x7FFF7FFFu, b = w1 & 0x7FFF7FFFu;
  const uint32_t k0 = (a << 16) | 3u, k1 = (a & 0xFFFF0000u) | 2u;
  const uint32_t k2 = (b << 16) | 1u, k3 = b & 0xFFFF0000u;
  uint32_t t1, t2, d2, d1;
  sort4_keys(k0, k1, k2, k3, t1, t2, d2, d1);
  kept2[0] = __uint_as_float(t1 & 0xFFFF0000u);
  kept2[1] = __uint_as_float(t2 & 0xFFFF0000u);
  drop2[0] = __uint_as_float(d1 & 0xFFFF0000u);
  drop2[1] = __uint_as_float(d2 & 0xFFFF0000u);
  top = t1;
}

// The two positions of 0..3 absent from a pair nibble (i0 | i1 << 2, i0 < i1),
// in the same encoding.
__device__ inline uint32_t other_pair(uint32_t n) {
  const uint32_t dm = 0xFu ^ ((1u << (n & 3u)) | (1u << (n >> 2)));
  return (uint32_t)__builtin_ctz(dm) | ((31u - (uint32_t)__builtin_clz(dm)) << 2);
}

// Selections of the packed-magnitude energy kernel.
enum { SEL_MAG = 0, SEL_WANDA = 1, SEL_P48 = 2 };

// Kept and dropped |x| of one bf16 unit as packed pairs: pk[0], pk[1] the
// four kept magnitudes, pk[2], pk[3] the four dropped ones (Wanda 2:4 or
// pairwise 4:8; magnitude 2:4 has its own faster path).  Units past the
// row's end (valid = false) are zeros and select anything.
template <int SEL>
__device__ inline void unit_mags_packed(const Unit<BF16T>& u, const float* __restrict__ norm,
                                        int64_t k0, bool valid, uint32_t (&pk)[4]) {
  if constexpr (SEL == SEL_WANDA) {
    const uint32_t mb = valid ? select_unit<BF16T, true>(u, norm, k0) : 0x44u;
    const uint32_t n0 = mb & 0xFu, n1 = mb >> 4;
    pk[0] = __builtin_amdgcn_perm(u.w[1], u.w[0], perm_sel(n0)) & 0x7FFF7FFFu;
    pk[1] = __builtin_amdgcn_perm(u.w[3], u.w[2], perm_sel(n1)) & 0x7FFF7FFFu;
    pk[2] = __builtin_amdgcn_perm(u.w[1], u.w[0], perm_sel(other_pair(n0))) & 0x7FFF7FFFu;
    pk[3] = __builtin_amdgcn_perm(u.w[3], u.w[2], perm_sel(other_pair(n1))) & 0x7FFF7FFFu;
  } else {
    // a bf16 pair (2p, 2p+1) is dword p of the unit
    const uint32_t nb = select_pairs48(u), dn = other_pair(nb);
    pk[0] = pick4(nb & 3u, u.w[0], u.w[1], u.w[2], u.w[3]) & 0x7FFF7FFFu;
    pk[1] = pick4(nb >> 2, u.w[0], u.w[1], u.w[2], u.w[3]) & 0x7FFF7FFFu;
    pk[2] = pick4(dn & 3u, u.w[0], u.w[1], u.w[2], u.w[3]) & 0x7FFF7FFFu;
    pk[3] = pick4(dn >> 2, u.w[0], u.w[1], u.w[2], u.w[3]) & 0x7FFF7FFFu;
  }
}

// Squared residual energy of N magnitudes (N = 4 or 8) under a per-row scale
// (s, inv) taken from a row maximum that no magnitude exceeds.  Each residual
// is one fp32 rounding of code*s - v; the squares go into two fp32 chains of
// fused multiply-adds that are added at the end (at most N/2 + 1 roundings
// after the residual's, < 3.6e-7 relative for N = 8).
template <int N>
__device__ inline float mag_sq_err_fp8(float s, float inv, const float* v) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int q = 0; q < N; q += 4) {
    const uint32_t w = enc_e4m3_x4(v[q] * inv, v[q + 1] * inv, v[q + 2] * inv, v[q + 3] * inv);
    const float e0 = __builtin_fmaf(dec_e4m3_hw<0>(w), s, -v[q + 0]);
    const float e1 = __builtin_fmaf(dec_e4m3_hw<1>(w), s, -v[q + 1]);
    const float e2 = __builtin_fmaf(dec_e4m3_hw<2>(w), s, -v[q + 2]);
    const float e3 = __builtin_fmaf(dec_e4m3_hw<3>(w), s, -v[q + 3]);
    a0 = __builtin_fmaf(e0, e0, a0);
    a1 = __builtin_fmaf(e1, e1, a1);
    a0 = __builtin_fmaf(e2, e2, a0);
    a1 = __builtin_fmaf(e3, e3, a1);
  }
  return a0 + a1;
}

// Same for symmetric INT.  v <= amax and inv = fp32(qmax / amax) give
// v * inv <= qmax * (1 + 2^-24)^2 < qmax + 1/2, so round-to-nearest-even
// never leaves [0, qmax] and the clamp of the encoder is a no-op here.
template <int N>
__device__ inline float mag_sq_err_int(float s, float inv, const float* v) {
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int q = 0; q < N; q += 2) {
    const float e0 = __builtin_fmaf(__builtin_rintf(v[q] * inv), s, -v[q]);
    const float e1 = __builtin_fmaf(__builtin_rintf(v[q + 1] * inv), s, -v[q + 1]);
    a0 = __builtin_fmaf(e0, e0, a0);
    a1 = __builtin_fmaf(e1, e1, a1);
  }
  return a0 + a1;
}

// fp32 sum of the squares of 8 residuals: four chains of two fused
// multiply-adds, added pairwise (4 roundings after the residuals').
__device__ inline float sq_sum8(const float* e) {
  float a[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = __builtin_fmaf(e[k + 4], e[k + 4], e[k] * e[k]);
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// Residuals of 8 values whose E2M1 codes are packed in pk (value 2j in the
// low nibble of byte j), decoded in hardware and scaled by m then s
// (x_hat = code * m * s; code * m is exact for the callers' m).
__device__ inline void e2m1_residuals8(uint32_t pk, float m, float s, const float* v, float* e) {
  const f32x2 c[4] = {dec_e2m1_hw_x2<0>(pk), dec_e2m1_hw_x2<1>(pk), dec_e2m1_hw_x2<2>(pk),
                      dec_e2m1_hw_x2<3>(pk)};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    e[2 * k] = __builtin_fmaf(c[k].x * m, s, -v[2 * k]);
    e[2 * k + 1] = __builtin_fmaf(c[k].y * m, s, -v[2 * k + 1]);
  }
}

// Squared residual energy of the 8 values of one unit under MXFP4 with block
// exponent ex (x_hat = code * 2^ex).
__device__ inline float unit_sq_err_mx8(const float* v, int ex) {
  float y[8], e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = __builtin_ldexpf(v[k], -ex);
  e2m1_residuals8(enc_e2m1_x8(y), 1.0f, __builtin_ldexpf(1.0f, ex), v, e);
  return sq_sum8(e);
}

// Same under NVFP4: bm = fp32 bits of the 16-value block's absolute maximum,
// s_t / gnv the tensor scale and block-scale multiplier.
__device__ inline float unit_sq_err_nv8(const float* v, uint32_t bm, float s_t, float gnv) {
  const float bval = dec_e4m3(enc_e4m3(__uint_as_float(bm) * gnv));
  const float d = bval * s_t;
  const float inv = d > 0.0f ? 1.0f / d : 0.0f;
  float y[8], e[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = v[k] * inv;
  e2m1_residuals8(enc_e2m1_x8(y), bval, s_t, v, e);
  return sq_sum8(e);
}

// Error energy of 4 kept values (one unit) under a block format whose block
// spans NB adjacent lanes' units (NV: 4 units = 16 kept, MX: 8 = 32);
// every lane of the wave must call this.  Returns the fp32 sum of the four
// squared fp32-rounded residuals.
template <bool NV>
__device__ inline float kept_block_err4(const float* v, float s_t, float gnv) {
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
  float r[4];
  uint32_t pk;
  float m, sc;
  if constexpr (NV) {
    const float bval = dec_e4m3(enc_e4m3(__uint_as_float(am) * gnv));
    const float d = bval * s_t;
    const float inv = d > 0.0f ? 1.0f / d : 0.0f;
    pk = enc_e2m1_x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    m = bval;
    sc = s_t;
  } else {
    w = (uint32_t)__shfl_xor((int)am, 4, 64);
    am = am > w ? am : w;
    const int ex = mx_exponent(am);
    pk = enc_e2m1_x4(__builtin_ldexpf(v[0], -ex), __builtin_ldexpf(v[1], -ex),
                     __builtin_ldexpf(v[2], -ex), __builtin_ldexpf(v[3], -ex));
    m = 1.0f;
    sc = __builtin_ldexpf(1.0f, ex);
  }
  const f32x2 c0 = dec_e2m1_hw_x2<0>(pk), c1 = dec_e2m1_hw_x2<1>(pk);
  r[0] = __builtin_fmaf(c0.x * m, sc, -v[0]);
  r[1] = __builtin_fmaf(c0.y * m, sc, -v[1]);
  r[2] = __builtin_fmaf(c1.x * m, sc, -v[2]);
  r[3] = __builtin_fmaf(c1.y * m, sc, -v[3]);
  return __builtin_fmaf(r[0], r[0], r[2] * r[2]) + __builtin_fmaf(r[1], r[1], r[3] * r[3]);
}

// Reduce rows r0..r1-1 of every partial column (rowpart[col][row], nrows per
// column) in a fixed order and write block blk's outputs: mode 0 = Sx2,
// Sdropped, kept error, dense error; mode 1 = E_prune, E_qkept, E_2:4,
// E_dense, R per pair.  Every thread of the workgroup must call this.
__device__ inline void finalize_rows(const double* __restrict__ rowpart, int64_t nrows,
                                     int64_t r0, int64_t r1, const FinalizeParams& f,
                                     double* __restrict__ out, int64_t blk) {
  constexpr int CB = 8;  // columns reduced together: CB independent loads per row
  __shared__ double sh[CB][kBlock / 64];
  __shared__ double sb[2 + 2 * kMaxQ];
  for (int cb = 0; cb < f.ncols; cb += CB) {
    double a[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) a[c] = 0.0;
    // branch-free body: columns past the end re-read the last one (ignored),
    // so all CB loads of a row can be in flight together
    const double* colp[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) colp[c] = rowpart + (int64_t)((cb + c) < f.ncols ? cb + c : f.ncols - 1) * nrows;
    // RU rows per thread per round, all loads issued before the adds; rows
    // past the end add +0.0 (partials are sums of squares, never -0.0), so
    // the order of additions per thread is rows t, t + kBlock, ... as ever
    constexpr int RU = 4;
    for (int64_t rb = r0 + threadIdx.x; rb < r1; rb += RU * kBlock) {
      double v[RU][CB];
#pragma unroll
      for (int u = 0; u < RU; ++u) {
        const int64_t r = rb + u * kBlock;
        const int64_t rc = r < r1 ? r : r0;
#pragma unroll
        for (int c = 0; c < CB; ++c) v[u][c] = colp[c][rc];
        if (r >= r1)
#pragma unroll
          for (int c = 0; c < CB; ++c) v[u][c] = 0.0;
      }
#pragma unroll
      for (int u = 0; u < RU; ++u)
#pragma unroll
        for (int c = 0; c < CB; ++c) a[c] += v[u][c];
    }
    // wave sums (xor shuffles, fixed order), then the waves' sums in order
#pragma unroll
    for (int c = 0; c < CB; ++c) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a[c] += __shfl_xor(a[c], o, 64);
    }
    if ((threadIdx.x & 63) == 0)
#pragma unroll
      for (int c = 0; c < CB; ++c) sh[c][threadIdx.x >> 6] = a[c];
    __syncthreads();
    if (threadIdx.x < CB && cb + (int)threadIdx.x < f.ncols) {
      double r = sh[threadIdx.x][0];
#pragma unroll
      for (int w = 1; w < kBlock / 64; ++w) r += sh[threadIdx.x][w];
      sb[cb + threadIdx.x] = r;
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
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

__global__ __launch_bounds__(kBlock) void k_energy_final1(const double* __restrict__ rowpart,
                                                          int64_t nrows, int64_t rpb,
                                                          FinalizeParams f,
                                                          double* __restrict__ out) {
  const int64_t blk = blockIdx.x;
  const int64_t r0 = blk * rpb;
  const int64_t r1 = (r0 + rpb) < nrows ? (r0 + rpb) : nrows;
  finalize_rows(rowpart, nrows, r0, r1, f, out, blk);
}

// Row partial sums go either to rowpart[col][row] (blocked reductions) or,
// when the whole operand is one block (ACC), into a per-team LDS accumulator
// that each team writes once, to rowpart[col][team] (nparts = all teams).
struct PartialSink {
  double* rowpart;
  int64_t stride;  // elements per column
  bool acc;
};

// Accumulator slots per column of a workgroup: one per team, or one per wave
// for teams of several waves.
template <int TEAM>
constexpr int kSinkSlots = kBlock / (TEAM > 64 ? 64 : TEAM);

// Called by one lane per team.  Whole-operand partials go to the team's own
// slot: its index for one-wave teams, the writing lane's wave for wider ones
// (distinct per team, so teams of one workgroup never add into one slot).
template <int TEAM>
__device__ inline void sink_put(const PartialSink& k, double* lacc, int64_t row, int col,
                                double v) {
  if (k.acc) lacc[col * kSinkSlots<TEAM> + (TEAM > 64 ? threadIdx.x >> 6 : threadIdx.x / TEAM)] += v;
  else k.rowpart[(int64_t)col * k.stride + row] = v;
}

// A row's column value from every lane's share v.  Whole-operand partials of
// multi-wave teams take each wave's sum into the wave's own slot (no
// workgroup barrier per row; the flush adds the slots in order); otherwise
// the team sum goes to the sink from the team's first lane.
template <int TEAM>
__device__ inline void sink_sum(const PartialSink& k, double* lacc, double* redd, int64_t row,
                                int col, double v, bool live) {
  if constexpr (TEAM > 64) {
    if (k.acc) {
      const double w = team_sum_f64<64>(v, redd);
      if (live && (threadIdx.x & 63) == 0) lacc[col * kSinkSlots<TEAM> + (threadIdx.x >> 6)] += w;
      return;
    }
  }
  const double a = team_sum_f64<TEAM>(v, redd);
  if (live && threadIdx.x % TEAM == 0) sink_put<TEAM>(k, lacc, row, col, a);
}

// One partial per workgroup: thread c adds column c over its slots in order.
template <int TEAM>
__device__ inline void sink_flush(const PartialSink& k, double* lacc, int ncols) {
  if (!k.acc) return;
  constexpr int NS = kSinkSlots<TEAM>;
  __syncthreads();
  const int c = threadIdx.x;
  if (c < ncols) {
    double a = 0.0;
    for (int i = 0; i < NS; ++i) a += lacc[c * NS + i];
    k.rowpart[(int64_t)c * k.stride + blockIdx.x] = a;
  }
}

template <int TEAM>
__device__ inline void sink_init(double* lacc, int ncols) {
  for (int i = threadIdx.x; i < ncols * kSinkSlots<TEAM>; i += kBlock) lacc[i] = 0.0;
  __syncthreads();
}

// Empty asm that claims to modify the packed magnitudes: values derived from
// them (unpacked floats) are then rebuilt inside each quantizer loop instead
// of being hoisted out of it, which would hold 8 floats per unit in
// registers for the whole row.
#ifndef SPARQ24_E_PIN
#define SPARQ24_E_PIN 1
#endif
template <int UPL>
__device__ inline void pin_packed(uint32_t (&pk)[UPL][4]) {
#if SPARQ24_E_PIN
#pragma unroll
  for (int j = 0; j < UPL; ++j)
#pragma unroll
    for (int h = 0; h < 4; ++h) asm volatile("" : "+v"(pk[j][h]));
#endif
}

// 4096-element rows under magnitude 2:4 without rotation fit 122 VGPRs
// without spilling: four waves per SIMD keep a whole 4096-row operand
// resident in one pass.
#ifndef SPARQ24_E_WAVES
#define SPARQ24_E_WAVES 4
#endif
// INT quantizers evaluated per unpacked unit in one pass of the bf16 kernel.
// 1: chunks of 2 or 4 share each unit's unpacking but raise register use
// past four waves per SIMD (magnitude 2:4, spills) or three (Wanda), which
// costs more than the shared unpacking saves.
constexpr int kIntChunk = 1;

template <int TEAM, int UPL, int ROT, int SEL>
constexpr int kEnergyWaves = (TEAM == 64 && UPL == 8 && !ROT && SEL == SEL_MAG) ? SPARQ24_E_WAVES : 1;

template <int TEAM, int UPL, int ROT, int SEL>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kEnergyWaves<TEAM, UPL, ROT, SEL>)))
void k_energy_rows_bf16(RowGeom g, const float* __restrict__ norm, EnergyParams p,
                        PartialSink sink) {
  __shared__ uint32_t redu[kBlock / 64];
  __shared__ double redd[kBlock / 64];
  __shared__ double lacc[(2 + 2 * kMaxQ) * kSinkSlots<TEAM>];
  const int ncols = 2 + p.kept.n + p.dense.n;
  sink_init<TEAM>(lacc, ncols);
  bool any_nv = false;
  for (int q = 0; q < p.dense.n; ++q) any_nv |= (p.dense.fmt[q] == CF_NV);
  float s_t = 0.f, gnv = 0.f;
  if (any_nv) {
    const float T = block_tensor_amax(p.nv_tamax, p.nv_partials, p.n_partials, redu);
    if (T >= 0x1p-64f) { s_t = T / 2688.0f; gnv = 448.0f / T; }
  }
  bool any_knv = false;
  for (int q = 0; q < p.kept.n; ++q) any_knv |= (p.kept.fmt[q] == CF_NV);
  float ks_t = 0.f, kgnv = 0.f;
  if (any_knv) {
    const float T = block_tensor_amax(p.kept_nv_tamax, p.kept_nv_partials, p.n_kept_partials, redu);
    if (T >= 0x1p-64f) { ks_t = T / 2688.0f; kgnv = 448.0f / T; }
  }
  const int64_t nrows = g.nrows;
  for_each_row_pipelined<BF16T, TEAM, UPL, ROT>(g, [&](Unit<BF16T>(&u)[UPL], int64_t row, int t) {
    const bool live = row < nrows;
    uint32_t pk[UPL][4];   // packed |x| bf16 pairs: kept (0, 1), dropped (2, 3)
    uint32_t am = 0;       // magnitude 2:4: max top key; otherwise packed kept max
    uint32_t amd2 = 0;     // packed dropped max (Wanda, pairwise 4:8)
    double kept2 = 0.0, drop = 0.0;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      if constexpr (SEL == SEL_MAG) {
        uint32_t t0, t1;
        sel16_mags_packed(u[j].w[0], u[j].w[1], pk[j][0], pk[j][2], t0);
        sel16_mags_packed(u[j].w[2], u[j].w[3], pk[j][1], pk[j][3], t1);
        const uint32_t um = t0 > t1 ? t0 : t1;
        am = am > um ? am : um;
      } else {
        const int64_t i = (int64_t)j * TEAM + t;
        unit_mags_packed<SEL>(u[j], norm, i * 8, i < g.nunits, pk[j]);
        am = pk_max_u16(am, pk_max_u16(pk[j][0], pk[j][1]));
        amd2 = pk_max_u16(amd2, pk_max_u16(pk[j][2], pk[j][3]));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double k0 = (double)mag_lo(pk[j][h]), k1 = (double)mag_hi(pk[j][h]);
        const double d0 = (double)mag_lo(pk[j][2 + h]), d1 = (double)mag_hi(pk[j][2 + h]);
        kept2 = __builtin_fma(k0, k0, kept2);  // exact squares
        kept2 = __builtin_fma(k1, k1, kept2);
        drop = __builtin_fma(d0, d0, drop);
        drop = __builtin_fma(d1, d1, drop);
      }
    }
    // kept and row maxima as fp32 bit patterns (for magnitude 2:4 the group
    // maximum is always kept, so the kept maximum is the row maximum)
    uint32_t amk, amd;
    if constexpr (SEL == SEL_MAG) {
      amk = team_max_u32<TEAM>(am & 0xFFFF0000u, redu);
      amd = amk;
    } else {
      amk = team_max_u32<TEAM>(unpack_max16(am) << 16, redu);
      amd = team_max_u32<TEAM>(unpack_max16(pk_max_u16(am, amd2)) << 16, redu);
    }
    sink_sum<TEAM>(sink, lacc, redd, row, 0, kept2 + drop, live);
    sink_sum<TEAM>(sink, lacc, redd, row, 1, drop, live);
    const float famk = __uint_as_float(amk), famd = __uint_as_float(amd);
    // INT quantizers run in chunks of up to kIntChunk per pass over the row:
    // each unit is unpacked once for the whole chunk.  A kept one with a
    // dense twin (same format and qmax) under magnitude 2:4 is evaluated by
    // the twin, since both take their scale from the same maximum and code
    // each kept value identically: the dense pass accumulates kept and
    // dropped positions apart and writes both columns.
    // (quantizer indices are read from the kernel arguments by position:
    // a pointer into them would force a private copy of the parameters)
    auto kept_ints = [&]<int NQ>(int c0) {
      pin_packed<UPL>(pk);
      int idx[NQ];
      float s[NQ], inv[NQ];
      double acc[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        idx[i] = SEL == SEL_MAG ? p.kept_int_solo[c0 + i] : p.kept_int[c0 + i];
        row_scale(famk, p.kept.qmax[idx[i]], s[i], inv[i]);
        acc[i] = 0.0;
      }
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const float v[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
#pragma unroll
        for (int i = 0; i < NQ; ++i) acc[i] += (double)mag_sq_err_int<4>(s[i], inv[i], v);
        __builtin_amdgcn_sched_barrier(0);  // one unit's values live at a time
      }
#pragma unroll
      for (int i = 0; i < NQ; ++i) sink_sum<TEAM>(sink, lacc, redd, row, 2 + idx[i], acc[i], live);
    };
    auto dense_ints = [&]<int NQ>(int c0) {
      pin_packed<UPL>(pk);
      int idx[NQ];
      float s[NQ], inv[NQ];
      double acck[NQ], accd[NQ];
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        idx[i] = p.dense_int[c0 + i];
        row_scale(famd, p.dense.qmax[idx[i]], s[i], inv[i]);
        acck[i] = accd[i] = 0.0;
      }
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const float vk[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
        const float vd[4] = {mag_lo(pk[j][2]), mag_hi(pk[j][2]), mag_lo(pk[j][3]), mag_hi(pk[j][3])};
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          acck[i] += (double)mag_sq_err_int<4>(s[i], inv[i], vk);
          accd[i] += (double)mag_sq_err_int<4>(s[i], inv[i], vd);
        }
        __builtin_amdgcn_sched_barrier(0);  // one unit's values live at a time
      }
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        int twin = -1;
        if (SEL == SEL_MAG)
          for (int k = 0; k < p.kept.n; ++k)
            if (p.kept_twin[k] == idx[i]) twin = k;
        if (twin >= 0) sink_sum<TEAM>(sink, lacc, redd, row, 2 + twin, acck[i], live);
        sink_sum<TEAM>(sink, lacc, redd, row, 2 + p.kept.n + idx[i], acck[i] + accd[i], live);
      }
    };
    auto chunks = [&](int n, auto&& run) {
      for (int c0 = 0; c0 < n; c0 += kIntChunk) {
        const int nq = n - c0 < kIntChunk ? n - c0 : kIntChunk;
        if constexpr (kIntChunk >= 4) {
          if (nq == 4) { run.template operator()<4>(c0); continue; }
          if (nq == 3) { run.template operator()<3>(c0); continue; }
        }
        if (nq == 2) run.template operator()<2>(c0);
        else run.template operator()<1>(c0);
      }
    };
    chunks(SEL == SEL_MAG ? p.n_kept_int_solo : p.n_kept_int, kept_ints);
    chunks(p.n_dense_int, dense_ints);

    // the other formats, one pass each
    for (int q = 0; q < p.kept.n; ++q) {
      const int fmt = p.kept.fmt[q];
      if (fmt == CF_INT8 || fmt == CF_INT16) continue;  // chunked above
      if (SEL == SEL_MAG && p.kept_twin[q] >= 0) continue;
      pin_packed<UPL>(pk);
      double acc = 0.0;
      if (fmt == CF_FP8) {
        float s, inv;
        row_scale(famk, p.kept.qmax[q], s, inv);
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const float v[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
          acc += (double)mag_sq_err_fp8<4>(s, inv, v);
        }
      } else if (fmt == CF_NV) {
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const float v[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
          acc += (double)kept_block_err4<true>(v, ks_t, kgnv);
        }
      } else if (fmt == CF_MX) {
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const float v[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
          acc += (double)kept_block_err4<false>(v, 0.f, 0.f);
        }
      }
      sink_sum<TEAM>(sink, lacc, redd, row, 2 + q, acc, live);
    }
    for (int q = 0; q < p.dense.n; ++q) {
      const int fmt = p.dense.fmt[q];
      if (fmt == CF_INT8 || fmt == CF_INT16) continue;  // chunked above
      pin_packed<UPL>(pk);
      double acc = 0.0;
      if (fmt == CF_FP8) {
        int twin = -1;
        if (SEL == SEL_MAG)
          for (int k = 0; k < p.kept.n; ++k)
            if (p.kept_twin[k] == q) twin = k;
        float s, inv;
        row_scale(famd, p.dense.qmax[q], s, inv);
        double acck = 0.0;  // kept positions; acc holds the dropped ones
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const float vk[4] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1])};
          const float vd[4] = {mag_lo(pk[j][2]), mag_hi(pk[j][2]), mag_lo(pk[j][3]), mag_hi(pk[j][3])};
          acck += (double)mag_sq_err_fp8<4>(s, inv, vk);
          acc += (double)mag_sq_err_fp8<4>(s, inv, vd);
        }
        if (twin >= 0) sink_sum<TEAM>(sink, lacc, redd, row, 2 + twin, acck, live);
        acc += acck;
      } else if (fmt == CF_MX || fmt == CF_NV) {
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          // the unit's |x| max (magnitude 2:4: its kept max, as each group
          // keeps its largest)
          const uint32_t km2 = SEL == SEL_MAG ? pk_max_u16(pk[j][0], pk[j][1])
                                              : pk_max_u16(pk_max_u16(pk[j][0], pk[j][1]),
                                                           pk_max_u16(pk[j][2], pk[j][3]));
          const uint32_t kh = km2 >> 16, kl = km2 & 0xFFFFu;
          uint32_t bm = (kh > kl ? kh : kl) << 16;  // fp32 bits of the unit's |x| max
          uint32_t w = (uint32_t)__shfl_xor((int)bm, 1, 64);
          bm = bm > w ? bm : w;
          const float vj[8] = {mag_lo(pk[j][0]), mag_hi(pk[j][0]), mag_lo(pk[j][1]), mag_hi(pk[j][1]),
                               mag_lo(pk[j][2]), mag_hi(pk[j][2]), mag_lo(pk[j][3]), mag_hi(pk[j][3])};
          if (fmt == CF_MX) {
            w = (uint32_t)__shfl_xor((int)bm, 2, 64);
            bm = bm > w ? bm : w;
            acc += (double)unit_sq_err_mx8(vj, mx_exponent(bm));
          } else {
            acc += (double)unit_sq_err_nv8(vj, bm, s_t, gnv);
          }
        }
      }
      sink_sum<TEAM>(sink, lacc, redd, row, 2 + p.kept.n + q, acc, live);
    }
  });
  sink_flush<TEAM>(sink, lacc, ncols);
}

template <class DT, int TEAM, int UPL, bool WANDA, int ROT>
SPARQ24_ROW_KERNEL void k_energy_rows(RowGeom g, const float* __restrict__ norm,
                                                        EnergyParams p, PartialSink sink) {
  __shared__ uint32_t redu[kBlock / 64];
  __shared__ double redd[kBlock / 64];
  __shared__ double lacc[(2 + 2 * kMaxQ) * kSinkSlots<TEAM>];
  const int ncols0 = 2 + p.kept.n + p.dense.n;
  sink_init<TEAM>(lacc, ncols0);

  bool any_nv = false;
  for (int q = 0; q < p.dense.n; ++q) any_nv |= (p.dense.fmt[q] == CF_NV);
  float s_t = 0.f, gnv = 0.f;
  if (any_nv) {
    const float T = block_tensor_amax(p.nv_tamax, p.nv_partials, p.n_partials, redu);
    if (T >= 0x1p-64f) { s_t = T / 2688.0f; gnv = 448.0f / T; }
  }
  bool any_knv = false;
  for (int q = 0; q < p.kept.n; ++q) any_knv |= (p.kept.fmt[q] == CF_NV);
  float ks_t = 0.f, kgnv = 0.f;
  if (any_knv) {
    const float T = block_tensor_amax(p.kept_nv_tamax, p.kept_nv_partials, p.n_kept_partials, redu);
    if (T >= 0x1p-64f) { ks_t = T / 2688.0f; kgnv = 448.0f / T; }
  }
  const int64_t nrows = g.nrows;

  for_each_row_pipelined<DT, TEAM, UPL, ROT>(g, [&](Unit<DT>(&u)[UPL], int64_t row, int t) {
    const bool writer = row < nrows && t == 0;
    uint32_t km[UPL];  // 8-bit kept mask per unit
    uint32_t mbs[UPL];
    double x2 = 0.0, drop = 0.0;
    uint32_t amd = 0, amk = 0;
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = (int64_t)j * TEAM + t;
      mbs[j] = 0;
      if (p.pairs48) {
        // pairwise 4:8 (zero units select pairs 0 and 1 of zeros: harmless)
        mbs[j] = select_pairs48(u[j]);
        km[j] = pairs48_mask(mbs[j]);
      } else {
        if (i < g.nunits) mbs[j] = select_unit<DT, WANDA>(u[j], norm, i * 8);
        const uint32_t n0 = mbs[j] & 0xFu, n1 = mbs[j] >> 4;
        km[j] = (1u << (n0 & 3u)) | (1u << (n0 >> 2)) | (16u << (n1 & 3u)) | (16u << (n1 >> 2));
      }
      const uint32_t ad = unit_absmax_e(u[j]);
      amd = amd > ad ? amd : ad;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = ((km[j] >> e) & 1u) ? u[j].absbits(e) : 0u;
        amk = amk > a ? amk : a;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double dv = (double)u[j].f(e);
        x2 = __builtin_fma(dv, dv, x2);  // exact square
        const double dd = ((km[j] >> e) & 1u) ? 0.0 : dv;
        drop = __builtin_fma(dd, dd, drop);
      }
    }
    amd = team_max_u32<TEAM>(amd, redu);
    amk = team_max_u32<TEAM>(amk, redu);
    x2 = team_sum_f64<TEAM>(x2, redd);
    drop = team_sum_f64<TEAM>(drop, redd);
    if (writer) {
      sink_put<TEAM>(sink, lacc, row, 0, x2);
      sink_put<TEAM>(sink, lacc, row, 1, drop);
    }
    const float famk = DT::to_f32(amk), famd = DT::to_f32(amd);

    // kept-side quantizers: per-row scale from the kept maximum.  Every
    // quantizer here is symmetric in sign, so residuals are taken on |x|.
    for (int q = 0; q < p.kept.n; ++q) {
      const int fmt = p.kept.fmt[q];
      double acc = 0.0;
      if (fmt == CF_MX || fmt == CF_NV) {
        // kept values of a unit in position order; dropped ones are not
        // part of the compressed row
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          const Kept<DT> kp = p.pairs48 ? gather_pairs48(u[j], mbs[j]) : gather_kept(u[j], mbs[j]);
          const float v[4] = {kp.f(0), kp.f(1), kp.f(2), kp.f(3)};
          acc += (double)(fmt == CF_NV ? kept_block_err4<true>(v, ks_t, kgnv)
                                       : kept_block_err4<false>(v, 0.f, 0.f));
        }
      } else if (fmt != CF_NONE) {
        float s, inv;
        row_scale(famk, p.kept.qmax[q], s, inv);
        if (fmt == CF_FP8) {
#pragma unroll
          for (int j = 0; j < UPL; ++j) {
            const Kept<DT> kp = p.pairs48 ? gather_pairs48(u[j], mbs[j]) : gather_kept(u[j], mbs[j]);
            const float v[4] = {__builtin_fabsf(kp.f(0)), __builtin_fabsf(kp.f(1)),
                                __builtin_fabsf(kp.f(2)), __builtin_fabsf(kp.f(3))};
            acc += (double)mag_sq_err_fp8<4>(s, inv, v);
          }
        } else {
#pragma unroll
          for (int j = 0; j < UPL; ++j) {
            const Kept<DT> kp = p.pairs48 ? gather_pairs48(u[j], mbs[j]) : gather_kept(u[j], mbs[j]);
            const float v[4] = {__builtin_fabsf(kp.f(0)), __builtin_fabsf(kp.f(1)),
                                __builtin_fabsf(kp.f(2)), __builtin_fabsf(kp.f(3))};
            acc += (double)mag_sq_err_int<4>(s, inv, v);
          }
        }
      }
      acc = team_sum_f64<TEAM>(acc, redd);
      if (writer) sink_put<TEAM>(sink, lacc, row, 2 + q, acc);
    }

    // dense quantizers
    for (int q = 0; q < p.dense.n; ++q) {
      const int fmt = p.dense.fmt[q];
      double acc = 0.0;
      if (fmt == CF_INT8 || fmt == CF_INT16 || fmt == CF_FP8) {
        float s, inv;
        row_scale(famd, p.dense.qmax[q], s, inv);
        if (fmt == CF_FP8) {
#pragma unroll
          for (int j = 0; j < UPL; ++j) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = __builtin_fabsf(u[j].f(e));
            acc += (double)mag_sq_err_fp8<8>(s, inv, v);
          }
        } else {
#pragma unroll
          for (int j = 0; j < UPL; ++j) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = __builtin_fabsf(u[j].f(e));
            acc += (double)mag_sq_err_int<8>(s, inv, v);
          }
        }
      } else if (fmt == CF_MX || fmt == CF_NV) {
#pragma unroll
        for (int j = 0; j < UPL; ++j) {
          uint32_t am = __float_as_uint(DT::to_f32(unit_absmax_e(u[j])));
          uint32_t w = (uint32_t)__shfl_xor((int)am, 1, 64);
          am = am > w ? am : w;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = u[j].f(e);
          if (fmt == CF_MX) {
            w = (uint32_t)__shfl_xor((int)am, 2, 64);
            am = am > w ? am : w;
            acc += (double)unit_sq_err_mx8(v, mx_exponent(am));
          } else {
            acc += (double)unit_sq_err_nv8(v, am, s_t, gnv);
          }
        }
      }
      acc = team_sum_f64<TEAM>(acc, redd);
      if (writer) sink_put<TEAM>(sink, lacc, row, 2 + p.kept.n + q, acc);
    }
  });
  sink_flush<TEAM>(sink, lacc, ncols0);
}

// Stage 1: sum of one column over one chunk of at most kChunk rows that lies
// inside one block of rows: grid (nblk * chunks_per_block, ncols).
constexpr int64_t kChunk = 16384;

__global__ __launch_bounds__(kBlock) void k_energy_colsum(const double* __restrict__ rowpart,
                                                          int64_t nrows, int64_t rpb, int64_t cpb,
                                                          double* __restrict__ csum, int ncols) {
  __shared__ double sh[kBlock];
  const int64_t chunk = blockIdx.x;
  const int c = blockIdx.y;
  const int64_t blk = chunk / cpb, k = chunk % cpb;
  const int64_t bend = (blk + 1) * rpb < nrows ? (blk + 1) * rpb : nrows;
  const int64_t r0 = blk * rpb + k * kChunk;
  const int64_t r1 = (r0 + kChunk) < bend ? (r0 + kChunk) : bend;
  const double* col = rowpart + (int64_t)c * nrows;
  double acc = 0.0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kBlock) acc += col[r];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = kBlock / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) csum[chunk * ncols + c] = sh[0];
}

// Stage 2: per block of rows, add its chunk sums in order and form the outputs.
__global__ __launch_bounds__(kBlock) void k_energy_combine(const double* __restrict__ csum,
                                                           int64_t nblk, int64_t cpb,
                                                           FinalizeParams f,
                                                           double* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (blk >= nblk) return;
  double sb[2 + 2 * kMaxQ];
  for (int c = 0; c < f.ncols; ++c) {
    double a = 0.0;
    for (int64_t k = 0; k < cpb; ++k) a += csum[(blk * cpb + k) * f.ncols + c];
    sb[c] = a;
  }
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

// One-kernel finalize when every block of rows is a single chunk: workgroup
// b sums each column over its rows (fixed order) and forms the outputs.
hipError_t launch_energy_rows(const RowDesc& d, bool wanda, const float* norm,
                              const EnergyParams& p, double* rowpart, int64_t rows_per_block,
                              int64_t* nparts, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const RowGeom g{d.x, d.R, d.B * d.R, nunits, d.bs, d.rs, d.rot};
  const bool acc = rows_per_block >= g.nrows;  // one block: per-team partials
  if (wanda && d.rot.n) return hipErrorInvalidValue;
  auto geom = [&](int, dim3 grid, PartialSink& k) {
    k.rowpart = rowpart;
    k.acc = acc;
    k.stride = acc ? (int64_t)grid.x : g.nrows;
    *nparts = acc ? (int64_t)grid.x : g.nrows;
  };
  if (d.dtype == 1) {  // bf16: packed-magnitude kernel
    const int sel = wanda ? SEL_WANDA : (p.pairs48 ? SEL_P48 : SEL_MAG);
    // LONG: rotation blocks over 512 elements, on whole-workgroup teams
    auto body = [&]<int TEAM, int UPL, bool LONG>() {
      auto go = [&]<int R, int SEL>() {
        constexpr auto K = k_energy_rows_bf16<TEAM, UPL, R, SEL>;
        const dim3 grid = persistent_grid(g.nrows, TEAM, resident_blocks<K>());
        PartialSink k;
        geom(TEAM, grid, k);
        hipLaunchKernelGGL(K, grid, dim3(kBlock), 0, s, g, norm, p, k);
        return hipGetLastError();
      };
      if constexpr (LONG) {
        return sel == SEL_P48 ? go.template operator()<3, SEL_P48>() : go.template operator()<3, SEL_MAG>();
      } else {
        if (sel == SEL_WANDA)  // rotated calls take no norms
          return go.template operator()<0, SEL_WANDA>();
        return with_rot<TEAM>(d.rot, [&]<int R>() {
          return sel == SEL_P48 ? go.template operator()<R, SEL_P48>()
                                : go.template operator()<R, SEL_MAG>();
        });
      }
    };
    if (d.rot.n > 512)
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return body.template operator()<TEAM, UPL, true>();
      });
    return with_row_variant<SPARQ24_WIDE_E>(nunits, [&]<int TEAM, int UPL>() {
      return body.template operator()<TEAM, UPL, false>();
    });
  }
  // fp32 and fp16 operands
  auto generic = [&]<class DT>() {
    auto go = [&]<int TEAM, int UPL, bool WANDA, int R>() {
      constexpr auto K = k_energy_rows<DT, TEAM, UPL, WANDA, R>;
      const dim3 grid = persistent_grid(g.nrows, TEAM, resident_blocks<K>());
      PartialSink k;
      geom(TEAM, grid, k);
      hipLaunchKernelGGL(K, grid, dim3(kBlock), 0, s, g, norm, p, k);
      return hipGetLastError();
    };
    if (d.rot.n > 512)  // long rotation blocks: whole-workgroup teams
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return go.template operator()<TEAM, UPL, false, 3>();
      });
    return with_row_variant<SPARQ24_WIDE_EG>(nunits, [&]<int TEAM, int UPL>() {
      if (wanda) return go.template operator()<TEAM, UPL, true, 0>();  // rotated calls take no norms
      return with_rot<TEAM>(d.rot, [&]<int R>() { return go.template operator()<TEAM, UPL, false, R>(); });
    });
  };
  if (d.dtype == 0) return generic.template operator()<F32T>();
  if (d.dtype == 2) return generic.template operator()<F16T>();
  return hipErrorInvalidValue;
}

// Upper bound of the partial rows launch_energy_rows writes per column.
int64_t energy_partial_rows(int64_t nrows) { return nrows + kBlock; }

int64_t energy_chunks_per_block(int64_t rows_per_block) {
  return (rows_per_block + kChunk - 1) / kChunk;
}

hipError_t launch_energy_finalize(const double* rowpart, int64_t nrows, int64_t rows_per_block,
                                  int64_t nblk, const FinalizeParams& f, double* csum, double* out,
                                  hipStream_t s) {
  const int64_t cpb = energy_chunks_per_block(rows_per_block);
  if (cpb == 1) {
    hipLaunchKernelGGL(k_energy_final1, dim3((unsigned)nblk), dim3(kBlock), 0, s, rowpart, nrows,
                       rows_per_block, f, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_energy_colsum, dim3((unsigned)(nblk * cpb), (unsigned)f.ncols),
                     dim3(kBlock), 0, s, rowpart, nrows, rows_per_block, cpb, csum, f.ncols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_energy_combine, dim3((unsigned)((nblk + kBlock - 1) / kBlock)),
                     dim3(kBlock), 0, s, csum, nblk, cpb, f, out);
  return hipGetLastError();
}

}  // namespace sparq24
