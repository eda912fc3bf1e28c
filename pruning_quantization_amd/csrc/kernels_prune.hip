// Online 2:4 prune-and-compress and fused prune + quantize of the kept values.
//
// Method: Qin, "Is 2:4 Sparsity Still Worth It?" (paper-daily.com English
// summary).  [PD §3]: a fused online kernel reads the operand once and writes
// the kept values and their position indices once.  [PD §4]: the 2:4 side
// quantizes the kept values (here one scale per row from their absolute
// maximum).  This file holds the gfx950 kernels; they read 16-byte vectors,
// select the top two of every four with integer keys in registers, gather
// the kept pairs with byte permutes and write values, metadata and scales in
// the same pass.
#include "dispatch.hpp"

namespace sparq24 {

// Store the 4 kept raw elements of a unit (storage type) at dst.
template <class DT>
__device__ inline void store_kept(const Unit<DT>& u, uint32_t mb, char* dst) {
  const Kept<DT> kp = gather_kept(u, mb);
  if constexpr (DT::ESIZE == 2) {
    st2(dst, kp.k[0], kp.k[1]);
  } else {
    st4(dst, kp.k[0], kp.k[1], kp.k[2], kp.k[3]);
  }
}

// ---------------------------------------------------------------------------
// K-contiguous, fully contiguous operand, magnitude score: the whole tensor is
// one run of units (rows never split a unit because K % 8 == 0, and the
// outputs of unit i sit at i in both value and metadata arrays).
// Each workgroup owns UPL consecutive chunks of 256 units.
// ---------------------------------------------------------------------------
template <class DT, int UPL>
__global__ __launch_bounds__(kBlock) void k_prune_compress_flat(
    const char* __restrict__ x, int64_t nunits, char* __restrict__ vals,
    uint8_t* __restrict__ meta) {
  const int64_t base = (int64_t)blockIdx.x * (kBlock * UPL) + threadIdx.x;
  Unit<DT> u[UPL];
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int64_t i = base + (int64_t)j * kBlock;
    if (i < nunits) load_unit(u[j], x + i * (8 * DT::ESIZE));
    else zero_unit(u[j]);
  }
#pragma unroll
  for (int j = 0; j < UPL; ++j) {
    const int64_t i = base + (int64_t)j * kBlock;
    if (i < nunits) {
      const uint32_t mb = select_unit<DT, false>(u[j], nullptr, 0);
      store_kept(u[j], mb, vals + i * (4 * DT::ESIZE));
      st(meta + i, (uint8_t)mb);
    }
  }
}

// ---------------------------------------------------------------------------
// K-contiguous rows with arbitrary row/batch strides (or Wanda scores, which
// need the position along K): a team of TEAM lanes walks one row in chunks of
// TEAM * UPL units.
// ---------------------------------------------------------------------------
template <class DT, int TEAM, int UPL, bool WANDA>
__global__ __launch_bounds__(kBlock) void k_prune_compress_rows(
    const char* __restrict__ x, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    const float* __restrict__ norm, char* __restrict__ vals, uint8_t* __restrict__ meta) {
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  if (r >= R) return;  // no team-wide synchronisation in this kernel
  const char* xr = x + b * bs + r * rs;
  const int64_t orow = b * R + r;
  char* vr = vals + orow * nunits * (4 * DT::ESIZE);
  uint8_t* mr = meta + orow * nunits;
  for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
    Unit<DT> u[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
      else zero_unit(u[j]);
    }
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (i < nunits) {
        const uint32_t mb = select_unit<DT, WANDA>(u[j], norm, i * 8);
        store_kept(u[j], mb, vr + i * (4 * DT::ESIZE));
        st(mr + i, (uint8_t)mb);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wanda 2:4 of bf16 rows with K % 16 == 0 and K <= 16 * kBlock * UPP: a
// whole workgroup is the team of one row, persistent over rows (row
// blockIdx.x, then + gridDim.x, ...).  Lane t owns the unit pairs t, t +
// kBlock, ... (16 positions each): their 16 channel norms are loaded once
// and held in registers for every row, each pair leaves as one 16-byte store
// of kept values and one 2-byte metadata store, and the next row's loads are
// in flight while the current row is selected and stored (two rows ahead
// measured slower).
// ---------------------------------------------------------------------------
template <int UPP>
__global__ __launch_bounds__(kBlock) void k_prune_compress_wanda_rows(
    const char* __restrict__ x, int64_t R, int64_t nrows, int64_t npairs, int64_t bs, int64_t rs,
    const float* __restrict__ norm, char* __restrict__ vals, uint8_t* __restrict__ meta) {
  const int t = threadIdx.x;
  float n[UPP][16];
  bool ok[UPP];
#pragma unroll
  for (int q = 0; q < UPP; ++q) {
    const int64_t p = t + (int64_t)q * kBlock;
    ok[q] = p < npairs;
    const float4* np = reinterpret_cast<const float4*>(norm + (ok[q] ? p * 16 : 0));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = np[c];
      n[q][4 * c] = v.x; n[q][4 * c + 1] = v.y; n[q][4 * c + 2] = v.z; n[q][4 * c + 3] = v.w;
    }
  }
  // (batch, row) of a flattened row index, stepped on the scalar unit
  int64_t row = blockIdx.x, b = row / R, r = row % R;
  auto load = [&](int64_t bb, int64_t rr, Unit<BF16T> (&u)[UPP][2]) {
    const char* xr = x + bb * bs + rr * rs;
#pragma unroll
    for (int q = 0; q < UPP; ++q) {
      const int64_t p = ok[q] ? t + (int64_t)q * kBlock : 0;
      load_unit(u[q][0], xr + p * 32);
      load_unit(u[q][1], xr + p * 32 + 16);
    }
  };
  Unit<BF16T> cur[UPP][2], nxt[UPP][2];
  load(b, r, cur);  // the grid never exceeds the row count
  for (; row < nrows; row += gridDim.x) {
    int64_t nb = b, nr = r + gridDim.x;
    while (nr >= R) { nr -= R; ++nb; }
    if (row + gridDim.x < nrows) load(nb, nr, nxt);
#pragma unroll
    for (int q = 0; q < UPP; ++q) {
      if (!ok[q]) continue;
      const int64_t p = t + (int64_t)q * kBlock;
      const uint32_t m0 = select_unit_norms<BF16T, true>(cur[q][0], n[q]);
      const uint32_t m1 = select_unit_norms<BF16T, true>(cur[q][1], n[q] + 8);
      const Kept<BF16T> k0 = gather_kept(cur[q][0], m0), k1 = gather_kept(cur[q][1], m1);
      st4(vals + (row * npairs + p) * 16, k0.k[0], k0.k[1], k1.k[0], k1.k[1]);
      st(reinterpret_cast<uint16_t*>(meta) + row * npairs + p, (uint16_t)(m0 | (m1 << 8)));
    }
    b = nb;
    r = nr;
#pragma unroll
    for (int q = 0; q < UPP; ++q) {
      cur[q][0] = nxt[q][0];
      cur[q][1] = nxt[q][1];
    }
  }
}

// ---------------------------------------------------------------------------
// Transposed operand (row_stride == 1, the reduction axis strided), e.g. V
// [heads, seq, head_dim] pruned along seq.  A workgroup stages a tile of
// KT positions x RT rows through LDS: loads run along the contiguous row
// axis, each thread then selects within one (row, unit) column, and the
// compressed tile is written back K-contiguous per row.
// ---------------------------------------------------------------------------
constexpr int kT_KT = 128;  // positions along K per tile (16 units)
constexpr int kT_RT = 64;   // rows per tile

// Loads move 16-byte chunks of a tile line (one k, kT_RT consecutive rows);
// a chunk that crosses the last row is read element by element.  Selection
// takes two adjacent rows per item (one 2E-byte LDS read per position), and
// the compressed tile leaves in 16-byte chunks (8-byte ones when a row of
// kept values is not a multiple of 16 bytes).
template <class DT, bool WANDA>
__global__ __launch_bounds__(kBlock) void k_prune_compress_T(
    const char* __restrict__ x, int64_t R, int64_t K, int64_t bs, int64_t ks,
    const float* __restrict__ norm, char* __restrict__ vals, uint8_t* __restrict__ meta) {
  constexpr int E = DT::ESIZE;
  constexpr int CE = 16 / E;                             // elements per 16-byte chunk
  constexpr int LINE = kT_RT * E;                        // bytes of a tile line
  constexpr int LCH = LINE / 16;                         // chunks per tile line
  constexpr int UT = kT_KT / 8;                          // units per tile row
  constexpr int OUT_ROW = kT_KT / 2 * E;                 // kept bytes per row per tile
  __shared__ __align__(16) char tile[kT_KT * LINE];      // [k][r]
  __shared__ __align__(16) char otile[kT_RT * OUT_ROW];  // [r][kept bytes]
  __shared__ __align__(16) uint8_t mtile[kT_RT * UT];    // [r][unit]

  const int64_t k0 = (int64_t)blockIdx.x * kT_KT;
  const int64_t r0 = (int64_t)blockIdx.y * kT_RT;
  const int64_t b = blockIdx.z;
  const char* xb = x + b * bs;
  const int rcount = (int)((R - r0) < kT_RT ? (R - r0) : kT_RT);
  const int kcount = (int)((K - k0) < kT_KT ? (K - k0) : kT_KT);  // multiple of 8

  // 1) load
  for (int c = threadIdx.x; c < kT_KT * LCH; c += kBlock) {
    const int kk = c / LCH, r = (c % LCH) * CE;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (kk < kcount && r < rcount) {
      const char* p = xb + (k0 + kk) * ks + (r0 + r) * E;
      if (r + CE <= rcount) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        v = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        uint32_t w[4] = {0, 0, 0, 0};
        for (int i = 0; i < rcount - r; ++i) {
          const uint32_t e = E == 2 ? (uint32_t)reinterpret_cast<const uint16_t*>(p)[i]
                                    : reinterpret_cast<const uint32_t*>(p)[i];
          if constexpr (E == 2) w[i >> 1] |= e << ((i & 1) * 16);
          else w[i] = e;
        }
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    *reinterpret_cast<uint4*>(tile + kk * LINE + r * E) = v;
  }
  __syncthreads();

  // 2) select per (row pair, unit)
  for (int item = threadIdx.x; item < (kT_RT / 2) * UT; item += kBlock) {
    const int rp = item % (kT_RT / 2), uu = item / (kT_RT / 2);
    const int rr = 2 * rp;
    if (rr < rcount && uu * 8 < kcount) {
      Unit<DT> u0, u1;
#pragma unroll
      for (int i = 0; i < DT::W; ++i) u0.w[i] = u1.w[i] = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const char* q = tile + (uu * 8 + i) * LINE + rr * E;
        if constexpr (E == 2) {
          const uint32_t two = *reinterpret_cast<const uint32_t*>(q);  // rows rr, rr + 1
          u0.w[i >> 1] |= (two & 0xFFFFu) << ((i & 1) * 16);
          u1.w[i >> 1] |= (two >> 16) << ((i & 1) * 16);
        } else {
          const uint2 two = *reinterpret_cast<const uint2*>(q);
          u0.w[i] = two.x;
          u1.w[i] = two.y;
        }
      }
      const uint32_t m0 = select_unit<DT, WANDA>(u0, norm, k0 + uu * 8);
      const uint32_t m1 = select_unit<DT, WANDA>(u1, norm, k0 + uu * 8);
      const Kept<DT> p0 = gather_kept(u0, m0), p1 = gather_kept(u1, m1);
      char* o0 = otile + rr * OUT_ROW + uu * 4 * E;
      if constexpr (E == 2) {
        *reinterpret_cast<uint2*>(o0) = make_uint2(p0.k[0], p0.k[1]);
        *reinterpret_cast<uint2*>(o0 + OUT_ROW) = make_uint2(p1.k[0], p1.k[1]);
      } else {
        *reinterpret_cast<uint4*>(o0) = make_uint4(p0.k[0], p0.k[1], p0.k[2], p0.k[3]);
        *reinterpret_cast<uint4*>(o0 + OUT_ROW) = make_uint4(p1.k[0], p1.k[1], p1.k[2], p1.k[3]);
      }
      mtile[rr * UT + uu] = (uint8_t)m0;
      mtile[(rr + 1) * UT + uu] = (uint8_t)m1;  // row rr + 1 past rcount is never written out
    }
  }
  __syncthreads();

  // 3) write: per row, kcount/2 kept elements and kcount/8 metadata bytes
  const int obytes = kcount / 2 * E;
  const int64_t vrow = K / 2 * E;  // bytes per output row of kept values
  if (vrow % 16 == 0) {
    const int nch = obytes / 16;   // obytes is a multiple of 16 here unless K's tail is short
    const int tail = obytes % 16;  // 0 or 8
    for (int item = threadIdx.x; item < kT_RT * (OUT_ROW / 16); item += kBlock) {
      const int rr = item / (OUT_ROW / 16), c = item % (OUT_ROW / 16);
      if (rr < rcount) {
        char* dst = vals + (b * R + r0 + rr) * vrow + k0 / 2 * E + c * 16;
        const char* src = otile + rr * OUT_ROW + c * 16;
        if (c < nch) {
          const uint4 v = *reinterpret_cast<const uint4*>(src);
          st4(dst, v.x, v.y, v.z, v.w);
        } else if (c == nch && tail) {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          st2(dst, v.x, v.y);
        }
      }
    }
  } else {
    for (int item = threadIdx.x; item < kT_RT * (OUT_ROW / 8); item += kBlock) {
      const int rr = item / (OUT_ROW / 8), c = item % (OUT_ROW / 8);
      if (rr < rcount && c < obytes / 8) {
        char* dst = vals + (b * R + r0 + rr) * vrow + k0 / 2 * E + c * 8;
        const uint2 v = *reinterpret_cast<const uint2*>(otile + rr * OUT_ROW + c * 8);
        st2(dst, v.x, v.y);
      }
    }
  }
  const int mbytes = kcount / 8;
  if ((K / 8) % 16 == 0 && mbytes == UT) {  // whole 16-byte metadata chunks
    for (int rr = threadIdx.x; rr < rcount; rr += kBlock) {
      const uint4 v = *reinterpret_cast<const uint4*>(mtile + rr * UT);
      st4(meta + (b * R + r0 + rr) * (K / 8) + k0 / 8, v.x, v.y, v.z, v.w);
    }
  } else {
    for (int item = threadIdx.x; item < kT_RT * UT; item += kBlock) {
      const int rr = item / UT, uu = item % UT;
      if (rr < rcount && uu < mbytes)
        meta[(b * R + r0 + rr) * (K / 8) + k0 / 8 + uu] = mtile[rr * UT + uu];
    }
  }
}

// Transposed 16-bit operand, magnitude score, R % 64 == 0 and K % 256 == 0
// (e.g. V [heads, seq, 128] pruned along seq): no LDS staging of the input.
// A tile is 256 positions x 64 rows; each workgroup walks kT8_Tiles tiles
// (tile index strided by the grid) with the next tile's loads in flight
// while it selects and stores the current one.  In a tile thread t owns the
// 8 x 8 block of rows 8 * (t % 8) .. + 7 and positions 8 * ((t / 8) % 16)
// .. + 7 of its 128-position half (t / 128): it loads one 16-byte chunk (8
// adjacent rows) per position, so each wave load instruction reads 8 whole
// 128-byte lines.  The block is transposed in registers with byte permutes
// (one per output dword) and each row's unit is selected through the LDS
// table.  Kept pairs and metadata bytes go through double-buffered LDS tiles
// (one barrier per tile) and leave in 16-byte chunks: a wave stores four
// whole 256-byte rows of kept values, metadata as 32-byte row segments.
constexpr int kT8_K = 256;     // positions per tile
constexpr int kT8_R = 64;      // rows per tile
constexpr int kT8_Tiles = 2;   // tiles per workgroup (grid = ceil(tiles / kT8_Tiles))

template <class DT>
__global__ __launch_bounds__(kBlock) void k_prune_compress_T8(
    const char* __restrict__ x, int64_t R, int64_t K, int64_t bs, int64_t ks,
    char* __restrict__ vals, uint8_t* __restrict__ meta, int64_t ntiles) {
  static_assert(DT::ESIZE == 2, "16-bit storage types");
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __shared__ SelLut lut[kSelLutEntries];
  __shared__ __align__(16) uint8_t mtile[2][kT8_R][kT8_K / 8];  // [buffer][row][unit]
  __shared__ __align__(16) char ktile[2][kT8_R][kT8_K];         // [buffer][row][kept bytes]
  const int t = threadIdx.x;
  const int rg = t & 7, pg = (t >> 3) & 15, half = t >> 7;
  const int64_t ntk = K / kT8_K, ntr = R / kT8_R;
  // tile -> (batch, row tile, position tile); first position and row of this thread
  auto origin = [&](int64_t tile, int64_t& b, int64_t& r0, int64_t& k0) {
    const int64_t kt = tile % ntk, q = tile / ntk;
    b = q / ntr;
    r0 = (q % ntr) * kT8_R + rg * 8;
    k0 = kt * kT8_K + half * 128 + pg * 8;
  };
  auto load = [&](int64_t tile, u32x4 (&c)[8]) {
    int64_t b, r0, k0;
    origin(tile, b, r0, k0);
    const char* src = x + b * bs + k0 * ks + r0 * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      c[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + i * ks));
  };
  u32x4 cur[8], nxt[8];
  int64_t tile = blockIdx.x;
  load(tile, cur);  // the grid never exceeds the tile count
  sel_lut_fill(lut);
  __syncthreads();
  for (int buf = 0; tile < ntiles; tile += gridDim.x, buf ^= 1) {
    const int64_t next = tile + gridDim.x;
    if (next < ntiles) load(next, nxt);
    const int ucol = half * 16 + pg;  // unit column within the tile
#pragma unroll
    for (int d = 0; d < 8; ++d) {  // row r0 + d: dword d / 2 of each chunk, half d % 2
      const uint32_t sel = (d & 1) ? 0x07060302u : 0x05040100u;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)  // positions 2q, 2q + 1
        w[q] = __builtin_amdgcn_perm(cur[2 * q + 1][d >> 1], cur[2 * q][d >> 1], sel);
      const Sel16 r = select16_lut(w, lut);
      *reinterpret_cast<uint2*>(&ktile[buf][rg * 8 + d][(half * 64 + pg * 4) * 2]) =
          make_uint2(r.k0, r.k1);
      mtile[buf][rg * 8 + d][ucol] = (uint8_t)r.mb;
    }
    __syncthreads();
    const int64_t qt = tile / ntk, kt = tile % ntk;
    const int64_t orow0 = (qt / ntr) * R + (qt % ntr) * kT8_R;  // the tile's first output row
#pragma unroll
    for (int i = 0; i < kT8_R * kT8_K / 16 / kBlock; ++i) {
      // 64 rows x 256 bytes of kept values in 16-byte chunks: a wave stores
      // four whole rows of the tile (whole 128-byte lines)
      const int c = t + kBlock * i, row = c >> 4, part = c & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(&ktile[buf][row][part * 16]);
      st4(vals + (orow0 + row) * K + kt * kT8_K + part * 16, v.x, v.y, v.z, v.w);
    }
    if (t < kT8_R * 2) {  // 64 rows x 32 metadata bytes, in 16-byte chunks
      const int row = t >> 1, part = t & 1;
      const uint4 v = *reinterpret_cast<const uint4*>(&mtile[buf][row][part * 16]);
      st4(meta + (orow0 + row) * (K / 8) + kt * (kT8_K / 8) + part * 16, v.x, v.y, v.z, v.w);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) cur[i] = nxt[i];
  }
}

// ---------------------------------------------------------------------------
// Fused prune + compress + quantize of the kept values, one scale per row.
// A team holds its whole row in registers: one read, then the kept absolute
// maximum (team reduction), then codes, metadata and the scale are written.
// The grid covers every row (one row per team): at 16384 x 4096 this measured
// 3.5% faster than persistent teams walking several rows.  CF (the code
// format) is a template parameter so each variant is straight-line code.
// ---------------------------------------------------------------------------
template <int CF>
__device__ inline void store_kept_codes(char* dst, const float* y, float qmax) {
  if constexpr (CF == CF_FP8) {
    st(reinterpret_cast<uint32_t*>(dst), enc_e4m3_x4(y[0], y[1], y[2], y[3]));
  } else {
    uint32_t r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __float_as_uint(int_round_magic(y[e], qmax));
    if constexpr (CF == CF_INT8) {
      const uint32_t lo = __builtin_amdgcn_perm(r[1], r[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm(r[3], r[2], 0x0c0c0400u);
      st(reinterpret_cast<uint32_t*>(dst), __builtin_amdgcn_perm(hi, lo, 0x05040100u));
    } else {
      st2(dst, __builtin_amdgcn_perm(r[1], r[0], 0x05040100u),
          __builtin_amdgcn_perm(r[3], r[2], 0x05040100u));
    }
  }
}

template <class DT, int TEAM, int UPL, bool WANDA, int CF, int PAT, int ROT>
SPARQ24_ROW_KERNEL void k_prune_quantize(RowGeom g, const float* __restrict__ norm, float qmax,
                                         char* __restrict__ codes, uint8_t* __restrict__ meta,
                                         float* __restrict__ scales) {
  __shared__ uint32_t red[kBlock / 64];
  constexpr int CB = CF == CF_INT16 ? 8 : 4;  // code bytes per unit
  // 16-bit magnitude 2:4: every unit is selected first and only its kept
  // pairs and metadata byte stay in registers.  The group's top key from the
  // top-2 network carries the group's |max| in its high half, and every group
  // keeps its largest element, so the row maximum of the top keys is the
  // kept maximum that sets the scale (no separate max pass; 1.5% faster at
  // 16384 x 4096).  Pairwise 4:8 can drop a row's largest element, so it
  // takes the kept maximum of the gathered values like Wanda.
  constexpr bool FAST16 = DT::ESIZE == 2 && !WANDA && PAT == PAT_24;
  __shared__ SelLut lut[FAST16 ? kSelLutEntries : 1];
  // the table is filled while the first row's loads are in flight
  auto pre = [&] {
    if constexpr (FAST16) {
      sel_lut_fill(lut);
      __syncthreads();
    }
  };
  for_each_row<DT, TEAM, UPL, ROT>(g, pre, [&](Unit<DT>(&u)[UPL], int64_t row, int t) {
    const bool active = row < g.nrows;
    uint32_t am = 0;
    uint32_t mb[UPL];
    uint32_t sk[FAST16 ? UPL : 1][2];      // kept pairs of each unit (16-bit magnitude 2:4)
    uint32_t mo[PAT == PAT_48 ? UPL : 1];  // neighbouring unit's nibble (4:8 meta bytes)
    if constexpr (FAST16) {
      uint32_t top = 0;
#pragma unroll
      for (int j = 0; j < UPL; ++j) {  // zero units select zeros
        const Sel16 r = select16_lut(u[j].w, lut);
        sk[j][0] = r.k0;
        sk[j][1] = r.k1;
        mb[j] = r.mb;
        top = top > r.topkey ? top : r.topkey;
      }
      am = top >> 16;
    } else {
#pragma unroll
      for (int j = 0; j < UPL; ++j) {
        const int64_t i = (int64_t)j * TEAM + t;
        uint32_t a;
        if constexpr (PAT == PAT_48) {
          mb[j] = select_pairs48(u[j]);  // zero units select zeros
          mo[j] = (uint32_t)__shfl_xor((int)mb[j], 1, 64);
          a = kept_absmax(gather_pairs48(u[j], mb[j]));
        } else {
          mb[j] = 0;
          if (i < g.nunits) mb[j] = select_unit<DT, WANDA>(u[j], norm, i * 8);
          a = kept_absmax(gather_kept(u[j], mb[j]));  // zero units gather zeros
        }
        am = am > a ? am : a;
      }
    }
    am = team_max_u32<TEAM>(am, red);
    if (!active) return;
    float s, inv;
    row_scale(DT::to_f32(am), qmax, s, inv);
    // per-row output bases; unit j of this lane sits at a constant offset
    char* crow = codes + (row * g.nunits + t) * CB;
    uint8_t* mrow = PAT == PAT_48 ? meta + row * (g.nunits / 2) + (t >> 1) : meta + row * g.nunits + t;
    auto emit = [&](int j) {
      Kept<DT> kp;
      uint32_t m;
      if constexpr (FAST16) {
        kp.k[0] = sk[j][0];
        kp.k[1] = sk[j][1];
        m = mb[j];
      } else if constexpr (PAT == PAT_48) {
        kp = gather_pairs48(u[j], mb[j]);
        m = mb[j];
      } else {
        kp = gather_kept(u[j], mb[j]);
        m = mb[j];
      }
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = kp.f(e) * inv;
      store_kept_codes<CF>(crow + j * TEAM * CB, y, qmax);
      if constexpr (PAT == PAT_48) {
        if ((t & 1) == 0) st(mrow + j * (TEAM / 2), (uint8_t)(m | (mo[j] << 4)));
      } else {
        st(mrow + j * TEAM, (uint8_t)m);
      }
    };
    if ((UPL - 1) * TEAM + t < g.nunits) {  // every unit of this lane exists
#pragma unroll
      for (int j = 0; j < UPL; ++j) emit(j);
    } else {
#pragma unroll
      for (int j = 0; j < UPL; ++j)
        if (j * TEAM + t < g.nunits) emit(j);
    }
    if (t == 0) scales[row] = s;
  });
}

// ---------------------------------------------------------------------------
// Pairwise 4:8 prune-and-compress [PD §6].  Same team walk as the 2:4 row
// kernel; one unit is one group of eight, whose nibble (p0 | p1 << 2) is
// paired with the neighbouring lane's (units 2m and 2m+1) into one byte.
// ---------------------------------------------------------------------------
template <class DT, int TEAM, int UPL>
__global__ __launch_bounds__(kBlock) void k_prune_compress_pairs48(
    const char* __restrict__ x, int64_t R, int64_t nunits, int64_t bs, int64_t rs,
    char* __restrict__ vals, uint8_t* __restrict__ meta) {
  const int t = threadIdx.x % TEAM;
  const int64_t r = (int64_t)blockIdx.x * (kBlock / TEAM) + threadIdx.x / TEAM;
  const int64_t b = blockIdx.y;
  const bool active = r < R;  // lanes of absent rows stay for the shuffles
  const char* xr = x + b * bs + (active ? r : 0) * rs;
  const int64_t orow = b * R + r;
  char* vr = vals + orow * nunits * (4 * DT::ESIZE);
  uint8_t* mr = meta + orow * (nunits / 2);
  for (int64_t c0 = 0; c0 < nunits; c0 += TEAM * UPL) {
    Unit<DT> u[UPL];
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      if (active && i < nunits) load_unit(u[j], xr + i * (8 * DT::ESIZE));
      else zero_unit(u[j]);
    }
#pragma unroll
    for (int j = 0; j < UPL; ++j) {
      const int64_t i = c0 + j * TEAM + t;
      const uint32_t nib = select_pairs48(u[j]);
      const uint32_t other = (uint32_t)__shfl_xor((int)nib, 1, 64);
      if (active && i < nunits) {
        const Kept<DT> kp = gather_pairs48(u[j], nib);
        if constexpr (DT::ESIZE == 2) st2(vr + i * 8, kp.k[0], kp.k[1]);
        else st4(vr + i * 16, kp.k[0], kp.k[1], kp.k[2], kp.k[3]);
        if ((i & 1) == 0) st(mr + (i >> 1), (uint8_t)(nib | (other << 4)));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_prune_compress(const RowDesc& d, bool wanda, const float* norm, void* vals,
                                 uint8_t* meta, hipStream_t s) {
  const int64_t nunits = d.K / 8;
  if (!d.kcontig) {
    if (!wanda && d.dtype != 0 && d.R % kT8_R == 0 && d.K % kT8_K == 0) {
      const int64_t ntiles = (d.K / kT8_K) * (d.R / kT8_R) * d.B;
      const dim3 grid((unsigned)((ntiles + kT8_Tiles - 1) / kT8_Tiles));
      if (d.dtype == 1)
        hipLaunchKernelGGL((k_prune_compress_T8<BF16T>), grid, dim3(kBlock), 0, s, d.x, d.R, d.K,
                           d.bs, d.ks, (char*)vals, meta, ntiles);
      else
        hipLaunchKernelGGL((k_prune_compress_T8<F16T>), grid, dim3(kBlock), 0, s, d.x, d.R, d.K,
                           d.bs, d.ks, (char*)vals, meta, ntiles);
      return hipGetLastError();
    }
    return with_dtype(d.dtype, [&]<class DT>() {
      dim3 grid((unsigned)((d.K + kT_KT - 1) / kT_KT), (unsigned)((d.R + kT_RT - 1) / kT_RT),
                (unsigned)d.B);
      if (wanda)
        hipLaunchKernelGGL((k_prune_compress_T<DT, true>), grid, dim3(kBlock), 0, s, d.x, d.R,
                           d.K, d.bs, d.ks, norm, (char*)vals, meta);
      else
        hipLaunchKernelGGL((k_prune_compress_T<DT, false>), grid, dim3(kBlock), 0, s, d.x, d.R,
                           d.K, d.bs, d.ks, norm, (char*)vals, meta);
      return hipGetLastError();
    });
  }
  if (d.flat && !wanda) {
    return with_dtype(d.dtype, [&]<class DT>() {
      constexpr int UPL = 4;
      const int64_t total = d.B * d.R * nunits;
      const int64_t nblk = (total + kBlock * UPL - 1) / (kBlock * UPL);
      hipLaunchKernelGGL((k_prune_compress_flat<DT, UPL>), dim3((unsigned)nblk), dim3(kBlock), 0,
                         s, d.x, total, (char*)vals, meta);
      return hipGetLastError();
    });
  }
  if (wanda && d.dtype == 1 && d.K % 16 == 0 && d.K <= 32 * kBlock) {
    // bf16 Wanda rows: persistent whole-workgroup teams with the norms in registers
    auto go = [&]<int UPP>() {
      constexpr auto Kn = k_prune_compress_wanda_rows<UPP>;
      const int64_t nrows = d.B * d.R;
      const int64_t cap = (int64_t)device_cu_count() * resident_blocks<Kn>();
      const int64_t grid = nrows < cap ? nrows : cap;
      hipLaunchKernelGGL(Kn, dim3((unsigned)grid), dim3(kBlock), 0, s, d.x, d.R, nrows,
                         d.K / 16, d.bs, d.rs, norm, (char*)vals, meta);
      return hipGetLastError();
    };
    return d.K <= 16 * kBlock ? go.template operator()<1>() : go.template operator()<2>();
  }
  return with_dtype(d.dtype, [&]<class DT>() {
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      if (wanda)
        hipLaunchKernelGGL((k_prune_compress_rows<DT, TEAM, UPL, true>), row_grid(d, TEAM),
                           dim3(kBlock), 0, s, d.x, d.R, nunits, d.bs, d.rs, norm, (char*)vals,
                           meta);
      else
        hipLaunchKernelGGL((k_prune_compress_rows<DT, TEAM, UPL, false>), row_grid(d, TEAM),
                           dim3(kBlock), 0, s, d.x, d.R, nunits, d.bs, d.rs, norm, (char*)vals,
                           meta);
      return hipGetLastError();
    });
  });
}

hipError_t launch_prune_compress_pairs48(const RowDesc& d, void* vals, uint8_t* meta,
                                        hipStream_t s) {
  const int64_t nunits = d.K / 8;
  return with_dtype(d.dtype, [&]<class DT>() {
    return with_loop_variant(nunits, [&]<int TEAM, int UPL>() {
      hipLaunchKernelGGL((k_prune_compress_pairs48<DT, TEAM, UPL>), row_grid(d, TEAM), dim3(kBlock),
                         0, s, d.x, d.R, nunits, d.bs, d.rs, (char*)vals, meta);
      return hipGetLastError();
    });
  });
}

hipError_t launch_prune_quantize(const RowDesc& d, int pat, bool wanda, const float* norm,
                                 int cfmt, float qmax, void* codes, uint8_t* meta, float* scales,
                                 hipStream_t s) {
  const int64_t nunits = d.K / 8;
  const RowGeom g{d.x, d.R, d.B * d.R, nunits, d.bs, d.rs, d.rot};
  if (wanda && d.rot.n) return hipErrorInvalidValue;  // rotated calls take no norms
  return with_dtype(d.dtype, [&]<class DT>() {
    // LONG: rotation blocks over 512 elements, on whole-workgroup teams
    auto body = [&]<int TEAM, int UPL, bool LONG>() -> hipError_t {
      auto go = [&]<bool W, int P, int CF, int R>() {
        hipLaunchKernelGGL((k_prune_quantize<DT, TEAM, UPL, W, CF, P, R>), stream_grid(g.nrows, TEAM),
                           dim3(kBlock), 0, s, g, norm, qmax, (char*)codes, meta, scales);
        return hipGetLastError();
      };
      auto fmt = [&]<bool W, int P, int R>() {
        if (cfmt == CF_FP8) return go.template operator()<W, P, CF_FP8, R>();
        if (cfmt == CF_INT8) return go.template operator()<W, P, CF_INT8, R>();
        return go.template operator()<W, P, CF_INT16, R>();
      };
      if constexpr (LONG) {
        return pat == PAT_48 ? fmt.template operator()<false, PAT_48, 3>()
                             : fmt.template operator()<false, PAT_24, 3>();
      } else {
        if (wanda) return fmt.template operator()<true, PAT_24, 0>();
        if (pat == PAT_48)
          return d.rot.n ? fmt.template operator()<false, PAT_48, 1>()
                         : fmt.template operator()<false, PAT_48, 0>();
        return d.rot.n ? fmt.template operator()<false, PAT_24, 1>()
                       : fmt.template operator()<false, PAT_24, 0>();
      }
    };
    if (d.rot.n > 512)
      return with_long_rot_variant(nunits, [&]<int TEAM, int UPL>() {
        return body.template operator()<TEAM, UPL, true>();
      });
    return with_row_variant<1>(nunits, [&]<int TEAM, int UPL>() {
      return body.template operator()<TEAM, UPL, false>();
    });
  });
}

}  // namespace sparq24
