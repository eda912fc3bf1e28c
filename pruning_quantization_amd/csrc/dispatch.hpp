// Compile-time variant dispatch for the row kernels.
#pragma once

#include <hip/hip_runtime.h>
#include "device_common.hpp"
#include "launch.hpp"

namespace sparq24 {

// Storage-type dispatch: f.template operator()<DT>().
template <class F>
inline hipError_t with_dtype(int dtype, F&& f) {
  switch (dtype) {
    case 0: return f.template operator()<F32T>();
    case 1: return f.template operator()<BF16T>();
    case 2: return f.template operator()<F16T>();
    default: return hipErrorInvalidValue;
  }
}

// Team shape for kernels that keep a whole row in registers: the smallest
// (TEAM lanes, UPL units per lane) with TEAM * UPL >= units of the row.
// WIDE = 1 uses two-wave teams (TEAM 128) for rows of 2049..4096 elements:
// half the per-wave arithmetic at the end of a row, which measured faster for
// the quantizers (and for the fp32 / fp16 energy kernel, whose one-wave form
// spills); the bf16 energy kernel, with many more team reductions, keeps
// one-wave teams.
template <int WIDE, class F>
inline hipError_t with_row_variant(int64_t nunits, F&& f) {
  if (nunits <= 16) return f.template operator()<16, 1>();
  if (nunits <= 32) return f.template operator()<32, 1>();
  if (nunits <= 64) return f.template operator()<64, 1>();
  if (nunits <= 128) return f.template operator()<64, 2>();
  if (nunits <= 256) return f.template operator()<64, 4>();
  if (nunits <= 512) {
    if constexpr (WIDE == 1) return f.template operator()<128, 4>();
    else return f.template operator()<64, 8>();
  }
  if (nunits <= 1024) return f.template operator()<64, 16>();
  if (nunits <= 2048) return f.template operator()<256, 8>();
  if (nunits <= 4096) return f.template operator()<256, 16>();
  return hipErrorInvalidValue;
}

// Team shape for kernels that stream a row in chunks (no whole-row state).
template <class F>
inline hipError_t with_loop_variant(int64_t nunits, F&& f) {
  if (nunits <= 16) return f.template operator()<16, 1>();
  if (nunits <= 32) return f.template operator()<32, 1>();
  if (nunits <= 64) return f.template operator()<64, 1>();
  if (nunits <= 128) return f.template operator()<64, 2>();
  if (nunits <= 256) return f.template operator()<64, 4>();
  return f.template operator()<64, 8>();
}

// Rotation variant of a launch on teams of TEAM lanes: 0 none, 1 blocks of
// up to 512 elements (unit by unit).  Longer blocks are launched as variant 3
// on the teams of with_long_rot_variant.
template <int TEAM, class F>
inline hipError_t with_rot(const Rot& r, F&& f) {
  if (r.n == 0) return f.template operator()<0>();
  if (r.n <= 512) return f.template operator()<1>();
  return hipErrorInvalidValue;
}

// Team shape for rotation blocks of 1024 .. 4096 elements on whole-workgroup
// teams (rotation variant 3): UPL registers of kBlock units per lane (rows of
// up to 8192 elements, the limit the ABI sets for such blocks).
template <class F>
inline hipError_t with_long_rot_variant(int64_t nunits, F&& f) {
  if (nunits <= kBlock) return f.template operator()<kBlock, 1>();
  if (nunits <= 2 * kBlock) return f.template operator()<kBlock, 2>();
  if (nunits <= 4 * kBlock) return f.template operator()<kBlock, 4>();
  return hipErrorInvalidValue;
}

inline dim3 row_grid(const RowDesc& d, int team) {
  const int64_t rpb = kBlock / team;
  return dim3((unsigned)((d.R + rpb - 1) / rpb), (unsigned)d.B, 1);
}

// Grid of a streaming row kernel: one team per row.  New workgroups start as
// old ones retire, so loads of fresh rows overlap the arithmetic of others.
inline dim3 stream_grid(int64_t nrows, int team) {
  const int64_t rpb = kBlock / team;
  const int64_t need = (nrows + rpb - 1) / rpb;
  return dim3((unsigned)(need > 0 ? need : 1));
}

// Grid of a persistent row kernel (the VALU-bound energy kernels): enough
// workgroups to fill every CU kBlocksPerCU times (at most one team per row).
constexpr int kBlocksPerCU = 4;
int device_cu_count();

// Workgroups of kernel K resident per CU (register and LDS limits) with
// `shmem` bytes of dynamic LDS, from the runtime's occupancy calculator:
// queried once per kernel without dynamic LDS, per launch with it.
template <auto K>
inline int occupancy_query(size_t shmem) {
  int b = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, reinterpret_cast<const void*>(K), kBlock,
                                                   shmem) != hipSuccess ||
      b < 1) {
    (void)hipGetLastError();
    b = shmem ? 1 : kBlocksPerCU;
  }
  return b;
}
template <auto K>
inline int resident_blocks(size_t shmem = 0) {
  if (shmem) return occupancy_query<K>(shmem);
  static const int n = occupancy_query<K>(0);
  return n;
}

// resident: workgroups of the kernel that fit on a CU at once.  A kernel
// whose registers allow fewer than kBlocksPerCU gets only as many, so the
// whole grid is resident and no second round of workgroups trails the first.
inline dim3 persistent_grid(int64_t nrows, int team, int resident = kBlocksPerCU) {
  const int64_t rpb = kBlock / team;
  const int64_t need = (nrows + rpb - 1) / rpb;
  const int per_cu = resident < kBlocksPerCU ? resident : kBlocksPerCU;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  const int64_t n = need < cap ? need : cap;
  return dim3((unsigned)(n > 0 ? n : 1));
}

}  // namespace sparq24
