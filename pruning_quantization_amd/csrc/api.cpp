// C-ABI entry points of libsparq24: argument validation (pure host code, run
// before any HIP call), variant selection, workspace sizing and launches on
// the caller's stream.  The operations are those of Qin, "Is 2:4 Sparsity
// Still Worth It?" (paper-daily.com English summary, sections 2-4); see
// include/sparq24.h for the contract of each call.
#include "sparq24.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <atomic>

#include "launch.hpp"

using namespace sparq24;

// Workspace of sparq24_predict_R_noalloc (see scratch_address below).
static __device__ __align__(256) char scratch[SPARQ24_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int esize(int dtype) { return dtype == SPARQ24_F32 ? 4 : 2; }

// Structural checks of an operand; fills the kernel view (strides in bytes,
// back-to-back batches folded into rows).
sparq24_status check_tensor(const sparq24_tensor* x, bool allow_transposed, RowDesc& d) {
  if (!x) return SPARQ24_ERR_INVALID;
  if (x->dtype != SPARQ24_F32 && x->dtype != SPARQ24_BF16 && x->dtype != SPARQ24_F16)
    return SPARQ24_ERR_INVALID;
  if (x->batch < 0 || x->rows < 0 || x->k < 0) return SPARQ24_ERR_INVALID;
  if (x->batch_stride < 0 || x->row_stride < 0 || x->k_stride < 0) return SPARQ24_ERR_INVALID;
  if (x->k % 8 != 0) return SPARQ24_ERR_SHAPE;
  const int es = esize(x->dtype);
  d.x = (const char*)x->data;
  d.dtype = x->dtype;
  d.rot.n = 0;
  d.rot.c = 0.0;
  d.B = x->batch;
  d.R = x->rows;
  d.K = x->k;
  if (d.B * d.R * d.K == 0) {  // empty: nothing to read
    d.kcontig = true;
    d.flat = true;
    d.bs = d.rs = d.ks = 0;
    return SPARQ24_OK;
  }
  if (!x->data) return SPARQ24_ERR_INVALID;
  if (!aligned16(x->data)) return SPARQ24_ERR_ALIGN;
  if (x->k_stride == 1 || x->k == 1) {
    d.kcontig = true;
    if (d.R > 1 && x->row_stride < d.K) return SPARQ24_ERR_UNSUPPORTED;
    if (d.B > 1 && x->batch_stride < (d.R - 1) * x->row_stride + d.K) return SPARQ24_ERR_UNSUPPORTED;
    if (d.R > 1 && (x->row_stride * es) % 16) return SPARQ24_ERR_ALIGN;
    if (d.B > 1 && (x->batch_stride * es) % 16) return SPARQ24_ERR_ALIGN;
    int64_t rs = d.R > 1 ? x->row_stride : d.K;
    int64_t bs = d.B > 1 ? x->batch_stride : d.R * rs;
    if (d.B > 1 && bs == d.R * rs) {  // batches back to back: fold into rows
      d.R *= d.B;
      d.B = 1;
      bs = d.R * rs;
    }
    d.rs = rs * es;
    d.bs = bs * es;
    d.ks = es;
    d.flat = (rs == d.K) && d.B == 1;
  } else if (x->row_stride == 1 || d.R == 1) {
    if (!allow_transposed) return SPARQ24_ERR_UNSUPPORTED;
    if (x->k_stride < d.R) return SPARQ24_ERR_UNSUPPORTED;
    if (d.B > 1 && x->batch_stride < (d.K - 1) * x->k_stride + d.R) return SPARQ24_ERR_UNSUPPORTED;
    if ((x->k_stride * es) % 16) return SPARQ24_ERR_ALIGN;
    if (d.B > 1 && (x->batch_stride * es) % 16) return SPARQ24_ERR_ALIGN;
    // the transposed kernels tile rows by 64 on grid.y (at most 65535 tiles)
    if ((d.R + 63) / 64 > 65535) return SPARQ24_ERR_UNSUPPORTED;
    d.kcontig = false;
    d.flat = false;
    d.rs = es;
    d.ks = x->k_stride * es;
    d.bs = (d.B > 1 ? x->batch_stride : d.K * x->k_stride) * es;
  } else {
    return SPARQ24_ERR_UNSUPPORTED;
  }
  if (d.B > 65535) return SPARQ24_ERR_UNSUPPORTED;
  return SPARQ24_OK;
}

sparq24_status check_score(int32_t score, const float* col_norm) {
  if (score != SPARQ24_SCORE_MAGNITUDE && score != SPARQ24_SCORE_WANDA) return SPARQ24_ERR_INVALID;
  if (score == SPARQ24_SCORE_WANDA) {
    if (!col_norm) return SPARQ24_ERR_INVALID;
    if (!aligned16(col_norm)) return SPARQ24_ERR_ALIGN;
  }
  return SPARQ24_OK;
}

// Hadamard block size: a power of two in 8..4096 dividing K (blocks over 512
// elements need K <= 8192, where one wave holds a row); fills d.rot with
// c = fp64 1/sqrt(n) (an exact power of two for even log2 n, else that power
// times the correctly rounded sqrt(1/2)).
sparq24_status check_rot(int32_t block, RowDesc& d) {
  if (block < 8 || block > 4096 || (block & (block - 1))) return SPARQ24_ERR_INVALID;
  if (d.K % block) return SPARQ24_ERR_SHAPE;
  if (block > 512 && d.K > 8192) return SPARQ24_ERR_UNSUPPORTED;
  int k = 0;
  while ((1 << k) < block) ++k;
  d.rot.n = block;
  d.rot.c = ldexp((k & 1) ? sqrt(0.5) : 1.0, -(k / 2));
  return SPARQ24_OK;
}

// Quantizer spec -> code container and qmax.  `allowed` is a bit set of
// sparq24_qfmt values the call accepts.
sparq24_status check_q(const sparq24_qspec* q, unsigned allowed, int& cfmt, float& qmax) {
  if (!q) return SPARQ24_ERR_INVALID;
  if (q->fmt < SPARQ24_Q_NONE || q->fmt > SPARQ24_Q_NVFP4) return SPARQ24_ERR_INVALID;
  if (!(allowed & (1u << q->fmt))) return SPARQ24_ERR_UNSUPPORTED;
  switch (q->fmt) {
    case SPARQ24_Q_NONE: cfmt = CF_NONE; qmax = 0.f; break;
    case SPARQ24_Q_INT:
      if (q->bits < 2 || q->bits > 16) return SPARQ24_ERR_UNSUPPORTED;
      cfmt = q->bits <= 8 ? CF_INT8 : CF_INT16;
      qmax = (float)((1 << (q->bits - 1)) - 1);
      break;
    case SPARQ24_Q_FP8_E4M3: cfmt = CF_FP8; qmax = 448.f; break;
    case SPARQ24_Q_MXFP4: cfmt = CF_MX; qmax = 6.f; break;
    case SPARQ24_Q_NVFP4:
      cfmt = CF_NV; qmax = 6.f;
      if (q->tensor_amax_in && ((uintptr_t)q->tensor_amax_in & 3u)) return SPARQ24_ERR_ALIGN;
      break;
  }
  return SPARQ24_OK;
}

// Workspace protocol shared by the calls: (ws == NULL, ws_bytes != NULL) is a
// size query; otherwise the call runs and needs ws/*ws_bytes only when the
// required size is non-zero.
sparq24_status workspace(void* ws, size_t* ws_bytes, size_t need, bool& query) {
  if (!ws && ws_bytes) {
    *ws_bytes = need;
    query = true;
    return SPARQ24_OK;
  }
  query = false;
  if (need == 0) return SPARQ24_OK;
  if (!ws || !ws_bytes || *ws_bytes < need) return SPARQ24_ERR_WORKSPACE;
  if (!aligned16(ws)) return SPARQ24_ERR_ALIGN;
  return SPARQ24_OK;
}

sparq24_status device_ok() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SPARQ24_ERR_DEVICE;
  }
  return SPARQ24_OK;
}

sparq24_status launched(hipError_t e) {
  if (e == hipSuccess) return SPARQ24_OK;
  (void)hipGetLastError();
  return SPARQ24_ERR_LAUNCH;
}

#define CHECK(expr)                              \
  do {                                           \
    sparq24_status _st = (expr);                 \
    if (_st != SPARQ24_OK) return _st;           \
  } while (0)

size_t staging_bytes(const RowDesc& d);
RowDesc staged_view(const RowDesc& d, void* ws);

// Energy-call planning: unique kept/dense quantizers, pair columns, workspace.
struct EnergyPlan {
  EnergyParams p;
  FinalizeParams f;
  const float* nv_in = nullptr;
  const float* knv_in = nullptr;  // NVFP4 on kept values
  bool need_nv_partials = false, need_knv_partials = false;
  bool nv_second_pass = false;
  int nparts = 0, nkparts = 0;
  int64_t nrows = 0, rpb = 0, nblk = 0;
  size_t off_rowpart = 0, off_csum = 0, off_parts = 0, off_kparts = 0, need = 0;
};

sparq24_status plan_energy(const RowDesc& d, const sparq24_qspec* kept_q,
                           const sparq24_qspec* dense_q, int npairs, int64_t rows_per_block,
                           EnergyPlan& pl) {
  memset(&pl.p, 0, sizeof(pl.p));
  memset(&pl.f, 0, sizeof(pl.f));
  const sparq24_qspec* kept_u[kMaxQ];
  const sparq24_qspec* dense_u[kMaxQ];
  int nk = 0, nd = 0;
  const unsigned kept_ok = (1u << SPARQ24_Q_NONE) | (1u << SPARQ24_Q_INT) |
                           (1u << SPARQ24_Q_FP8_E4M3) | (1u << SPARQ24_Q_MXFP4) |
                           (1u << SPARQ24_Q_NVFP4);
  const unsigned dense_ok = kept_ok & ~(1u << SPARQ24_Q_NONE);
  auto same = [](const sparq24_qspec* a, const sparq24_qspec* b) {
    return a->fmt == b->fmt && (a->fmt != SPARQ24_Q_INT || a->bits == b->bits) &&
           (a->fmt != SPARQ24_Q_NVFP4 || a->tensor_amax_in == b->tensor_amax_in);
  };
  for (int i = 0; i < npairs; ++i) {
    int cf;
    float qm;
    CHECK(check_q(&kept_q[i], kept_ok, cf, qm));
    CHECK(check_q(&dense_q[i], dense_ok, cf, qm));
    if (dense_q[i].fmt == SPARQ24_Q_MXFP4 && d.K % 32) return SPARQ24_ERR_SHAPE;
    if (dense_q[i].fmt == SPARQ24_Q_NVFP4 && d.K % 16) return SPARQ24_ERR_SHAPE;
    // block formats on kept values block the compressed row (K/2 values)
    if (kept_q[i].fmt == SPARQ24_Q_MXFP4 && d.K % 64) return SPARQ24_ERR_SHAPE;
    if (kept_q[i].fmt == SPARQ24_Q_NVFP4 && d.K % 32) return SPARQ24_ERR_SHAPE;
  }
  for (int i = 0; i < npairs; ++i) {
    int ki = -1, di = -1;
    for (int j = 0; j < nk; ++j)
      if (same(kept_u[j], &kept_q[i])) ki = j;
    if (ki < 0) { kept_u[nk] = &kept_q[i]; ki = nk++; }
    for (int j = 0; j < nd; ++j)
      if (same(dense_u[j], &dense_q[i])) di = j;
    if (di < 0) { dense_u[nd] = &dense_q[i]; di = nd++; }
    pl.f.kcol[i] = 2 + ki;
    pl.f.dcol[i] = di;  // fixed up below once nk is known
  }
  int n_nv = 0, n_knv = 0;
  for (int j = 0; j < nk; ++j) {
    float qm;
    int cf;
    check_q(kept_u[j], kept_ok, cf, qm);
    pl.p.kept.fmt[j] = cf;
    pl.p.kept.qmax[j] = qm;
    if (cf == CF_NV) {
      ++n_knv;
      pl.knv_in = kept_u[j]->tensor_amax_in;
    }
  }
  for (int j = 0; j < nd; ++j) {
    float qm;
    int cf;
    check_q(dense_u[j], dense_ok, cf, qm);
    pl.p.dense.fmt[j] = cf;
    pl.p.dense.qmax[j] = qm;
    if (cf == CF_NV) {
      ++n_nv;
      pl.nv_in = dense_u[j]->tensor_amax_in;
    }
  }
  if (n_nv > 1 || n_knv > 1) return SPARQ24_ERR_UNSUPPORTED;
  for (int j = 0; j < nk; ++j) {
    pl.p.kept_twin[j] = -1;
    const int cf = pl.p.kept.fmt[j];
    if (cf != CF_INT8 && cf != CF_INT16 && cf != CF_FP8) continue;
    for (int i = 0; i < nd; ++i)
      if (pl.p.dense.fmt[i] == cf && pl.p.dense.qmax[i] == pl.p.kept.qmax[j]) pl.p.kept_twin[j] = i;
  }
  auto is_int = [](int cf) { return cf == CF_INT8 || cf == CF_INT16; };
  pl.p.n_kept_int = pl.p.n_kept_int_solo = pl.p.n_dense_int = 0;
  for (int j = 0; j < nk; ++j) {
    if (!is_int(pl.p.kept.fmt[j])) continue;
    pl.p.kept_int[pl.p.n_kept_int++] = j;
    if (pl.p.kept_twin[j] < 0) pl.p.kept_int_solo[pl.p.n_kept_int_solo++] = j;
  }
  for (int i = 0; i < nd; ++i)
    if (is_int(pl.p.dense.fmt[i])) pl.p.dense_int[pl.p.n_dense_int++] = i;
  pl.p.kept.n = nk;
  pl.p.dense.n = nd;
  for (int i = 0; i < npairs; ++i) pl.f.dcol[i] += 2 + nk;
  pl.f.ncols = 2 + nk + nd;
  pl.f.npairs = npairs;
  pl.nrows = d.B * d.R;
  pl.rpb = rows_per_block == 0 ? pl.nrows : rows_per_block;
  pl.nblk = (pl.nrows + pl.rpb - 1) / pl.rpb;
  pl.need_nv_partials = n_nv == 1 && pl.nv_in == nullptr;
  // bf16 rows of up to 4096 elements without rotation: the energy pass
  // itself leaves the tensor maximum's partials (one per workgroup of its
  // grid, at most energy_max_workgroups()) and a second pass evaluates the dense
  // NVFP4 quantizer; otherwise a maximum pass runs first
  pl.nv_second_pass = pl.need_nv_partials && d.dtype == 1 && d.rot.n == 0 && d.K <= 4096;
  pl.nparts = !pl.need_nv_partials ? 0
              : pl.nv_second_pass ? energy_max_workgroups()
                                  : absmax_partial_count(d);
  pl.need_knv_partials = n_knv == 1 && pl.knv_in == nullptr;
  pl.nkparts = pl.need_knv_partials ? absmax_partial_count(d) : 0;
  const size_t rowpart = (size_t)pl.f.ncols * (size_t)energy_partial_rows(pl.nrows) * sizeof(double);
  const size_t sums = (size_t)pl.f.ncols * (size_t)pl.nblk *
                      (size_t)energy_chunks_per_block(pl.rpb) * sizeof(double);
  pl.off_rowpart = staging_bytes(d);
  pl.off_csum = pl.off_rowpart + round_up(rowpart, kAlign);
  pl.off_parts = pl.off_csum + round_up(sums, kAlign);
  pl.off_kparts = pl.off_parts + round_up((size_t)pl.nparts * sizeof(uint32_t), kAlign);
  pl.need = pl.off_kparts + round_up((size_t)pl.nkparts * sizeof(uint32_t), kAlign);
  return SPARQ24_OK;
}

sparq24_status run_energy(RowDesc d, int32_t score, const float* col_norm, EnergyPlan& pl,
                          double* out, void* ws, hipStream_t stream) {
  char* w = (char*)ws;
  if (!d.kcontig) {
    CHECK(launched(launch_transpose_rows(d, ws, stream)));
    d = staged_view(d, ws);
  }
  double* rowpart = (double*)(w + pl.off_rowpart);
  uint32_t* parts = (uint32_t*)(w + pl.off_parts);
  if (pl.nv_second_pass) {
    pl.p.defer_nv = 1;
    pl.p.max_out = parts;
  } else if (pl.need_nv_partials) {
    CHECK(launched(launch_absmax_partials(d, parts, stream)));
    pl.p.nv_partials = parts;
    pl.p.n_partials = pl.nparts;
  }
  pl.p.nv_tamax = pl.nv_in;
  if (pl.need_knv_partials) {
    uint32_t* kparts = (uint32_t*)(w + pl.off_kparts);
    CHECK(launched(launch_kept_absmax_partials(d, pl.p.pairs48 ? PAT_48 : PAT_24,
                                               score == SPARQ24_SCORE_WANDA, col_norm, kparts,
                                               stream)));
    pl.p.kept_nv_partials = kparts;
    pl.p.n_kept_partials = pl.nkparts;
  }
  pl.p.kept_nv_tamax = pl.knv_in;
  int64_t nparts = 0, grid = 0;
  CHECK(launched(launch_energy_rows(d, score == SPARQ24_SCORE_WANDA, col_norm, pl.p, rowpart,
                                    pl.rpb, &nparts, stream, &grid)));
  if (pl.nv_second_pass) {
    int qnv = 0;
    for (int q = 0; q < pl.p.dense.n; ++q)
      if (pl.p.dense.fmt[q] == CF_NV) qnv = q;
    if (grid > pl.nparts) return SPARQ24_ERR_LAUNCH;  // the maxima buffer holds one per workgroup
    CHECK(launched(launch_energy_nv_dense(d, parts, (int)grid, 2 + pl.p.kept.n + qnv, rowpart,
                                          pl.rpb, grid, stream)));
  }
  double* csum = (double*)(w + pl.off_csum);
  if (pl.rpb >= pl.nrows)  // one block: reduce the per-workgroup partials
    return launched(launch_energy_finalize(rowpart, nparts, nparts, 1, pl.f, csum, out, stream));
  return launched(launch_energy_finalize(rowpart, pl.nrows, pl.rpb, pl.nblk, pl.f, csum, out, stream));
}

// Transposed operands are staged as dense K-contiguous rows at the start of
// the workspace; the calls then run on that copy.
size_t staging_bytes(const RowDesc& d) {
  if (d.kcontig) return 0;
  return round_up((size_t)(d.B * d.R * d.K) * (size_t)esize(d.dtype), kAlign);
}

RowDesc staged_view(const RowDesc& d, void* ws) {
  RowDesc v = d;
  v.x = (const char*)ws;
  v.R = d.B * d.R;
  v.B = 1;
  v.rs = d.K * esize(d.dtype);
  v.bs = v.R * v.rs;
  v.ks = esize(d.dtype);
  v.kcontig = true;
  v.flat = true;
  return v;
}

}  // namespace

extern "C" {

sparq24_status sparq24_prune_compress(const sparq24_tensor* x, int32_t score, const float* col_norm,
                                      void* values, uint8_t* meta, hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, true, d));
  CHECK(check_score(score, col_norm));
  if (d.B * d.R * d.K == 0) return SPARQ24_OK;
  if (!values || !meta) return SPARQ24_ERR_INVALID;
  if (!aligned16(values) || !aligned16(meta)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_prune_compress(d, score == SPARQ24_SCORE_WANDA, col_norm, values, meta, stream));
}

}  // extern "C"

namespace {

// Shared bodies of the calls; rot_block != 0 rotates the operand on load.
sparq24_status quantize_any(const sparq24_tensor* x, int32_t rot_block, const sparq24_qspec* q,
                            void* codes, void* scales, float* tensor_scale_out, void* ws,
                            size_t* ws_bytes, hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, true, d));
  if (rot_block) CHECK(check_rot(rot_block, d));
  int cfmt;
  float qmax;
  CHECK(check_q(q, (1u << SPARQ24_Q_INT) | (1u << SPARQ24_Q_FP8_E4M3) | (1u << SPARQ24_Q_MXFP4) |
                       (1u << SPARQ24_Q_NVFP4),
                cfmt, qmax));
  if (cfmt == CF_MX && d.K % 32) return SPARQ24_ERR_SHAPE;
  if (cfmt == CF_NV && d.K % 16) return SPARQ24_ERR_SHAPE;
  if ((cfmt == CF_INT8 || cfmt == CF_INT16 || cfmt == CF_FP8) && d.K / 8 > kMaxRowUnits)
    return SPARQ24_ERR_SHAPE;
  const bool nv_parts = cfmt == CF_NV && q->tensor_amax_in == nullptr;
  const int nparts = nv_parts ? absmax_partial_count(d) : 0;
  const size_t stage = staging_bytes(d);
  const size_t need = stage + round_up((size_t)nparts * sizeof(uint32_t), kAlign);
  bool query;
  CHECK(workspace(ws, ws_bytes, need, query));
  if (query) return SPARQ24_OK;
  if (d.B * d.R * d.K == 0) return SPARQ24_OK;
  if (!codes || !scales) return SPARQ24_ERR_INVALID;
  if (cfmt == CF_NV && !tensor_scale_out) return SPARQ24_ERR_INVALID;
  if (!aligned16(codes) || !aligned16(scales)) return SPARQ24_ERR_ALIGN;
  if (cfmt == CF_NV && ((uintptr_t)tensor_scale_out & 3u)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  if (stage) {
    CHECK(launched(launch_transpose_rows(d, ws, stream)));
    d = staged_view(d, ws);
  }
  if (cfmt == CF_MX) return launched(launch_quant_mx(d, codes, (uint8_t*)scales, stream));
  if (cfmt == CF_NV) {
    uint32_t* parts = (uint32_t*)((char*)ws + stage);
    if (nv_parts) CHECK(launched(launch_absmax_partials(d, parts, stream)));
    return launched(launch_quant_nv(d, q->tensor_amax_in, parts, nparts, codes, (uint8_t*)scales,
                                    tensor_scale_out, stream));
  }
  return launched(launch_quant_rows(d, cfmt, qmax, codes, (float*)scales, stream));
}

sparq24_status prune_quantize_any(const sparq24_tensor* x, int32_t rot_block, int pat,
                                  int32_t score, const float* col_norm, const sparq24_qspec* q,
                                  void* codes, uint8_t* meta, void* scales,
                                  float* tensor_scale_out, void* ws, size_t* ws_bytes,
                                  hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, true, d));
  if (rot_block) CHECK(check_rot(rot_block, d));
  CHECK(check_score(score, col_norm));
  int cfmt;
  float qmax;
  CHECK(check_q(q, (1u << SPARQ24_Q_INT) | (1u << SPARQ24_Q_FP8_E4M3) | (1u << SPARQ24_Q_MXFP4) |
                       (1u << SPARQ24_Q_NVFP4),
                cfmt, qmax));
  const bool block = cfmt == CF_MX || cfmt == CF_NV;
  if (pat == PAT_48 && d.K % 16) return SPARQ24_ERR_SHAPE;
  if (cfmt == CF_MX && d.K % 64) return SPARQ24_ERR_SHAPE;  // 32 kept values per block
  if (cfmt == CF_NV && d.K % 32) return SPARQ24_ERR_SHAPE;  // 16 kept values per block
  if (!block && d.K / 8 > kMaxRowUnits) return SPARQ24_ERR_SHAPE;
  const bool nv_parts = cfmt == CF_NV && q->tensor_amax_in == nullptr;
  const int nparts = nv_parts ? absmax_partial_count(d) : 0;
  const size_t stage = staging_bytes(d);
  const size_t need = stage + round_up((size_t)nparts * sizeof(uint32_t), kAlign);
  bool query;
  CHECK(workspace(ws, ws_bytes, need, query));
  if (query) return SPARQ24_OK;
  if (d.B * d.R * d.K == 0) return SPARQ24_OK;
  if (!codes || !meta || !scales) return SPARQ24_ERR_INVALID;
  if (cfmt == CF_NV && !tensor_scale_out) return SPARQ24_ERR_INVALID;
  if (!aligned16(codes) || !aligned16(meta) || !aligned16(scales)) return SPARQ24_ERR_ALIGN;
  if (cfmt == CF_NV && ((uintptr_t)tensor_scale_out & 3u)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  if (stage) {
    CHECK(launched(launch_transpose_rows(d, ws, stream)));
    d = staged_view(d, ws);
  }
  const bool wanda = score == SPARQ24_SCORE_WANDA;
  if (block) {
    uint32_t* parts = (uint32_t*)((char*)ws + stage);
    if (nv_parts) CHECK(launched(launch_kept_absmax_partials(d, pat, wanda, col_norm, parts, stream)));
    return launched(launch_prune_quant_fp4(d, pat, wanda, col_norm, cfmt, q->tensor_amax_in, parts,
                                           nparts, codes, meta, (uint8_t*)scales,
                                           tensor_scale_out, stream));
  }
  return launched(launch_prune_quantize(d, pat, wanda, col_norm, cfmt, qmax, codes, meta,
                                        (float*)scales, stream));
}

// mode 0: error_energy (one pair, raw sums); 1: predict_R
// Validation and planning shared by the energy calls.
sparq24_status energy_plan(const sparq24_tensor* x, int32_t rot_block, int pat, int32_t score,
                           const float* col_norm, const sparq24_qspec* kept_q,
                           const sparq24_qspec* dense_q, int32_t npairs, int64_t rows_per_block,
                           int mode, RowDesc& d, EnergyPlan& pl) {
  CHECK(check_tensor(x, true, d));
  if (rot_block) CHECK(check_rot(rot_block, d));
  CHECK(check_score(score, col_norm));
  if (pat == PAT_48 && score != SPARQ24_SCORE_MAGNITUDE) return SPARQ24_ERR_UNSUPPORTED;
  if (!kept_q || !dense_q) return SPARQ24_ERR_INVALID;
  if (npairs < 1 || npairs > SPARQ24_MAX_PAIRS) return SPARQ24_ERR_INVALID;
  if (rows_per_block < 0) return SPARQ24_ERR_INVALID;
  if (pat == PAT_48 && d.K % 16) return SPARQ24_ERR_SHAPE;
  if (d.B * d.R == 0 || d.K == 0) return SPARQ24_ERR_SHAPE;
  if (d.K / 8 > kMaxRowUnits) return SPARQ24_ERR_SHAPE;
  CHECK(plan_energy(d, kept_q, dense_q, npairs, rows_per_block, pl));
  pl.p.pairs48 = pat == PAT_48 ? 1 : 0;
  pl.f.mode = mode;
  return SPARQ24_OK;
}

sparq24_status energy_any(const sparq24_tensor* x, int32_t rot_block, int pat, int32_t score,
                          const float* col_norm, const sparq24_qspec* kept_q,
                          const sparq24_qspec* dense_q, int32_t npairs, int64_t rows_per_block,
                          int mode, double* out, void* ws, size_t* ws_bytes, hipStream_t stream) {
  RowDesc d;
  EnergyPlan pl;
  CHECK(energy_plan(x, rot_block, pat, score, col_norm, kept_q, dense_q, npairs, rows_per_block,
                    mode, d, pl));
  bool query;
  CHECK(workspace(ws, ws_bytes, pl.need, query));
  if (query) return SPARQ24_OK;
  if (!out) return SPARQ24_ERR_INVALID;
  if (!aligned16(out)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return run_energy(d, score, col_norm, pl, out, ws, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free predict_R.  Its workspace is `scratch`, the static device
// array at the top of this file: every GPU the library runs on holds one copy
// until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory,
// so the device address of the current device's copy is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; kernels
// and copies only ever receive that address.
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

sparq24_status scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SPARQ24_ERR_DEVICE;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {  // two threads racing here both store the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SPARQ24_ERR_DEVICE;
    }
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *addr = p;
  return SPARQ24_OK;
}

int32_t pattern_code(int32_t pattern) {
  return pattern == SPARQ24_PATTERN_24 ? PAT_24 : (pattern == SPARQ24_PATTERN_PAIRS48 ? PAT_48 : -1);
}

}  // namespace

extern "C" {

sparq24_status sparq24_quantize(const sparq24_tensor* x, const sparq24_qspec* q, void* codes,
                                void* scales, float* tensor_scale_out, void* ws, size_t* ws_bytes,
                                hipStream_t stream) {
  return quantize_any(x, 0, q, codes, scales, tensor_scale_out, ws, ws_bytes, stream);
}

sparq24_status sparq24_prune_quantize(const sparq24_tensor* x, int32_t score, const float* col_norm,
                                      const sparq24_qspec* q, void* codes, uint8_t* meta,
                                      void* scales, float* tensor_scale_out, void* ws,
                                      size_t* ws_bytes, hipStream_t stream) {
  return prune_quantize_any(x, 0, PAT_24, score, col_norm, q, codes, meta, scales,
                            tensor_scale_out, ws, ws_bytes, stream);
}

sparq24_status sparq24_prune_quantize_pairs48(const sparq24_tensor* x, const sparq24_qspec* q,
                                              void* codes, uint8_t* meta, void* scales,
                                              float* tensor_scale_out, void* ws,
                                              size_t* ws_bytes, hipStream_t stream) {
  return prune_quantize_any(x, 0, PAT_48, SPARQ24_SCORE_MAGNITUDE, nullptr, q, codes, meta,
                            scales, tensor_scale_out, ws, ws_bytes, stream);
}

sparq24_status sparq24_error_energy(const sparq24_tensor* x, int32_t score, const float* col_norm,
                                    const sparq24_qspec* kept_q, const sparq24_qspec* dense_q,
                                    int64_t rows_per_block, double* out, void* ws,
                                    size_t* ws_bytes, hipStream_t stream) {
  return energy_any(x, 0, PAT_24, score, col_norm, kept_q, dense_q, 1, rows_per_block, 0, out, ws,
                    ws_bytes, stream);
}

sparq24_status sparq24_predict_R(const sparq24_tensor* x, int32_t score, const float* col_norm,
                                 const sparq24_qspec* kept_q, const sparq24_qspec* dense_q,
                                 int32_t npairs, int64_t rows_per_block, double* out, void* ws,
                                 size_t* ws_bytes, hipStream_t stream) {
  return energy_any(x, 0, PAT_24, score, col_norm, kept_q, dense_q, npairs, rows_per_block, 1, out,
                    ws, ws_bytes, stream);
}

sparq24_status sparq24_predict_R_noalloc(const sparq24_tensor* x, int32_t score,
                                         const float* col_norm, const sparq24_qspec* kept_q,
                                         const sparq24_qspec* dense_q, int32_t npairs,
                                         int64_t rows_per_block, double* out, hipStream_t stream) {
  RowDesc d;
  EnergyPlan pl;
  CHECK(energy_plan(x, 0, PAT_24, score, col_norm, kept_q, dense_q, npairs, rows_per_block, 1, d,
                    pl));
  if (pl.need > (size_t)SPARQ24_NOALLOC_SCRATCH_BYTES) return SPARQ24_ERR_WORKSPACE;
  if (!out) return SPARQ24_ERR_INVALID;
  if (!aligned16(out)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  void* ws = nullptr;
  CHECK(scratch_address(&ws));
  return run_energy(d, score, col_norm, pl, out, ws, stream);
}

sparq24_status sparq24_prune_compress_pairs48(const sparq24_tensor* x, void* values,
                                              uint8_t* meta, hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, false, d));
  if (d.K % 16) return SPARQ24_ERR_SHAPE;
  if (d.B * d.R * d.K == 0) return SPARQ24_OK;
  if (!values || !meta) return SPARQ24_ERR_INVALID;
  if (!aligned16(values) || !aligned16(meta)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_prune_compress_pairs48(d, values, meta, stream));
}

sparq24_status sparq24_predict_R_pairs48(const sparq24_tensor* x, const sparq24_qspec* kept_q,
                                         const sparq24_qspec* dense_q, int32_t npairs,
                                         int64_t rows_per_block, double* out, void* ws,
                                         size_t* ws_bytes, hipStream_t stream) {
  return energy_any(x, 0, PAT_48, SPARQ24_SCORE_MAGNITUDE, nullptr, kept_q, dense_q, npairs,
                    rows_per_block, 1, out, ws, ws_bytes, stream);
}

sparq24_status sparq24_hadamard(const sparq24_tensor* x, int32_t block, void* out, void* ws,
                                size_t* ws_bytes, hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, true, d));
  CHECK(check_rot(block, d));
  const size_t stage = staging_bytes(d);
  bool query;
  CHECK(workspace(ws, ws_bytes, stage, query));
  if (query) return SPARQ24_OK;
  if (d.B * d.R * d.K == 0) return SPARQ24_OK;
  if (!out) return SPARQ24_ERR_INVALID;
  if (!aligned16(out)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  if (stage) {
    CHECK(launched(launch_transpose_rows(d, ws, stream)));
    d = staged_view(d, ws);
  }
  return launched(launch_hadamard(d, out, stream));
}

sparq24_status sparq24_quantize_rot(const sparq24_tensor* x, int32_t block,
                                    const sparq24_qspec* q, void* codes, void* scales,
                                    float* tensor_scale_out, void* ws, size_t* ws_bytes,
                                    hipStream_t stream) {
  if (block == 0) return SPARQ24_ERR_INVALID;
  return quantize_any(x, block, q, codes, scales, tensor_scale_out, ws, ws_bytes, stream);
}

sparq24_status sparq24_prune_quantize_rot(const sparq24_tensor* x, int32_t block, int32_t pattern,
                                          const sparq24_qspec* q, void* codes, uint8_t* meta,
                                          void* scales, float* tensor_scale_out, void* ws,
                                          size_t* ws_bytes, hipStream_t stream) {
  const int32_t pat = pattern_code(pattern);
  if (block == 0 || pat < 0) return SPARQ24_ERR_INVALID;
  return prune_quantize_any(x, block, pat, SPARQ24_SCORE_MAGNITUDE, nullptr, q, codes, meta,
                            scales, tensor_scale_out, ws, ws_bytes, stream);
}

sparq24_status sparq24_predict_R_rot(const sparq24_tensor* x, int32_t block, int32_t pattern,
                                     const sparq24_qspec* kept_q, const sparq24_qspec* dense_q,
                                     int32_t npairs, int64_t rows_per_block, double* out,
                                     void* ws, size_t* ws_bytes, hipStream_t stream) {
  const int32_t pat = pattern_code(pattern);
  if (block == 0 || pat < 0) return SPARQ24_ERR_INVALID;
  return energy_any(x, block, pat, SPARQ24_SCORE_MAGNITUDE, nullptr, kept_q, dense_q, npairs,
                    rows_per_block, 1, out, ws, ws_bytes, stream);
}

sparq24_status sparq24_operator_error(const sparq24_tensor* a, const sparq24_tensor* b,
                                     const sparq24_side* sides, int32_t nsides, double* out,
                                     void* ws, size_t* ws_bytes, hipStream_t stream) {
  RowDesc d, e;
  CHECK(check_tensor(a, false, d));
  CHECK(check_tensor(b, false, e));
  if (d.dtype != SPARQ24_BF16 || e.dtype != SPARQ24_BF16) return SPARQ24_ERR_UNSUPPORTED;
  if (!sides || nsides < 1 || nsides > SPARQ24_MAX_PAIRS) return SPARQ24_ERR_INVALID;
  if (d.K != e.K) return SPARQ24_ERR_SHAPE;
  if (d.K % 64) return SPARQ24_ERR_SHAPE;  // GEMM K slabs (and every block format)
  if (d.K / 8 > kMaxRowUnits) return SPARQ24_ERR_SHAPE;
  if (d.B * d.R == 0 || e.B * e.R == 0 || d.K == 0) return SPARQ24_ERR_SHAPE;
  if (d.B > 1 || e.B > 1) return SPARQ24_ERR_UNSUPPORTED;  // rows must share one stride
  SideParams sp[SPARQ24_MAX_PAIRS];
  int nv_sides = 0;
  for (int i = 0; i < nsides; ++i) {
    const int pat = sides[i].pattern == SPARQ24_PATTERN_24        ? PAT_24
                    : sides[i].pattern == SPARQ24_PATTERN_PAIRS48 ? PAT_48
                    : sides[i].pattern == SPARQ24_PATTERN_DENSE   ? PAT_DENSE
                                                                  : -1;
    if (pat < 0) return SPARQ24_ERR_INVALID;
    int cf;
    float qm;
    const unsigned ok = (pat == PAT_DENSE ? 0u : (1u << SPARQ24_Q_NONE)) | (1u << SPARQ24_Q_INT) |
                        (1u << SPARQ24_Q_FP8_E4M3) | (1u << SPARQ24_Q_MXFP4) |
                        (1u << SPARQ24_Q_NVFP4);
    CHECK(check_q(&sides[i].q, ok, cf, qm));
    sp[i] = SideParams{pat, cf, qm, sides[i].q.tensor_amax_in, nullptr, 0};
    if (cf == CF_NV && !sides[i].q.tensor_amax_in) ++nv_sides;
  }
  const int64_t M = d.R, N = e.R, K = d.K;
  const int64_t nt = gemm_col_tiles(N);
  const int nparts = nv_sides ? absmax_partial_count(d) : 0;
  const size_t delta_bytes = round_up((size_t)M * (size_t)(2 * K) * 2, kAlign);
  const size_t part_bytes = round_up((size_t)(1 + nsides) * (size_t)M * (size_t)nt * sizeof(float), kAlign);
  const size_t need = delta_bytes + part_bytes + round_up((size_t)nparts * sizeof(uint32_t), kAlign);
  bool query;
  CHECK(workspace(ws, ws_bytes, need, query));
  if (query) return SPARQ24_OK;
  if (!out) return SPARQ24_ERR_INVALID;
  if (!aligned16(out)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  char* w = (char*)ws;
  void* delta = w;
  float* part = (float*)(w + delta_bytes);
  uint32_t* parts = (uint32_t*)(w + delta_bytes + part_bytes);
  const int64_t lda = d.rs / 2, ldb = e.rs / 2;
  CHECK(launched(launch_gemm_rowsq(d.x, lda, e.x, ldb, M, N, K, K, part, stream)));
  for (int i = 0; i < nsides; ++i) {
    if (sp[i].fmt == CF_NV && !sp[i].tamax_in) {
      if (sp[i].pattern == PAT_DENSE) CHECK(launched(launch_absmax_partials(d, parts, stream)));
      else CHECK(launched(launch_kept_absmax_partials(d, sp[i].pattern, false, nullptr, parts, stream)));
      sp[i].partials = parts;
      sp[i].nparts = nparts;
    }
    CHECK(launched(launch_side_delta(d, sp[i], delta, stream)));
    CHECK(launched(launch_gemm_rowsq(delta, 2 * K, e.x, ldb, M, N, 2 * K, K,
                                     part + (size_t)(1 + i) * (size_t)M * (size_t)nt, stream)));
  }
  return launched(launch_rowsq_final(part, M, nt, 1 + nsides, out, stream));
}

sparq24_status sparq24_sparse_gemm(const void* values, const uint8_t* meta, int64_t m, int64_t k,
                                   const sparq24_tensor* b, float* c, hipStream_t stream) {
  RowDesc e;
  CHECK(check_tensor(b, false, e));
  if (m < 0 || k < 0) return SPARQ24_ERR_INVALID;
  if (e.dtype != SPARQ24_BF16) return SPARQ24_ERR_UNSUPPORTED;
  if (e.B > 1) return SPARQ24_ERR_UNSUPPORTED;
  if (k != e.K || k % 64) return SPARQ24_ERR_SHAPE;
  if (m == 0 || e.R == 0) return SPARQ24_OK;
  if (!values || !meta || !c) return SPARQ24_ERR_INVALID;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(c)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_sparse_gemm(values, meta, m, k, e.x, e.rs / 2, e.R, c, e.R, stream));
}

sparq24_status sparq24_dense_gemm(const sparq24_tensor* a, const sparq24_tensor* b, float* c,
                                  hipStream_t stream) {
  RowDesc d, e;
  CHECK(check_tensor(a, false, d));
  CHECK(check_tensor(b, false, e));
  if (d.dtype != SPARQ24_BF16 || e.dtype != SPARQ24_BF16) return SPARQ24_ERR_UNSUPPORTED;
  if (d.B > 1 || e.B > 1) return SPARQ24_ERR_UNSUPPORTED;
  if (d.K != e.K || d.K % 64) return SPARQ24_ERR_SHAPE;
  if (d.R == 0 || e.R == 0) return SPARQ24_OK;
  if (!c) return SPARQ24_ERR_INVALID;
  if (!aligned16(c)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_dense_gemm(d.x, d.rs / 2, d.R, d.K, e.x, e.rs / 2, e.R, c, e.R, stream));
}

sparq24_status sparq24_fp8_gemm(const uint8_t* a, const float* scale_a, int64_t m,
                                const uint8_t* b, const float* scale_b, int64_t n, int64_t k,
                                float* c, hipStream_t stream) {
  if (m < 0 || n < 0 || k < 0) return SPARQ24_ERR_INVALID;
  if (k % 128) return SPARQ24_ERR_SHAPE;
  if (m == 0 || n == 0) return SPARQ24_OK;
  if (!a || !b || !scale_a || !scale_b || !c) return SPARQ24_ERR_INVALID;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || ((uintptr_t)scale_a & 3u) ||
      ((uintptr_t)scale_b & 3u))
    return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_fp8_gemm(a, k, scale_a, m, k, b, k, scale_b, n, c, n, stream));
}

sparq24_status sparq24_col_l2norm(const sparq24_tensor* x, float* norms, void* ws,
                                  size_t* ws_bytes, hipStream_t stream) {
  RowDesc d;
  CHECK(check_tensor(x, false, d));
  const size_t need = round_up((size_t)col_strips(d) * (size_t)d.K * sizeof(double), kAlign);
  bool query;
  CHECK(workspace(ws, ws_bytes, need, query));
  if (query) return SPARQ24_OK;
  if (d.K == 0) return SPARQ24_OK;
  if (!norms) return SPARQ24_ERR_INVALID;
  if (!aligned16(norms)) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_col_l2norm(d, (double*)ws, norms, stream));
}

sparq24_status sparq24_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return SPARQ24_OK;
  if (!src || !dst) return SPARQ24_ERR_INVALID;
  if (!aligned16(src) || !aligned16(dst) || bytes % 16) return SPARQ24_ERR_ALIGN;
  CHECK(device_ok());
  return launched(launch_copy(src, dst, bytes, stream));
}

double sparq24_bits_per_element(const sparq24_qspec* q, int32_t sparse24, int64_t row_len,
                                int32_t value_bits, int64_t tensor_elems) {
  if (!q || row_len < 0 || tensor_elems < 0 || sparse24 < 0 || sparse24 > 2) return -1.0;
  double v, row = 0.0, block = 0.0, tensor = 0.0;
  switch (q->fmt) {
    case SPARQ24_Q_INT:
      if (q->bits < 2 || q->bits > 16) return -1.0;
      v = q->bits;
      row = row_len ? 32.0 / (double)row_len : 0.0;
      break;
    case SPARQ24_Q_FP8_E4M3:
      v = 8;
      row = row_len ? 32.0 / (double)row_len : 0.0;
      break;
    case SPARQ24_Q_NONE:
      if (value_bits <= 0) return -1.0;
      v = value_bits;
      break;
    case SPARQ24_Q_MXFP4:
      v = 4;
      block = 8.0 / 32.0;
      break;
    case SPARQ24_Q_NVFP4:
      v = 4;
      block = 8.0 / 16.0;
      tensor = tensor_elems ? 32.0 / (double)tensor_elems : 0.0;
      break;
    default:
      return -1.0;
  }
  if (sparse24 == 0) return v + row + block + tensor;
  // half the values are kept; block scales cover kept values; position bits:
  // 2 per kept value (2:4) or 2 per kept pair (pairwise 4:8)
  const double index = sparse24 == 1 ? 1.0 : 0.5;
  return v / 2.0 + index + row + block / 2.0 + tensor;
}

const char* sparq24_status_string(sparq24_status s) {
  switch (s) {
    case SPARQ24_OK: return "ok";
    case SPARQ24_ERR_INVALID: return "invalid argument";
    case SPARQ24_ERR_UNSUPPORTED: return "unsupported dtype, format, bits or layout";
    case SPARQ24_ERR_SHAPE: return "unsupported shape";
    case SPARQ24_ERR_ALIGN: return "misaligned pointer or stride";
    case SPARQ24_ERR_WORKSPACE: return "workspace missing or too small";
    case SPARQ24_ERR_DEVICE: return "no usable HIP device";
    case SPARQ24_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* sparq24_version(void) { return "0.1.0"; }

}  // extern "C"
