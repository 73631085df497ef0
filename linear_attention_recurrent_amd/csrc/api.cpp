// C ABI of the DeltaLog decode library: host-side argument checks and the
// launch sequence.  The operations, layouts and status codes are documented in
// include/deltalog.h.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "deltalog.h"
#include "launch.hpp"

namespace {

// Arrays read or written with 16-byte vector accesses need 16-byte alignment;
// arrays of one scalar per tile (and the output) need 4.
bool misaligned(const void* ptr, uintptr_t align = 16) {
  return (reinterpret_cast<uintptr_t>(ptr) & (align - 1)) != 0;
}

int check_dims(const dl_dims* d) {
  if (d == nullptr) return DL_EINVAL;
  if (d->variant < DL_GDN || d->variant > DL_RWKV6) return DL_EINVAL;
  if (d->batch < 0 || d->heads < 1) return DL_EINVAL;
  if (d->log_len < 1 || d->log_len > DL_MAX_LOG_LEN) return DL_EINVAL;
  if (static_cast<int64_t>(d->batch) * d->heads > INT32_MAX) return DL_EINVAL;
  if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128)) return DL_EUNSUPPORTED;
  if (d->base_dtype != DL_BASE_F32 && d->base_dtype != DL_BASE_BF16) return DL_EINVAL;
  return DL_OK;
}

int check_pool(const dl_pool* p, int variant) {
  if (p == nullptr) return DL_EINVAL;
  if (!p->base || !p->log_k || !p->log_u || !p->log_c || !p->fill) return DL_EINVAL;
  if (misaligned(p->base) || misaligned(p->log_k) || misaligned(p->log_u) ||
      misaligned(p->log_c, variant == DL_GDN ? 4 : 16) || misaligned(p->fill, 4))
    return DL_EALIGN;
  return DL_OK;
}

int check_io(const dl_dims* d, const dl_step_io* io) {
  if (io == nullptr) return DL_EINVAL;
  if (!io->q || !io->k || !io->v || !io->decay || !io->out) return DL_EINVAL;
  const bool rwkv = d->variant == DL_RWKV6;
  if (rwkv && (io->beta != nullptr || io->eta != nullptr || io->bonus == nullptr)) return DL_EUNSUPPORTED;
  // GDN/KDA: exactly one of beta (given step size) and eta (Kaczmarz step size)
  if (!rwkv && ((io->beta == nullptr) == (io->eta == nullptr) || io->bonus != nullptr)) return DL_EUNSUPPORTED;
  if (io->eta != nullptr && !(io->eps >= 0.f)) return DL_EINVAL;
  if (misaligned(io->q) || misaligned(io->k) || misaligned(io->v) ||
      misaligned(io->decay, rwkv || d->variant == DL_KDA ? 16 : 4) || misaligned(io->out, 4) ||
      (io->beta && misaligned(io->beta, 4)) || (io->eta && misaligned(io->eta, 4)) ||
      (io->bonus && misaligned(io->bonus)))
    return DL_EALIGN;
  return DL_OK;
}

dl::PoolArgs pool_args(const dl_dims* d, const dl_pool* p) {
  return dl::PoolArgs{p->base, p->log_k, p->log_u, p->log_c, p->fill, d->heads, d->log_len, d->batch * d->heads};
}

bool bf16_base(const dl_dims* d) { return d->base_dtype == DL_BASE_BF16;
}

dl::StepArgs step_args(const dl_step_io* io) {
  return dl::StepArgs{io->q, io->k, io->v, io->decay, io->beta, io->bonus, io->out, io->eta, io->eps};
}

int hip_status(hipError_t e) { return e == hipSuccess ? DL_OK : DL_EHIP; }

}  // namespace

extern "C" {

int dl_init_state(const dl_dims* dims, const dl_pool* pool, const float* init_base,
                  const int32_t* init_fill, void* stream) {
  int rc = check_dims(dims);
  if (rc != DL_OK || dims->batch == 0) return rc;
  if ((rc = check_pool(pool, dims->variant)) != DL_OK) return rc;
  if (init_base && misaligned(init_base)) return DL_EALIGN;
  const int batch = dims->batch, heads = dims->heads;
  std::vector<int32_t> fills(static_cast<size_t>(batch) * heads, 0);
  if (init_fill) {
    for (int b = 0; b < batch; ++b) {
      if (init_fill[b] < 0 || init_fill[b] >= dims->log_len) return DL_EINVAL;
      for (int h = 0; h < heads; ++h) fills[static_cast<size_t>(b) * heads + h] = init_fill[b];
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(pool->fill, fills.data(), fills.size() * sizeof(int32_t),
                                hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return DL_EHIP;
  e = dl::launch_init(dims->variant, bf16_base(dims), dims->dk, dims->dv, batch * heads, pool_args(dims, pool),
                      init_base, st);
  if (e != hipSuccess) return DL_EHIP;
  return hip_status(hipStreamSynchronize(st));
}

int dl_decode_step(const dl_dims* dims, const dl_pool* pool, const dl_step_io* io, void* stream) {
  int rc = check_dims(dims);
  if (rc != DL_OK || dims->batch == 0) return rc;
  if ((rc = check_pool(pool, dims->variant)) != DL_OK) return rc;
  if ((rc = check_io(dims, io)) != DL_OK) return rc;
  return hip_status(dl::launch_decode(dims->variant, bf16_base(dims), dims->dk, dims->dv, dims->batch * dims->heads,
                                      pool_args(dims, pool), step_args(io),
                                      static_cast<hipStream_t>(stream)));
}

// The shortest log length at which dl_merge folds on the matrix cores: where the fp32
// MFMA fold measured faster than the vector fold on full logs (one MI355X, every tile
// holding L - 1 entries; MFMA time over vector time at L = 4, 8, 16, 32, 64):
//   128 x 128, fp32 base        32   (GDN B=64 H=32: 0.93 0.95 0.90 1.27 1.83;
//                                      KDA B=128 H=32: 0.91 0.97 0.96 1.32 1.71)
//   128 x 128, bf16 base, GDN   32   (0.95 1.02 1.02 1.12 1.25)
//   128 x 128, bf16 base, else  64   (KDA: 0.87 0.82 0.88 0.96 1.23)
//   128 x 64 / 64 x 128, fp32   64   (0.95 0.97 0.97 0.94 1.24 / 0.96 0.96 0.96 0.91 1.07)
//   64 x 64, and 128 x 64 / 64 x 128 with a bf16 base: never (at most 1.04, mostly < 0.95)
// The vector fold streams its stages from one in-register tile and loads each stage's
// entries with 16-byte loads issued together; the matrix fold holds the tile in MFMA
// accumulators and wins once the rank-n update's arithmetic outweighs the shared traffic.
static int merge_mfma_min_len(const dl_dims* d) {
  const bool bf = bf16_base(d);
  if (d->dk == 128 && d->dv == 128) return bf ? (d->variant == DL_GDN ? 32 : 64) : 32;
  if ((d->dk == 128) != (d->dv == 128)) return bf ? DL_MAX_LOG_LEN + 1 : 64;
  return DL_MAX_LOG_LEN + 1;
}

static bool merge_on_mfma(const dl_dims* dims, int32_t unit) {
  if (unit == DL_UNIT_VALU) return false;
  if (unit == DL_UNIT_MFMA) return true;
  return dims->log_len >= merge_mfma_min_len(dims);
}

// Fold every log holding >= min_fill entries (arguments already checked).
static hipError_t launch_fold(const dl_dims* dims, const dl_pool* pool, int32_t min_fill, int32_t unit,
                              hipStream_t st) {
  const int tiles = dims->batch * dims->heads;
  if (merge_on_mfma(dims, unit))
    return dl::launch_merge_mfma(dims->variant, bf16_base(dims), dims->dk, dims->dv, tiles,
                                 pool_args(dims, pool), min_fill, st);
  return dl::launch_merge(dims->variant, bf16_base(dims), dims->dk, dims->dv, tiles, pool_args(dims, pool),
                          min_fill, st);
}

int dl_merge_on(const dl_dims* dims, const dl_pool* pool, int32_t min_fill, int32_t unit, void* stream) {
  int rc = check_dims(dims);
  if (rc != DL_OK) return rc;
  if (min_fill < DL_MERGE_DUE || min_fill > dims->log_len) return DL_EINVAL;
  if (unit != DL_UNIT_AUTO && unit != DL_UNIT_VALU && unit != DL_UNIT_MFMA) return DL_EINVAL;
  if (dims->batch == 0) return DL_OK;
  if ((rc = check_pool(pool, dims->variant)) != DL_OK) return rc;
  // a log is due when it holds L entries; the decode step folds it in the call that fills it
  if (min_fill == DL_MERGE_DUE) return DL_OK;
  return hip_status(launch_fold(dims, pool, min_fill, unit, static_cast<hipStream_t>(stream)));
}

int dl_merge(const dl_dims* dims, const dl_pool* pool, int32_t min_fill, void* stream) {
  return dl_merge_on(dims, pool, min_fill, DL_UNIT_AUTO, stream);
}

int dl_merge_unit(const dl_dims* dims) {
  const int rc = check_dims(dims);
  if (rc != DL_OK) return rc;
  return merge_on_mfma(dims, DL_UNIT_AUTO) ? DL_UNIT_MFMA : DL_UNIT_VALU;
}

int dl_eager_step(const dl_dims* dims, float* state, const dl_step_io* io, void* stream) {
  int rc = check_dims(dims);
  if (rc != DL_OK || dims->batch == 0) return rc;
  if (dims->base_dtype != DL_BASE_F32) return DL_EUNSUPPORTED;  // the eager state is fp32
  if ((rc = check_io(dims, io)) != DL_OK) return rc;
  if (state == nullptr) return DL_EINVAL;
  if (misaligned(state)) return DL_EALIGN;
  return hip_status(dl::launch_eager(dims->variant, dims->dk, dims->dv, dims->batch * dims->heads,
                                     dims->heads, state, step_args(io), static_cast<hipStream_t>(stream)));
}

int dl_prefill(const dl_dims* dims, const dl_pool* pool, const dl_prefill_io* io, void* stream) {
  int rc = check_dims(dims);
  if (rc != DL_OK) return rc;
  if (io == nullptr || io->tokens < 0) return DL_EINVAL;
  // the prefill kernels address one chunk's rows of a sequence (32 tokens x heads rows
  // of up to 512 bytes) with 32-bit offsets
  if (static_cast<int64_t>(dims->heads) * 32 * 512 > INT32_MAX) return DL_EINVAL;
  if (dims->batch == 0) return DL_OK;
  if ((rc = check_pool(pool, dims->variant)) != DL_OK) return rc;
  if (io->tokens > 0) {  // an empty prompt only folds: its pointers are not looked at
    if (!io->q || !io->k || !io->v || !io->decay || !io->out) return DL_EINVAL;
    const bool rwkv = dims->variant == DL_RWKV6;
    if (rwkv && (io->beta != nullptr || io->eta != nullptr || io->bonus == nullptr)) return DL_EUNSUPPORTED;
    if (!rwkv && ((io->beta == nullptr) == (io->eta == nullptr) || io->bonus != nullptr)) return DL_EUNSUPPORTED;
    if (io->eta != nullptr && !(io->eps >= 0.f)) return DL_EINVAL;
    if (misaligned(io->q) || misaligned(io->k) || misaligned(io->v) ||
        misaligned(io->decay, dims->variant == DL_GDN ? 4 : 16) || (io->bonus && misaligned(io->bonus)) ||
        misaligned(io->out, 4) || (io->beta && misaligned(io->beta, 4)) || (io->eta && misaligned(io->eta, 4)))
      return DL_EALIGN;
  }
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int tiles = dims->batch * dims->heads;
  // fold any pending log first: the prefill starts from the dense state in the base
  hipError_t e = launch_fold(dims, pool, 1, DL_UNIT_AUTO, st);
  if (e != hipSuccess || io->tokens == 0) return hip_status(e);
  const dl::PrefillArgs a{io->q, io->k, io->v, io->decay, io->beta, io->eta, io->bonus, io->out, io->eps, io->tokens};
  return hip_status(dl::launch_prefill(dims->variant, bf16_base(dims), dims->dk, dims->dv, tiles,
                                       pool_args(dims, pool), a, st));
}

const char* dl_status_string(int status) {
  switch (status) {
    case DL_OK: return "DL_OK: success";
    case DL_EINVAL: return "DL_EINVAL: invalid argument (null pointer, dims, log length or fill out of range)";
    case DL_EUNSUPPORTED: return "DL_EUNSUPPORTED: unsupported head size or variant/pointer combination";
    case DL_EALIGN: return "DL_EALIGN: a device pointer is not aligned as required";
    case DL_EHIP: return "DL_EHIP: the HIP runtime reported an error";
    default: return "unknown deltalog status";
  }
}

}  // extern "C"
