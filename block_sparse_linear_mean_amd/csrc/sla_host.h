// Host-side helpers shared by the libsla entry points: argument validation and launch checks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sla.h"

namespace sla {

// Key blocks per fp32 partial state when summing the linear states over all keys: the shortest
// run for which all the runs fit in one wave of workgroups, two per compute unit (512 in all: the
// kernel's occupancy), since a second, nearly empty wave would double the pass; at least 4 blocks
// (each run writes a d x d fp32 partial that the fixed-order final sum reads again) and at most 32.
// Depends on the shapes only, so the partial sums and their order are reproducible.
inline int kv_sum_run(int64_t nb, int64_t heads) {
  int64_t r = (nb * heads + 511) / 512;
  while (r < 32 && heads * ((nb + r - 1) / r) > 512) ++r;
  return int(r < 4 ? 4 : (r > 32 ? 32 : r));
}

inline int elem_bytes(int32_t dtype) { return dtype == SLA_BF16 ? 2 : 4; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates one [B, H, N, d] input descriptor (see the conventions in sla.h).
inline sla_status check_tensor(const sla_tensor* t) {
  if (t == nullptr || t->ptr == nullptr) return SLA_ERR_NULL;
  if (t->dtype != SLA_BF16 && t->dtype != SLA_F32) return SLA_ERR_UNSUPPORTED;
  if (t->B < 1 || t->H < 1 || t->N < SLA_BLOCK || t->N % SLA_BLOCK != 0) return SLA_ERR_SHAPE;
  if (t->d != 64 && t->d != 128) return SLA_ERR_UNSUPPORTED;
  if (t->N / SLA_BLOCK > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  if (t->sN < t->d || t->sH < 1 || t->sB < 1) return SLA_ERR_SHAPE;
  // the attention kernel's tile copies address rows through 32-bit per-lane byte offsets
  if (t->sN > SLA_MAX_ROW_STRIDE) return SLA_ERR_UNSUPPORTED;
  const int64_t eb = elem_bytes(t->dtype);
  if (!aligned16(t->ptr) || (t->sN * eb) % 16 || (t->sH * eb) % 16 || (t->sB * eb) % 16)
    return SLA_ERR_ALIGN;
  return SLA_OK;
}

inline bool same_geometry(const sla_tensor* a, const sla_tensor* b) {
  return a->dtype == b->dtype && a->B == b->B && a->N == b->N && a->d == b->d;
}

inline sla_status check_valid_len(int32_t n_valid, int32_t N) {
  if (n_valid <= N - SLA_BLOCK || n_valid > N) return SLA_ERR_RANGE;
  return SLA_OK;
}

inline sla_status launch_status() {
  return hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_HIP;
}

// Key blocks touched by a sliding window of w tokens on either side of the diagonal block.
inline int32_t window_reach(int32_t w) { return w > 0 ? (w + SLA_BLOCK - 2) / SLA_BLOCK : -1; }

}  // namespace sla
