// Marginal aggregation: per map row, the sums S = sum_j H_j and u = sum_j z_j over the
// row's marginal key blocks, which the linear branch of the attention epilogue reads
// as phi(q)^T S / (phi(q) . u).
//
// Method: marginal pairs get linear attention through per-key-block states (SLA
// analysis page for arXiv 2509.24006: critical pairs FlashAttention, marginal pairs
// linear attention at O(N d^2)).
//
// Design: one workgroup per (map row, 1024-float slice of the d x d state); every
// thread sums one float4 column over the row's marginal list in ascending order, so
// results are deterministic.  The reads are gathers of whole per-block states and are
// served mostly from L2 / the infinity cache, since neighbouring query blocks share
// most of their marginal blocks.
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

template <int D>
__global__ __launch_bounds__(256) void marginal_states_kernel(const float* __restrict__ H,
                                                              const float* __restrict__ z, int Hq, int Hkv,
                                                              int Hs, int nqb, int nkb, int group_map,
                                                              const int* __restrict__ rowptr,
                                                              const int* __restrict__ idx, float* __restrict__ S,
                                                              float* __restrict__ u) {
  const int64_t r = blockIdx.x;
  const int slice = blockIdx.y;
  const int64_t bs = r / nqb;
  const int b = int(bs / Hs), s = int(bs % Hs);
  const int g = group_map ? s : s / (Hq / Hkv);
  const int64_t hbase = (int64_t(b) * Hkv + g) * nkb;
  const int beg = rowptr[r], end = rowptr[r + 1];
  const int t = threadIdx.x;
  const int64_t e = int64_t(slice) * 1024 + 4 * t;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int p = beg; p < end; ++p) {
    const int64_t j = idx[p];
    if (uint64_t(j) >= uint64_t(nkb)) continue;   // malformed list entry
    acc += *reinterpret_cast<const f32x4*>(H + (hbase + j) * D * D + e);
  }
  *reinterpret_cast<f32x4*>(S + r * D * D + e) = acc;
  if (slice == 0 && t < D / 4) {
    f32x4 zs = {0.f, 0.f, 0.f, 0.f};
    for (int p = beg; p < end; ++p) {
      const int64_t j = idx[p];
      if (uint64_t(j) >= uint64_t(nkb)) continue;
      zs += *reinterpret_cast<const f32x4*>(z + (hbase + j) * D + 4 * t);
    }
    *reinterpret_cast<f32x4*>(u + r * D + 4 * t) = zs;
  }
}

sla_status launch_marginal_states(const float* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const int* rowptr, const int* idx, float* S, float* u,
                                  hipStream_t st) {
  const int Hs = group_map ? Hkv : Hq;
  const int64_t rows = int64_t(B) * Hs * nqb;
  dim3 grid(uint32_t(rows), d * d / 1024);
  if (d == 128)
    marginal_states_kernel<128><<<grid, 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, rowptr, idx, S, u);
  else
    marginal_states_kernel<64><<<grid, 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, rowptr, idx, S, u);
  return launch_status();
}

}  // namespace sla

extern "C" sla_status sla_marginal_states(const float* H, const float* z, int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t nqb, int32_t nkb, int32_t d, int32_t group_map,
                                          const int32_t* marg_rowptr, const int32_t* marg_idx, float* S, float* u,
                                          void* stream) {
  using namespace sla;
  if (H == nullptr || z == nullptr || marg_rowptr == nullptr || marg_idx == nullptr || S == nullptr ||
      u == nullptr)
    return SLA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || nqb < 1 || nkb < 1) return SLA_ERR_SHAPE;
  if (d != 64 && d != 128) return SLA_ERR_UNSUPPORTED;
  if (!aligned16(H) || !aligned16(z) || !aligned16(S) || !aligned16(u)) return SLA_ERR_ALIGN;
  return launch_marginal_states(H, z, B, Hq, Hkv, nqb, nkb, d, group_map ? 1 : 0, marg_rowptr, marg_idx, S, u,
                                static_cast<hipStream_t>(stream));
}
