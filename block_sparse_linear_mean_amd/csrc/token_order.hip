// Token reordering: a 3-D Hilbert order of the video latent grid, and the row gather / scatter
// that applies it to Q, K, V (and undoes it on O).
//
// Method: reordering the tokens along a Hilbert curve makes the tokens of one 64-token block
// more alike, which raises the sparsity the block prediction finds ("2025稀疏注意力架构综述",
// section 11 SpargeAttn, the token-reordering remark).  The curve: Skilling's transform from
// axes to the transposed Hilbert index (J. Skilling, "Programming the Hilbert curve", AIP
// Conf. Proc. 707, 2004) on the cube of side 2^b that holds the (t, h, w) grid; cells are
// visited in increasing index.
//
// Design: the order depends only on the grid shape, so it is built once on the host (sorting
// T H W 64-bit keys) and uploaded by the caller.  Applying it is a pure row copy, HBM-bound:
// one thread per 16 bytes, rows of one head contiguous in the output, so every wavefront reads
// and writes whole rows (256 or 512 bytes at d = 128).
#include "sla_device.h"
#include "sla_host.h"

#include <algorithm>
#include <utility>
#include <vector>

namespace sla {

// Hilbert index of (c[0], c[1], c[2]) on the cube of side 2^bits (bits <= 21).
static uint64_t hilbert3(uint32_t c0, uint32_t c1, uint32_t c2, int bits) {
  uint32_t x[3] = {c0, c1, c2};
  // undo the excess work of the recursive construction, top level first
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1) {
    const uint32_t p = q - 1;
    for (int i = 0; i < 3; ++i) {
      if (x[i] & q) {
        x[0] ^= p;                       // invert the low bits of the first axis
      } else {
        const uint32_t t = (x[0] ^ x[i]) & p;
        x[0] ^= t;                       // exchange low bits with the first axis
        x[i] ^= t;
      }
    }
  }
  // Gray encode across the axes
  x[1] ^= x[0];
  x[2] ^= x[1];
  uint32_t flip = 0;
  for (uint32_t q = 1u << (bits - 1); q > 1; q >>= 1)
    if (x[2] & q) flip ^= q - 1;
  for (int i = 0; i < 3; ++i) x[i] ^= flip;
  // read the transposed index level by level, axis 0 first
  uint64_t h = 0;
  for (int level = bits - 1; level >= 0; --level)
    for (int i = 0; i < 3; ++i) h = (h << 1) | ((x[i] >> level) & 1u);
  return h;
}

// out[b,h,n] = x[b,h,order[n]] (gather) or out[b,h,order[n]] = x[b,h,n] (scatter) for n < n_order;
// rows n >= n_order are copied in place.  One thread per 16-byte chunk of a row.
template <int CHUNKS>
__global__ __launch_bounds__(256) void permute_rows_kernel(const unsigned char* __restrict__ x, int64_t sB,
                                                           int64_t sH, int64_t sN, int H, int N,
                                                           const int* __restrict__ order, int n_order,
                                                           int scatter, unsigned char* __restrict__ out) {
  constexpr int kRows = 256 / CHUNKS;            // rows per workgroup
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int n = blockIdx.x * kRows + threadIdx.x / CHUNKS, c = threadIdx.x % CHUNKS;
  if (n >= N) return;
  int src = n, dst = n;
  if (n < n_order) {
    const int o = order[n];
    const bool ok = unsigned(o) < unsigned(n_order);    // an entry out of range is left in place
    if (scatter) dst = ok ? o : n;
    else src = ok ? o : n;
  }
  const f32x4 v = *reinterpret_cast<const f32x4*>(x + int64_t(b) * sB + int64_t(h) * sH + int64_t(src) * sN + 16 * c);
  *reinterpret_cast<f32x4*>(out + ((int64_t(bh) * N + dst) * CHUNKS + c) * 16) = v;
}

}  // namespace sla

extern "C" sla_status sla_hilbert_order(int32_t T, int32_t H, int32_t W, int32_t* order) {
  using namespace sla;
  if (order == nullptr) return SLA_ERR_NULL;
  if (T < 1 || H < 1 || W < 1) return SLA_ERR_SHAPE;
  const int64_t n = int64_t(T) * H * W;
  if (n > int64_t(INT32_MAX) || std::max({T, H, W}) > (1 << 21)) return SLA_ERR_RANGE;
  int bits = 1;
  while ((int64_t(1) << bits) < std::max({T, H, W})) ++bits;
  std::vector<std::pair<uint64_t, int32_t>> keys;
  keys.reserve(size_t(n));
  for (int32_t t = 0; t < T; ++t)
    for (int32_t h = 0; h < H; ++h)
      for (int32_t w = 0; w < W; ++w)
        keys.emplace_back(hilbert3(uint32_t(t), uint32_t(h), uint32_t(w), bits), int32_t((int64_t(t) * H + h) * W + w));
  std::sort(keys.begin(), keys.end());            // keys are distinct: the index is a bijection
  for (int64_t i = 0; i < n; ++i) order[i] = keys[size_t(i)].second;
  return SLA_OK;
}

extern "C" sla_status sla_permute_rows(const sla_tensor* x, const int32_t* order, int32_t n_order, int32_t inverse,
                                       void* out, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(x);
  if (st != SLA_OK) return st;
  if (out == nullptr || (order == nullptr && n_order > 0)) return SLA_ERR_NULL;
  if (n_order < 0 || n_order > x->N) return SLA_ERR_RANGE;
  if (!aligned16(out)) return SLA_ERR_ALIGN;
  if (out == x->ptr) return SLA_ERR_UNSUPPORTED;   // not in place
  const int row_bytes = x->d * (x->dtype == SLA_BF16 ? 2 : 4);
  const int chunks = row_bytes / 16;
  const int rows_per_wg = 256 / chunks;
  const int eb = x->dtype == SLA_BF16 ? 2 : 4;
  const dim3 grid(uint32_t((x->N + rows_per_wg - 1) / rows_per_wg), uint32_t(x->B * x->H));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned char* xp = static_cast<const unsigned char*>(x->ptr);
  unsigned char* op = static_cast<unsigned char*>(out);
  const int64_t sB = x->sB * eb, sH = x->sH * eb, sN = x->sN * eb;
#define SLA_PERM_LAUNCH(C) \
  permute_rows_kernel<C><<<grid, 256, 0, s>>>(xp, sB, sH, sN, x->H, x->N, order, n_order, inverse ? 1 : 0, op)
  switch (chunks) {
    case 8: SLA_PERM_LAUNCH(8); break;     // bf16 d64
    case 16: SLA_PERM_LAUNCH(16); break;   // bf16 d128, fp32 d64
    case 32: SLA_PERM_LAUNCH(32); break;   // fp32 d128
    default: return SLA_ERR_UNSUPPORTED;
  }
#undef SLA_PERM_LAUNCH
  return launch_status();
}
