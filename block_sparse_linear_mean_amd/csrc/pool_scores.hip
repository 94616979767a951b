// Prediction step: block mean pooling of Q and K, pooled scores and their row softmax.
//
// Method: mean-pool Q and K over 64-token blocks and score pooled blocks against each
// other, then softmax each row ("2025稀疏注意力架构综述", section 11 SpargeAttn, the
// prediction formulas; SLA analysis page for arXiv 2509.24006, mean-pooled compressed
// prediction that turns the N x N problem into an (N/b)^2 classification).
//
// Both passes are small next to attention: pooling is HBM-bound (Q and K read once),
// scoring is fp64 FMA work on the pooled vectors.  The classification ranks these
// scores, so they are computed in fp64 from the fp32 pooled vectors and rounded once:
// each stored score is the correctly rounded fp32 of a near-exact fp64 dot product.
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

// One workgroup pools one (b, h, block i): 256 threads, each loads 8 consecutive
// features of a row per pass and sums in fp64 (exact for bf16 inputs); partial sums
// are combined in a fixed order, so the result does not depend on scheduling.
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ x, int64_t sB, int64_t sH,
                                                   int64_t sN, int H, int nb, int n_valid,
                                                   float* __restrict__ out) {
  constexpr int kTpr = D / 8;          // threads per row
  constexpr int kRpp = 256 / kTpr;     // rows per pass
  constexpr int kPasses = kBlock / kRpp;
  const int i = blockIdx.x;
  const int bh = blockIdx.y;
  const int h = bh % H, b = bh / H;
  const int t = threadIdx.x;
  const int cg = t % kTpr, rg = t / kTpr;
  const int rows = min(kBlock, n_valid - kBlock * i);
  const T* base = x + int64_t(b) * sB + int64_t(h) * sH + int64_t(kBlock * i) * sN + cg * 8;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int r = rg + p * kRpp;
    if (r < rows) {
      float v[8];
      In<T>::load8_f32(base + int64_t(r) * sN, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += double(v[e]);
    }
  }
  __shared__ double part[kRpp][D + 1];
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][cg * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
#pragma unroll 4
    for (int r = 0; r < kRpp; ++r) s += part[r][t];
    out[(int64_t(bh) * nb + i) * D + t] = float(s / double(rows));
  }
}

// Pooled scores, one 64 x 64 tile of one score matrix per workgroup.
// scores[b,s,i,j] = fp32(scale * sum_r qsum[i,r] * kpool[j,r]) with a sequential fp64
// FMA chain over r; qsum sums the group's pooled queries in fp64 when group_sum is set.
template <int D>
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ qpool,
                                                     const float* __restrict__ kpool, int Hq, int Hkv,
                                                     int Hs, int nb, int group_sum, int causal,
                                                     double scale, float* __restrict__ scores) {
  const int bs = blockIdx.z;
  const int b = bs / Hs, s = bs % Hs;
  const int G = Hq / Hkv;
  const int g = group_sum ? s : s / G;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int tx = t % 16, ty = t / 16;
  float* out = scores + int64_t(bs) * nb * nb;

  if (causal && j0 > i0 + 63) {   // the whole tile lies above the diagonal
    for (int e = t; e < 64 * 64; e += 256) {
      const int ii = i0 + e / 64, jj = j0 + e % 64;
      if (ii < nb && jj < nb) out[int64_t(ii) * nb + jj] = -__builtin_inff();
    }
    return;
  }

  __shared__ double qs[64][33];
  __shared__ float ks[64][33];
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;

  const int gh0 = group_sum ? g * G : s;
  const int ngh = group_sum ? G : 1;
  for (int r0 = 0; r0 < D; r0 += 32) {
    for (int e = t; e < 64 * 32; e += 256) {
      const int row = e / 32, col = e % 32;
      const int ii = i0 + row, jj = j0 + row;
      double qv = 0.0;
      if (ii < nb) {
        for (int hh = 0; hh < ngh; ++hh)
          qv += double(qpool[((int64_t(b) * Hq + gh0 + hh) * nb + ii) * D + r0 + col]);
      }
      qs[row][col] = qv;
      ks[row][col] = jj < nb ? kpool[((int64_t(b) * Hkv + g) * nb + jj) * D + r0 + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      double qa[4], kb[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[a] = qs[ty + 16 * a][r];
#pragma unroll
      for (int c = 0; c < 4; ++c) kb[c] = double(ks[tx + 16 * c][r]);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[a][c] = __fma_rn(qa[a], kb[c], acc[a][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int ii = i0 + ty + 16 * a;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int jj = j0 + tx + 16 * c;
      if (ii < nb && jj < nb) {
        const float v = (causal && jj > ii) ? -__builtin_inff() : float(acc[a][c] * scale);
        out[int64_t(ii) * nb + jj] = v;
      }
    }
  }
}

// Row softmax of the score rows (diagnostic output): one wavefront per row.
__global__ __launch_bounds__(64) void probs_kernel(const float* __restrict__ scores, int nb,
                                                   float* __restrict__ probs) {
  const int64_t row = blockIdx.x;
  const float* s = scores + row * nb;
  float* p = probs + row * nb;
  const int lane = threadIdx.x;
  float m = -__builtin_inff();
  for (int j = lane; j < nb; j += 64) m = fmaxf(m, s[j]);
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float sum = 0.f;
  for (int j = lane; j < nb; j += 64) sum += __expf(s[j] - m);
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float inv = 1.f / sum;
  for (int j = lane; j < nb; j += 64) p[j] = __expf(s[j] - m) * inv;
}

template <typename T>
static void launch_pool(const sla_tensor* x, int n_valid, float* out, hipStream_t st) {
  const int nb = x->N / kBlock;
  dim3 grid(nb, x->B * x->H);
  const T* p = static_cast<const T*>(x->ptr);
  if (x->d == 128)
    pool_kernel<T, 128><<<grid, 256, 0, st>>>(p, x->sB, x->sH, x->sN, x->H, nb, n_valid, out);
  else
    pool_kernel<T, 64><<<grid, 256, 0, st>>>(p, x->sB, x->sH, x->sN, x->H, nb, n_valid, out);
}

}  // namespace sla

extern "C" sla_status sla_pool_scores(const sla_tensor* q, const sla_tensor* k, int32_t n_valid,
                                      int32_t group_sum, int32_t causal, float scale, float* q_pool,
                                      float* k_pool, float* scores, float* probs, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if (!same_geometry(q, k) || q->H % k->H != 0) return SLA_ERR_SHAPE;
  if (q_pool == nullptr || k_pool == nullptr || scores == nullptr) return SLA_ERR_NULL;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale)) return SLA_ERR_RANGE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = q->N / kBlock;
  if (q->dtype == SLA_BF16) {
    launch_pool<bf16raw>(q, n_valid, q_pool, s);
    launch_pool<bf16raw>(k, n_valid, k_pool, s);
  } else {
    launch_pool<float>(q, n_valid, q_pool, s);
    launch_pool<float>(k, n_valid, k_pool, s);
  }
  const int Hs = group_sum ? k->H : q->H;
  const int tiles = (nb + 63) / 64;
  dim3 grid(tiles, tiles, q->B * Hs);
  if (q->d == 128)
    scores_kernel<128><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, group_sum ? 1 : 0,
                                            causal ? 1 : 0, double(scale), scores);
  else
    scores_kernel<64><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, group_sum ? 1 : 0,
                                           causal ? 1 : 0, double(scale), scores);
  if (probs != nullptr) probs_kernel<<<dim3(q->B * Hs * nb), 64, 0, s>>>(scores, nb, probs);
  return launch_status();
}
