// Prediction step: block mean pooling of Q and K, pooled scores and their row softmax.
//
// Method: mean-pool Q and K over 64-token blocks and score pooled blocks against each
// other, then softmax each row ("2025稀疏注意力架构综述", section 11 SpargeAttn, the
// prediction formulas; SLA analysis page for arXiv 2509.24006, mean-pooled compressed
// prediction that turns the N x N problem into an (N/b)^2 classification).
//
// Both passes are small next to attention: pooling is HBM-bound (Q and K read once),
// scoring is fp64 matrix-core work on the pooled vectors.  The classification ranks these
// scores, so they are computed in fp64 from the fp32 pooled vectors and rounded once:
// each stored score is the correctly rounded fp32 of a near-exact fp64 dot product.
#include <type_traits>

#include "sla_device.h"
#include "sla_host.h"

namespace sla {

// One workgroup pools kPoolBlocks consecutive blocks of one (b, h) of Q or K (grid y runs over
// the Q heads, then the nhk K heads; nhk = 0 when the key block means come from the key-state
// pass): 256 threads; each thread owns 8 consecutive features of one
// row group, issues all of its 16-byte loads before summing, and sums in fp64 (exact for bf16
// inputs); partial sums are combined in a fixed order, so the result does not depend on
// scheduling.
constexpr int kPoolBlocks = 1;   // one block per workgroup: the most loads in flight chip-wide

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ q, int64_t qsB, int64_t qsH, int64_t qsN,
                                                   int Hq, const T* __restrict__ k, int64_t ksB, int64_t ksH,
                                                   int64_t ksN, int Hkv, int nhk, int nb, int n_valid,
                                                   float* __restrict__ qout, float* __restrict__ kout) {
  constexpr int kTpr = D / 8;          // threads per row
  constexpr int kRpp = 256 / kTpr;     // rows per pass
  constexpr int kPasses = kBlock / kRpp;
  const int y = blockIdx.y;
  const int B = gridDim.y / (Hq + nhk);
  const bool is_q = y < B * Hq;
  const int bh = is_q ? y : y - B * Hq;            // (b, h) index within its tensor
  const int H = is_q ? Hq : Hkv;
  const int h = bh % H, b = bh / H;
  const T* x = is_q ? q : k;
  const int64_t sB = is_q ? qsB : ksB, sH = is_q ? qsH : ksH, sN = is_q ? qsN : ksN;
  float* out = is_q ? qout : kout;
  const int t = threadIdx.x;
  const int cg = t % kTpr, rg = t / kTpr;
  __shared__ double part[kRpp][D + 1];
  for (int ib = 0; ib < kPoolBlocks; ++ib) {
    const int i = blockIdx.x * kPoolBlocks + ib;
    if (i >= nb) break;
    const int rows = min(kBlock, n_valid - kBlock * i);
    const T* base = x + int64_t(b) * sB + int64_t(h) * sH + int64_t(kBlock * i) * sN + cg * 8;
    float v[kPasses][8];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int r = rg + p * kRpp;
      In<T>::load8_f32(base + int64_t(min(r, rows - 1)) * sN, v[p]);   // in-bounds stand-in for padding
    }
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      if (rg + p * kRpp < rows)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += double(v[p][e]);
    __syncthreads();                     // the previous block's partial sums have been read
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
}

// Group sums of the pooled queries: qsum[b,g,i,r] = sum over the group's heads h (ascending) of
// q_pool[b,h,i,r], in fp64 (exact for the fp32 pooled values in practice).  One thread per element.
__global__ __launch_bounds__(256) void qsum_kernel(const float* __restrict__ qpool, int Hq, int Hkv, int nb, int d,
                                                   double* __restrict__ qsum) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int bg = blockIdx.y, b = bg / Hkv, g = bg % Hkv, G = Hq / Hkv;
  if (e >= int64_t(nb) * d) return;
  double s = 0.0;
  for (int hh = 0; hh < G; ++hh) s += double(qpool[(int64_t(b) * Hq + g * G + hh) * nb * d + e]);
  qsum[int64_t(bg) * nb * d + e] = s;
}

// Pooled scores on the fp64 matrix cores: one 64 (i) x 64 (j) tile of one score matrix per
// workgroup, each wavefront a 32 x 32 quarter as 2 x 2 products of the 16x16x4 fp64 instruction.
// scores[b,s,i,j] = fp32(scale * sum_r qv[i,r] * kpool[j,r]) with the sum in fp64; qv is the
// fp64 group sum of the pooled queries (QSUM: qsum_kernel's output, one row per (b, s)) or, for
// a single query head per score matrix (no group sum, or groups of one head), that head's pooled
// queries: s is then the query head.  The operands come straight from global memory (the pooled
// vectors are small and stay in cache): in 16-feature chunk c, lane group g = lane / 16 holds
// features 16 c + 4 g .. 16 c + 4 g + 3 of its row and feeds them to four consecutive k-steps,
// so one 16-byte load per row and chunk serves four instructions; A and B use the same feature
// order, so every product pairs matching features.  The sum is taken in a different order from
// the oracle's, so the fp64 values may differ in their last bits; rounded to fp32 they agree
// except on an fp32 rounding boundary.
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
constexpr int kScI = 64, kScJ = 64;

template <int D, bool QSUM>
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ qpool,
                                                     const float* __restrict__ kpool, int Hq, int Hkv,
                                                     int Hs, int nb, int group_sum, int causal,
                                                     double scale, const double* __restrict__ qsum,
                                                     float* __restrict__ scores) {
  constexpr int kC = D / 16;                     // 16-feature chunks
  const int bs = blockIdx.z;
  const int b = bs / Hs, s = bs % Hs;
  const int G = Hq / Hkv;
  const int g = group_sum ? s : s / G;
  const int i0 = blockIdx.y * kScI, j0 = blockIdx.x * kScJ;
  const int t = threadIdx.x;
  float* out = scores + int64_t(bs) * nb * nb;

  if (causal && j0 > i0 + kScI - 1) {   // the whole tile lies above the diagonal
    for (int e = t; e < kScI * kScJ; e += 256) {
      const int ii = i0 + e / kScJ, jj = j0 + e % kScJ;
      if (ii < nb && jj < nb) out[int64_t(ii) * nb + jj] = -__builtin_inff();
    }
    return;
  }

  const int lane = t % kWave, w = t / kWave;
  const int li = lane % 16, lg = lane / 16;
  const int wi = i0 + 32 * (w / 2), wj = j0 + 32 * (w % 2);

  // a[tt][c]: features 16 c + 4 lg + 0..3 of query row wi + 16 tt + li; kv[uu][c] likewise for key
  // row wj + 16 uu + li (rows past nb read row nb - 1 and are not stored); all loads are issued
  // before the first product
  typedef typename std::conditional<QSUM, f64x4, f32x4>::type AVec;
  AVec a[2][kC];
  f32x4 kv[2][kC];
  const float* kp[2];
  const float* qpf[2];
  const double* qpd[2];
#pragma unroll
  for (int uu = 0; uu < 2; ++uu)
    kp[uu] = kpool + ((int64_t(b) * Hkv + g) * nb + min(wj + 16 * uu + li, nb - 1)) * D + 4 * lg;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int ii = min(wi + 16 * tt + li, nb - 1);
    qpd[tt] = QSUM ? qsum + (int64_t(bs) * nb + ii) * D + 4 * lg : nullptr;
    qpf[tt] = QSUM ? nullptr : qpool + ((int64_t(b) * Hq + s) * nb + ii) * D + 4 * lg;
  }
  if constexpr (QSUM) {
    // operand-major order (measured faster here with the fp64 group sums)
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int c = 0; c < kC; ++c) kv[uu][c] = *reinterpret_cast<const f32x4*>(kp[uu] + 16 * c);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        const f64x2 lo = *reinterpret_cast<const f64x2*>(qpd[tt] + 16 * c);
        const f64x2 hi = *reinterpret_cast<const f64x2*>(qpd[tt] + 16 * c + 2);
        a[tt][c] = f64x4{lo[0], lo[1], hi[0], hi[1]};
      }
  } else {
    // chunk-major order: the products of chunk c wait only for the loads of chunks 0 .. c
    // (wan13b: 23.7 -> 21.1 us)
#pragma unroll
    for (int c = 0; c < kC; ++c) {
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) kv[uu][c] = *reinterpret_cast<const f32x4*>(kp[uu] + 16 * c);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) a[tt][c] = *reinterpret_cast<const f32x4*>(qpf[tt] + 16 * c);
    }
  }

  __builtin_amdgcn_sched_barrier(0);           // keep every load ahead of the products

  f64x4 acc[2][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) acc[tt][uu] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int c = 0; c < kC; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
          acc[tt][uu] = __builtin_amdgcn_mfma_f64_16x16x4f64(double(a[tt][c][m]), double(kv[uu][c][m]), acc[tt][uu],
                                                            0, 0, 0);

  // lane holds rows wi + 16 tt + 4 e + lg, column wj + 16 uu + li of the tile in acc[tt][uu][e]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int jj = wj + 16 * uu + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = wi + 16 * tt + 4 * e + lg;
        if (ii < nb && jj < nb)
          out[int64_t(ii) * nb + jj] = (causal && jj > ii) ? -__builtin_inff() : float(acc[tt][uu][e] * scale);
      }
    }
}

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
static void launch_pool(const sla_tensor* q, const sla_tensor* k, int n_valid, bool pool_k, float* qout,
                        float* kout, hipStream_t st) {
  const int nb = q->N / kBlock;
  const int nhk = pool_k ? k->H : 0;
  dim3 grid((nb + kPoolBlocks - 1) / kPoolBlocks, q->B * (q->H + nhk));
  const T* qp = static_cast<const T*>(q->ptr);
  const T* kp = static_cast<const T*>(k->ptr);
  if (q->d == 128)
    pool_kernel<T, 128><<<grid, 256, 0, st>>>(qp, q->sB, q->sH, q->sN, q->H, kp, k->sB, k->sH, k->sN, k->H, nhk,
                                              nb, n_valid, qout, kout);
  else
    pool_kernel<T, 64><<<grid, 256, 0, st>>>(qp, q->sB, q->sH, q->sN, q->H, kp, k->sB, k->sH, k->sN, k->H, nhk,
                                             nb, n_valid, qout, kout);
}

}  // namespace sla

extern "C" size_t sla_pool_scores_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                                                  int32_t group_sum) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || N < sla::kBlock || N % sla::kBlock || (d != 64 && d != 128)) return 0;
  return (group_sum && Hq / Hkv > 1) ? size_t(B) * Hkv * (N / sla::kBlock) * d * sizeof(double) : 0;
}

extern "C" sla_status sla_pool_scores(const sla_tensor* q, const sla_tensor* k, int32_t n_valid,
                                      int32_t group_sum, int32_t causal, float scale, int32_t pooled, float* q_pool,
                                      float* k_pool, float* scores, float* probs, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if (!same_geometry(q, k) || q->H % k->H != 0) return SLA_ERR_SHAPE;
  if (q_pool == nullptr || k_pool == nullptr) return SLA_ERR_NULL;
  if (scores == nullptr && probs != nullptr) return SLA_ERR_NULL;
  if (!aligned16(q_pool) || !aligned16(k_pool)) return SLA_ERR_ALIGN;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale)) return SLA_ERR_RANGE;
  if (pooled < 0 || pooled > 3) return SLA_ERR_RANGE;
  const size_t need = scores ? sla_pool_scores_workspace_bytes(q->B, q->H, k->H, q->N, q->d, group_sum) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))) return SLA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = q->N / kBlock;
  const bool pool_q = !(pooled & SLA_POOLED_Q), pool_k = !(pooled & SLA_POOLED_K);
  if (pool_q) {
    if (q->dtype == SLA_BF16) launch_pool<bf16raw>(q, k, n_valid, pool_k, q_pool, k_pool, s);
    else launch_pool<float>(q, k, n_valid, pool_k, q_pool, k_pool, s);
  } else if (pool_k) {
    // the key block means only: the same kernel with K in the place of Q
    if (q->dtype == SLA_BF16) launch_pool<bf16raw>(k, k, n_valid, false, k_pool, k_pool, s);
    else launch_pool<float>(k, k, n_valid, false, k_pool, k_pool, s);
  }
  if (scores == nullptr) return launch_status();   // pooling only
  const int Hs = group_sum ? k->H : q->H;
  const double* qsum = nullptr;
  if (group_sum && q->H / k->H > 1) {             // the group sums once, instead of in every tile
    double* qs = static_cast<double*>(workspace);
    qsum_kernel<<<dim3(uint32_t((int64_t(nb) * q->d + 255) / 256), uint32_t(q->B * k->H)), 256, 0, s>>>(
        q_pool, q->H, k->H, nb, q->d, qs);
    qsum = qs;
  }
  dim3 grid((nb + kScJ - 1) / kScJ, (nb + kScI - 1) / kScI, q->B * Hs);
  const int gs = group_sum ? 1 : 0, ca = causal ? 1 : 0;
  if (q->d == 128) {
    if (qsum) scores_kernel<128, true><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, gs, ca, double(scale), qsum, scores);
    else scores_kernel<128, false><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, gs, ca, double(scale), qsum, scores);
  } else {
    if (qsum) scores_kernel<64, true><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, gs, ca, double(scale), qsum, scores);
    else scores_kernel<64, false><<<grid, 256, 0, s>>>(q_pool, k_pool, q->H, k->H, Hs, nb, gs, ca, double(scale), qsum, scores);
  }
  if (probs != nullptr) probs_kernel<<<dim3(q->B * Hs * nb), 64, 0, s>>>(scores, nb, probs);
  return launch_status();
}

namespace sla {

// Smooth-K shift of one (batch, KV head): the mean of its valid key rows, taken from the block
// means, mu[r] = sum_j c_j kpool[j][r] / n_valid with c_j the valid rows of block j (SLA analysis
// page: the open-source code zero-means K).  One workgroup per (8 features, head); each thread
// sums a strided set of blocks in fp64, then a fixed-order LDS tree; one rounding to fp32.
__global__ __launch_bounds__(256) void key_mean_kernel(const float* __restrict__ kpool, int nb, int d,
                                                       int n_valid, float* __restrict__ mu) {
  const int bg = blockIdx.y, r0 = 8 * blockIdx.x, t = threadIdx.x;
  double s[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) s[m] = 0.0;
  for (int j = t; j < nb; j += 256) {
    const double c = double(min(kBlock, n_valid - kBlock * j));    // >= 1: at most one partial block
    const float* p = kpool + (int64_t(bg) * nb + j) * d + r0;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[m] += c * double(a[m]);
      s[4 + m] += c * double(b[m]);
    }
  }
  __shared__ double red[256][9];
#pragma unroll
  for (int m = 0; m < 8; ++m) red[t][m] = s[m];
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) {
#pragma unroll
      for (int m = 0; m < 8; ++m) red[t][m] += red[t + w][m];
    }
    __syncthreads();
  }
  if (t < 8) mu[int64_t(bg) * d + r0 + t] = float(red[0][t] / double(n_valid));
}

}  // namespace sla

extern "C" sla_status sla_key_mean(const float* k_pool, int32_t B, int32_t Hkv, int32_t nkb, int32_t d,
                                   int32_t n_valid, float* k_mean, void* stream) {
  using namespace sla;
  if (k_pool == nullptr || k_mean == nullptr) return SLA_ERR_NULL;
  if (B < 1 || Hkv < 1 || nkb < 1 || nkb > (1 << 24) || (d != 64 && d != 128)) return SLA_ERR_SHAPE;
  sla_status st = check_valid_len(n_valid, nkb * kBlock);
  if (st != SLA_OK) return st;
  if (!aligned16(k_pool) || !aligned16(k_mean)) return SLA_ERR_ALIGN;
  key_mean_kernel<<<dim3(d / 8, B * Hkv), 256, 0, static_cast<hipStream_t>(stream)>>>(k_pool, nkb, d, n_valid,
                                                                                       k_mean);
  return launch_status();
}
