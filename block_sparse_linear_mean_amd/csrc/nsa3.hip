// NSA with its three parallel branches: compressed tokens, selected blocks, sliding window.
//
// Method ("Sparse Attention 方法综述", section 2 NSA and its key-parameter table): a query attends
// in parallel to (1) compressed tokens, each summarising a window of 32 keys taken every 16 keys,
// which gives a cheap global view; (2) the top 16 key blocks of 64 tokens its GQA group selected;
// (3) the last 512 tokens; the three outputs are merged.  Here a compressed token is the mean of
// its window, each branch is its own softmax attention, and the merge is a per-token gated sum
// O = sum_b sigmoid(q . w_b) O_b with caller weights w_b per head (zero weights: every gate 1/2).
//
// Design: the three branches are three passes of the selected-block attention kernel over
// explicit block lists (so every pass keeps its copy pipeline; one workgroup per query block and
// query head, the heads of a GQA group back to back on one XCD): the selection map from
// sla_block_map (no window), a
// generated window list (blocks i - 8 .. i, token-level band mask in the kernel) and a generated
// list of compressed-token blocks (a causal limit on the window end).  Compression is one HBM
// pass over K and V; the gated merge one pass over the three fp32 branch outputs.
#include "sla_device.h"
#include "sla_host.h"

#include <algorithm>

namespace sla {

sla_status launch_causal_pass(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int n_valid,
                              int n_keys, float scale, int window, int cmp_block, int cmp_stride, const int* rowptr,
                              const int* idx, const uint8_t* flags, float* out, hipStream_t st);

// Compressed tokens: out[b,g,m,:] = mean of rows m * stride .. m * stride + block - 1, for m < M;
// rows M .. Mpad - 1 are zero.  One thread per (token m, 8 features), fp32 sums, one rounding.
template <typename T, int D>
__global__ __launch_bounds__(256) void compress_kernel(const T* __restrict__ x, int64_t sB, int64_t sH, int64_t sN,
                                                       int H, int M, int Mpad, int block, int stride,
                                                       T* __restrict__ out) {
  constexpr int kC = D / 8;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int m = e / kC, c = e % kC;
  if (m >= Mpad) return;
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  if (m < M) {
    const T* src = x + int64_t(b) * sB + int64_t(h) * sH + int64_t(m) * stride * sN + 8 * c;
    for (int r = 0; r < block; ++r) {
      float v[8];
      In<T>::load8_f32(src + int64_t(r) * sN, v);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += v[u];
    }
    const float inv = 1.f / float(block);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] *= inv;
  }
  T* dst = out + (int64_t(bh) * Mpad + m) * D + 8 * c;
  if constexpr (sizeof(T) == 2) {
    f32x8 f;
#pragma unroll
    for (int u = 0; u < 8; ++u) f[u] = acc[u];
    *reinterpret_cast<bf16x8*>(dst) = cvt8(f);
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// Window lists: row r = (bg, i) holds blocks i - min(i, reach) .. i (flag bit 1).  Row offsets in
// closed form: row i of a head starts at P(i) = sum over i' < i of (min(i', reach) + 1).
__device__ __forceinline__ int64_t window_prefix(int64_t i, int64_t reach) {
  const int64_t full = i < reach + 1 ? i : reach + 1;
  int64_t s = full * (full + 1) / 2;
  if (i > reach + 1) s += (i - reach - 1) * (reach + 1);
  return s;
}
__global__ __launch_bounds__(256) void window_lists_kernel(int rows, int nqb, int reach, int* __restrict__ rowptr,
                                                           int* __restrict__ idx, uint8_t* __restrict__ flags) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r > rows) return;
  const int bg = r / nqb, i = r % nqb;
  const int64_t off = int64_t(bg) * window_prefix(nqb, reach) + window_prefix(i, reach);
  rowptr[r] = int(off);
  if (r == rows) return;
  const int n = (i < reach ? i : reach) + 1;
  for (int k = 0; k < n; ++k) {
    idx[off + k] = i - n + 1 + k;
    flags[off + k] = 2;
  }
}

// Compressed-token block lists: query block i sees compressed tokens m <= m_max(i), the last one
// whose window ends at or before its last valid row; its list is key blocks 0 .. m_max / 64.
__device__ __forceinline__ int cmp_count(int i, int n_valid, int M, int block, int stride) {
  const int t = min(kBlock * i + kBlock - 1, n_valid - 1);
  if (t < block - 1 || M == 0) return 0;
  const int m = min((t - block + 1) / stride, M - 1);
  return m / kBlock + 1;
}
// Row offsets of one head's compressed lists: an exclusive prefix of the per-block counts, by one
// workgroup of 1024 threads (4 query blocks per thread, then a scan of the thread sums in LDS);
// head[i] for i = 0 .. nqb (head[nqb] = entries per head).  nqb <= 4096.
__global__ __launch_bounds__(1024) void cmp_prefix_kernel(int nqb, int n_valid, int M, int block, int stride,
                                                          int* __restrict__ head) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  int c[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * t + k;
    c[k] = i < nqb ? cmp_count(i, n_valid, M, block, stride) : 0;
    sum += c[k];
  }
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {       // inclusive scan (Hillis-Steele)
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - sum;                        // exclusive prefix of this thread's first block
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * t + k;
    if (i < nqb) head[i] = run;
    run += c[k];
  }
  if (t == 1023) head[nqb] = part[1023];           // entries per head
}

// Lists of every row from one head's offsets (head[0 .. nqb], written by cmp_prefix_kernel).
__global__ __launch_bounds__(256) void cmp_lists_kernel(int rows, int nqb, int n_valid, int M, int block, int stride,
                                                        const int* __restrict__ head, int* __restrict__ rowptr,
                                                        int* __restrict__ idx, uint8_t* __restrict__ flags) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r > rows) return;
  const int bg = r / nqb, i = r % nqb;
  const int64_t off = int64_t(bg) * head[nqb] + head[i];
  rowptr[r] = int(off);
  if (r == rows) return;
  const int n = cmp_count(i, n_valid, M, block, stride);
  for (int k = 0; k < n; ++k) {
    idx[off + k] = k;
    flags[off + k] = 1;
  }
}

// out[t] = sum_b sigmoid(q_t . w_b[h]) O_b[t] for valid rows, 0 for padded rows.  D / 8 lanes per
// row, 8 features per lane; the three gate dot products reduced across the row's lanes.
template <typename T, int D>
__global__ __launch_bounds__(256) void nsa_combine_kernel(const T* __restrict__ q, int64_t sB, int64_t sH, int64_t sN,
                                                          int Hq, int N, int n_valid, const float* __restrict__ w,
                                                          const float* __restrict__ oc, const float* __restrict__ os,
                                                          const float* __restrict__ ow, void* __restrict__ out,
                                                          int out_f32) {
  constexpr int kL = D / 8;                 // lanes per row
  constexpr int kRows = 256 / kL;
  const int bh = blockIdx.y, b = bh / Hq, h = bh % Hq;
  const int t = blockIdx.x * kRows + threadIdx.x / kL, c = threadIdx.x % kL;   // N % kRows == 0
  float qv[8];
  In<T>::load8_f32(q + int64_t(b) * sB + int64_t(h) * sH + int64_t(t) * sN + 8 * c, qv);
  float dots[3];
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    const float* wb = w + (int64_t(br) * Hq + h) * D + 8 * c;
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += qv[u] * wb[u];
#pragma unroll
    for (int m = 1; m < kL; m <<= 1) s += __shfl_xor(s, m);
    dots[br] = s;
  }
  const bool ok = t < n_valid;
  const int64_t base = (int64_t(bh) * N + t) * D + 8 * c;
  f32x8 o;
  const float* srcs[3] = {oc, os, ow};
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = 0.f;
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    const float g = 1.f / (1.f + __expf(-dots[br]));
    const f32x4 lo = *reinterpret_cast<const f32x4*>(srcs[br] + base);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(srcs[br] + base + 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      o[u] += g * lo[u];
      o[4 + u] += g * hi[u];
    }
  }
  if (!ok) {
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = 0.f;
  }
  if (out_f32) {
    float* dst = static_cast<float*>(out) + base;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
  } else {
    *reinterpret_cast<bf16x8*>(static_cast<u16*>(out) + base) = cvt8(o);
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e < n) *reinterpret_cast<f32x4*>(p + e) = f32x4{0.f, 0.f, 0.f, 0.f};
}

struct Nsa3Layout {
  int M, Mpad, reach, rows;
  int64_t n_win, n_cmp;
  size_t kc, vc, wrp, widx, wfl, chead, crp, cidx, cfl, oc, os, ow, total;
};

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

static Nsa3Layout nsa3_layout(int B, int Hq, int Hkv, int N, int d, int eb, int n_valid, int window, int block,
                              int stride) {
  Nsa3Layout L{};
  const int nqb = N / kBlock;
  L.M = n_valid >= block ? (n_valid - block) / stride + 1 : 0;
  L.Mpad = L.M > 0 ? (L.M + kBlock - 1) / kBlock * kBlock : kBlock;
  L.reach = window_reach(window);
  L.rows = B * Hkv * nqb;
  L.n_win = L.reach >= 0 ? int64_t(L.rows) * (L.reach + 1) : 0;
  L.n_cmp = int64_t(L.rows) * (L.Mpad / kBlock);
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += al256(bytes); return o; };
  L.kc = take(size_t(B) * Hkv * L.Mpad * d * eb);
  L.vc = take(size_t(B) * Hkv * L.Mpad * d * eb);
  L.wrp = take(size_t(L.rows + 1) * 4);
  L.widx = take(size_t(std::max<int64_t>(L.n_win, 1)) * 4);
  L.wfl = take(size_t(std::max<int64_t>(L.n_win, 1)));
  L.chead = take(size_t(nqb + 1) * 4);
  L.crp = take(size_t(L.rows + 1) * 4);
  L.cidx = take(size_t(std::max<int64_t>(L.n_cmp, 1)) * 4);
  L.cfl = take(size_t(std::max<int64_t>(L.n_cmp, 1)));
  const size_t ob = size_t(B) * Hq * N * d * 4;
  L.oc = take(ob);
  L.os = take(ob);
  L.ow = take(ob);
  L.total = off;
  return L;
}

}  // namespace sla

extern "C" size_t sla_nsa3_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d, int32_t dtype,
                                          int32_t n_valid, int32_t window_tokens, int32_t cmp_block,
                                          int32_t cmp_stride) {
  using namespace sla;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || N < kBlock || N % kBlock || (d != 64 && d != 128) ||
      cmp_block < 1 || cmp_stride < 1 || window_tokens < 0 || n_valid <= N - kBlock || n_valid > N)
    return 0;
  return nsa3_layout(B, Hq, Hkv, N, d, dtype == SLA_BF16 ? 2 : 4, n_valid, window_tokens, cmp_block, cmp_stride)
      .total;
}

extern "C" sla_status sla_nsa3_fwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                                   float scale, const int32_t* sel_rowptr, const int32_t* sel_idx,
                                   const uint8_t* sel_flags, int32_t window_tokens, int32_t cmp_block,
                                   int32_t cmp_stride, const float* w_gates, void* out, int32_t out_dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if (!same_geometry(q, k) || !same_geometry(k, v) || k->H != v->H || q->H % k->H != 0) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale) || window_tokens < 0 || cmp_block < 1 || cmp_stride < 1)
    return SLA_ERR_RANGE;
  if (sel_rowptr == nullptr || sel_idx == nullptr || sel_flags == nullptr || w_gates == nullptr || out == nullptr)
    return SLA_ERR_NULL;
  if (!aligned16(out) || !aligned16(w_gates)) return SLA_ERR_ALIGN;
  if (out_dtype != SLA_BF16 && out_dtype != SLA_F32) return SLA_ERR_UNSUPPORTED;
  const int B = q->B, Hq = q->H, Hkv = k->H, N = q->N, d = q->d, nqb = N / kBlock;
  if (nqb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  const int eb = q->dtype == SLA_BF16 ? 2 : 4;
  const Nsa3Layout L = nsa3_layout(B, Hq, Hkv, N, d, eb, n_valid, window_tokens, cmp_block, cmp_stride);
  if (workspace == nullptr || workspace_bytes < L.total || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = q->dtype == SLA_BF16;

  // 1. compressed tokens of K and V ([B, Hkv, Mpad, d], the input dtype)
  const dim3 cgrid(uint32_t((int64_t(L.Mpad) * (d / 8) + 255) / 256), uint32_t(B * Hkv));
#define SLA_CMP_LAUNCH(TT, DD)                                                                                   \
  do {                                                                                                           \
    compress_kernel<TT, DD><<<cgrid, 256, 0, s>>>(static_cast<const TT*>(k->ptr), k->sB, k->sH, k->sN, Hkv, L.M, \
                                                  L.Mpad, cmp_block, cmp_stride, reinterpret_cast<TT*>(ws + L.kc)); \
    compress_kernel<TT, DD><<<cgrid, 256, 0, s>>>(static_cast<const TT*>(v->ptr), v->sB, v->sH, v->sN, Hkv, L.M, \
                                                  L.Mpad, cmp_block, cmp_stride, reinterpret_cast<TT*>(ws + L.vc)); \
  } while (0)
  if (d == 128) {
    if (bf) SLA_CMP_LAUNCH(bf16raw, 128);
    else SLA_CMP_LAUNCH(float, 128);
  } else {
    if (bf) SLA_CMP_LAUNCH(bf16raw, 64);
    else SLA_CMP_LAUNCH(float, 64);
  }
#undef SLA_CMP_LAUNCH
  // 2. block lists of the window and compressed branches
  const dim3 lgrid(uint32_t((L.rows + 1 + 255) / 256));
  if (L.reach >= 0)
    window_lists_kernel<<<lgrid, 256, 0, s>>>(L.rows, nqb, L.reach, reinterpret_cast<int*>(ws + L.wrp),
                                              reinterpret_cast<int*>(ws + L.widx), ws + L.wfl);
  cmp_prefix_kernel<<<1, 1024, 0, s>>>(nqb, n_valid, L.M, cmp_block, cmp_stride, reinterpret_cast<int*>(ws + L.chead));
  cmp_lists_kernel<<<lgrid, 256, 0, s>>>(L.rows, nqb, n_valid, L.M, cmp_block, cmp_stride,
                                         reinterpret_cast<const int*>(ws + L.chead), reinterpret_cast<int*>(ws + L.crp),
                                         reinterpret_cast<int*>(ws + L.cidx), ws + L.cfl);
  // 3. the three branches, each normalised on its own, into fp32 buffers
  float* oc = reinterpret_cast<float*>(ws + L.oc);
  float* os = reinterpret_cast<float*>(ws + L.os);
  float* ow = reinterpret_cast<float*>(ws + L.ow);
  sla_tensor kc = *k, vc = *v;
  kc.ptr = ws + L.kc; vc.ptr = ws + L.vc;
  kc.N = vc.N = L.Mpad;
  kc.sN = vc.sN = d;
  kc.sH = vc.sH = int64_t(L.Mpad) * d;
  kc.sB = vc.sB = int64_t(Hkv) * L.Mpad * d;
  if ((st = launch_causal_pass(q, &kc, &vc, n_valid, L.M, scale, 0, cmp_block, cmp_stride,
                               reinterpret_cast<const int*>(ws + L.crp), reinterpret_cast<const int*>(ws + L.cidx),
                               ws + L.cfl, oc, s)) != SLA_OK)
    return st;
  if ((st = launch_causal_pass(q, k, v, n_valid, n_valid, scale, 0, 0, 0, sel_rowptr, sel_idx, sel_flags, os, s)) !=
      SLA_OK)
    return st;
  if (L.reach >= 0) {
    if ((st = launch_causal_pass(q, k, v, n_valid, n_valid, scale, window_tokens, 0, 0,
                                 reinterpret_cast<const int*>(ws + L.wrp), reinterpret_cast<const int*>(ws + L.widx),
                                 ws + L.wfl, ow, s)) != SLA_OK)
      return st;
  } else {
    const int64_t n = int64_t(B) * Hq * N * d;      // no window: that branch is 0 (a multiple of 4 floats)
    zero_f32_kernel<<<dim3(uint32_t((n / 4 + 255) / 256)), 256, 0, s>>>(ow, n);
  }
  // 4. gated merge
  const int rows_per_wg = 256 / (d / 8);
  const dim3 mgrid(uint32_t(N / rows_per_wg), uint32_t(B * Hq));
#define SLA_MERGE_LAUNCH(TT, DD)                                                                                   \
  nsa_combine_kernel<TT, DD><<<mgrid, 256, 0, s>>>(static_cast<const TT*>(q->ptr), q->sB, q->sH, q->sN, Hq, N, n_valid, \
                                                   w_gates, oc, os, ow, out, out_dtype == SLA_F32)
  if (d == 128) {
    if (bf) SLA_MERGE_LAUNCH(bf16raw, 128);
    else SLA_MERGE_LAUNCH(float, 128);
  } else {
    if (bf) SLA_MERGE_LAUNCH(bf16raw, 64);
    else SLA_MERGE_LAUNCH(float, 64);
  }
#undef SLA_MERGE_LAUNCH
  return launch_status();
}
