// Classification step: per query-block row, label every key block critical, marginal
// or negligible and emit CSR lists of the critical and marginal blocks (and, optionally, the
// marginal set as a bit mask per row, the form the marginal aggregation consumes).
//
// Method: each (query block, key block) pair falls in one of three classes — the top
// share of a row is critical, the bottom share negligible, the rest marginal (SLA
// analysis page for arXiv 2509.24006, comparison tables; "2025稀疏注意力架构综述",
// section 10 SLA).  The NSA-style causal variant selects a fixed number of 64-token
// blocks per query block and adds a sliding window ("Sparse Attention 方法综述",
// section 2 NSA, key-parameter table).
//
// One wavefront owns one row.  Scores are mapped to an order-preserving uint32 key
// (larger key = more important; -0 -> +0; every NaN -> 0, the lowest key), so the
// row's total order is (key descending, block index ascending).  The boundary of the
// top-n set is found by an MSB-first 8-bit radix select over LDS histograms (four
// passes; the critical and the kept boundary of a row side by side in the same passes), and
// equal keys at the boundary are taken in ascending block order by a ballot prefix count.  The lists are written with ballot compaction, which emits
// ascending block indices.  Everything is integer work: results are bit-exact.
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;                     // -0 equals +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  return (uint64_t(1) << threadIdx.x) - 1;          // one wavefront per workgroup
}

// For each selection q: T[q] = the largest key such that at least n[q] candidates (j < ncand)
// have key >= T[q], i.e. the key of the n[q]-th most important candidate, and take[q] = how many
// candidates with key == T[q] belong to the top n[q] (n[q] clamped to 1 .. ncand; callers handle
// the degenerate cases).  MSB-first 8-bit radix select over LDS histograms (hist: NS x 256
// words), the NS selections side by side so that their dependent LDS round trips overlap; the
// first digit's histogram has no prefix filter and serves every selection.
template <int M, int NS>
__device__ void radix_thresholds(const uint32_t (&key)[M], int ncand, const int (&n)[NS], uint32_t* hist,
                                 uint32_t (&T)[NS], int (&take)[NS]) {
  const int lane = threadIdx.x;
  uint32_t prefix[NS];
  int rem[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    prefix[q] = 0;
    rem[q] = min(max(n[q], 1), ncand);
  }
#pragma unroll 1
  for (int dgt = 3; dgt >= 0; --dgt) {
    const int shift = 8 * dgt;
    const int nh = dgt == 3 ? 1 : NS;            // histograms built in this pass
    for (int q = lane; q < 256 * nh; q += kWave) hist[q] = 0u;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int j = lane + kWave * m;
      if (j < ncand) {
        const uint32_t k = key[m];
        if (dgt == 3) {
          atomicAdd(&hist[k >> 24], 1u);
        } else {
#pragma unroll
          for (int q = 0; q < NS; ++q)
            if ((k >> (shift + 8)) == (prefix[q] >> (shift + 8))) atomicAdd(&hist[256 * q + ((k >> shift) & 255u)], 1u);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const uint32_t* hq = hist + (dgt == 3 ? 0 : 256 * q);
      // lane l owns bins 255-4l .. 252-4l (descending), so lane order is key order
      uint32_t c[4], lsum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hq[255 - (4 * lane + e)];
        lsum += c[e];
      }
      uint32_t incl = lsum;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const uint32_t excl = incl - lsum;
      const bool hit = excl < uint32_t(rem[q]) && uint32_t(rem[q]) <= incl;
      int bin = 0;
      uint32_t above = excl;
      if (hit) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (above + c[e] >= uint32_t(rem[q])) {
            bin = 255 - (4 * lane + e);
            break;
          }
          above += c[e];
        }
      }
      const uint64_t hm = __ballot(hit);
      const int src = __ffsll(static_cast<unsigned long long>(hm)) - 1;
      bin = __shfl(bin, src);
      above = __shfl(above, src);
      prefix[q] |= uint32_t(bin) << shift;
      rem[q] -= int(above);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    T[q] = prefix[q];
    take[q] = rem[q];
  }
}

// in[m] = candidate j = lane + 64 m is among the n most important of the first ncand, given the
// threshold (T, take) of n from radix_thresholds.
template <int M>
__device__ void top_set(const uint32_t (&key)[M], int ncand, int n, uint32_t T, int take, bool (&in)[M]) {
  const int lane = threadIdx.x;
  if (n <= 0 || n >= ncand) {
#pragma unroll
    for (int m = 0; m < M; ++m) in[m] = n > 0 && lane + kWave * m < ncand;
    return;
  }
  int seen = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool valid = lane + kWave * m < ncand;
    const bool eq = valid && key[m] == T;
    const uint64_t em = __ballot(eq);
    const int before = seen + __popcll(em & lanes_below());
    in[m] = valid && (key[m] > T || (eq && before < take));
    seen += __popcll(em);
  }
}

// Writes the blocks with sel[m] set, ascending, at out[0..limit); returns how many were set.
template <int M>
__device__ int compact_write(const bool (&sel)[M], int* out, uint8_t* flags_out, const uint8_t (&flag)[M],
                             int limit) {
  const int lane = threadIdx.x;
  int pos = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint64_t bm = __ballot(sel[m]);
    const int at = pos + __popcll(bm & lanes_below());
    if (sel[m] && at < limit) {
      out[at] = lane + kWave * m;
      if (flags_out) flags_out[at] = flag[m];
    }
    pos += __popcll(bm);
  }
  return pos;
}

template <int M>
__global__ __launch_bounds__(64) void classify_kernel(const float* __restrict__ scores, int nkb, int n_crit,
                                                      int n_negl, int64_t rows, int* __restrict__ crit_rowptr,
                                                      int* __restrict__ crit_idx, uint8_t* __restrict__ crit_flags,
                                                      int* __restrict__ marg_rowptr, int* __restrict__ marg_idx,
                                                      uint32_t* __restrict__ marg_bits, int* __restrict__ row_counts) {
  __shared__ uint32_t hist[2 * 256];
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const float* s = scores + r * nkb;
  uint32_t key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = lane + kWave * m;
    key[m] = j < nkb ? order_key(s[j]) : 0u;
  }
  const int n_keep = nkb - n_negl;       // critical + marginal
  const int n_marg = n_keep - n_crit;
  bool crit[M], keep[M];
  const int nsel[2] = {n_crit, n_keep};
  uint32_t T[2];
  int take[2];
  radix_thresholds<M, 2>(key, nkb, nsel, hist, T, take);   // both boundaries in the same passes
  top_set<M>(key, nkb, n_crit, T[0], take[0], crit);
  top_set<M>(key, nkb, n_keep, T[1], take[1], keep);
  uint8_t one[M];
#pragma unroll
  for (int m = 0; m < M; ++m) one[m] = 1;
  compact_write<M>(crit, crit_idx + r * n_crit, crit_flags ? crit_flags + r * n_crit : nullptr, one, n_crit);
  if (marg_idx != nullptr || marg_bits != nullptr) {
    bool marg[M];
#pragma unroll
    for (int m = 0; m < M; ++m) marg[m] = keep[m] && !crit[m];
    if (marg_idx != nullptr) compact_write<M>(marg, marg_idx + r * n_marg, nullptr, one, n_marg);
    if (marg_bits != nullptr) {
      // block j = lane + 64 m is bit j % 32 of word j / 32: one ballot fills words 2m and 2m + 1
      const int nw = (nkb + 31) / 32;
      uint32_t* out = marg_bits + r * nw;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint64_t bm = __ballot(marg[m]);
        if (lane < 2 && 2 * m + lane < nw) out[2 * m + lane] = uint32_t(bm >> (32 * lane));
      }
    }
  }
  if (lane == 0) {
    crit_rowptr[r] = int(r * n_crit);
    if (marg_rowptr) marg_rowptr[r] = int(r * n_marg);
    row_counts[3 * r + 0] = n_crit;
    row_counts[3 * r + 1] = n_marg;
    row_counts[3 * r + 2] = n_negl;
    if (r == rows - 1) {
      crit_rowptr[rows] = int(rows * n_crit);
      if (marg_rowptr) marg_rowptr[rows] = int(rows * n_marg);
    }
  }
}

// Causal (NSA-style) rows: candidates j <= i, top min(n_sel, i+1) selected, united with the
// window blocks i - reach .. i.  Writes a padded list per row (row_cap entries) and counts.
template <int M>
__global__ __launch_bounds__(64) void select_causal_kernel(const float* __restrict__ scores, int nb, int n_sel,
                                                           int reach, int row_cap, int* __restrict__ pad_idx,
                                                           uint8_t* __restrict__ pad_flags,
                                                           int* __restrict__ row_counts) {
  __shared__ uint32_t hist[256];
  const int64_t r = blockIdx.x;
  const int i = int(r % nb);
  const int lane = threadIdx.x;
  const int ncand = i + 1;
  const float* s = scores + r * nb;
  uint32_t key[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = lane + kWave * m;
    key[m] = j < ncand ? order_key(s[j]) : 0u;
  }
  bool sel[M];
  const int nsel[1] = {min(n_sel, ncand)};
  uint32_t T[1];
  int take[1];
  radix_thresholds<M, 1>(key, ncand, nsel, hist, T, take);
  top_set<M>(key, ncand, nsel[0], T[0], take[0], sel);
  bool mem[M];
  uint8_t flag[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = lane + kWave * m;
    const bool win = reach >= 0 && j <= i && j >= i - reach;
    mem[m] = sel[m] || win;
    flag[m] = uint8_t((sel[m] ? 1 : 0) | (win ? 2 : 0));
  }
  const int cnt = min(row_cap, compact_write<M>(mem, pad_idx + r * row_cap, pad_flags + r * row_cap, flag, row_cap));
  if (lane == 0) {
    row_counts[3 * r + 0] = cnt;
    row_counts[3 * r + 1] = 0;
    row_counts[3 * r + 2] = ncand - cnt;
  }
}

// Exclusive prefix sum of the per-row critical counts (one workgroup, fixed order).
__global__ __launch_bounds__(1024) void rowptr_scan_kernel(const int* __restrict__ row_counts, int64_t rows,
                                                           int* __restrict__ rowptr, int* __restrict__ marg_rowptr) {
  __shared__ int wsum[16];
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave;
  int carry = 0;
  for (int64_t base = 0; base < rows; base += 1024) {
    const int64_t rr = base + t;
    const int v = rr < rows ? row_counts[3 * rr] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
      int ws = lane < 16 ? wsum[lane] : 0;
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const int y = __shfl_up(ws, off);
        if (lane >= off) ws += y;
      }
      if (lane < 16) wsum[lane] = ws;
    }
    __syncthreads();
    const int wbase = w > 0 ? wsum[w - 1] : 0;
    if (rr < rows) {
      rowptr[rr] = carry + wbase + incl - v;
      if (marg_rowptr) marg_rowptr[rr] = 0;
    }
    const int total = wsum[15];
    __syncthreads();
    carry += total;
  }
  if (t == 0) {
    rowptr[rows] = carry;
    if (marg_rowptr) marg_rowptr[rows] = 0;
  }
}

__global__ __launch_bounds__(64) void compact_rows_kernel(const int* __restrict__ rowptr,
                                                          const int* __restrict__ pad_idx,
                                                          const uint8_t* __restrict__ pad_flags, int row_cap,
                                                          int* __restrict__ idx, uint8_t* __restrict__ flags) {
  const int64_t r = blockIdx.x;
  const int beg = rowptr[r], cnt = min(rowptr[r + 1] - beg, row_cap);
  for (int e = threadIdx.x; e < cnt; e += kWave) {
    idx[beg + e] = pad_idx[r * row_cap + e];
    if (flags) flags[beg + e] = pad_flags[r * row_cap + e];
  }
}

}  // namespace sla

extern "C" sla_status sla_block_map(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                                    int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                                    int32_t* crit_rowptr, int32_t* crit_idx, uint8_t* crit_flags,
                                    int64_t crit_cap, int32_t* marg_rowptr, int32_t* marg_idx, int64_t marg_cap,
                                    uint32_t* marg_bits,
                                    int32_t* row_counts, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  using namespace sla;
  if (scores == nullptr || crit_rowptr == nullptr || crit_idx == nullptr || row_counts == nullptr)
    return SLA_ERR_NULL;
  if (B < 1 || Hs < 1 || nqb < 1 || nkb < 1) return SLA_ERR_SHAPE;
  if (nkb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  if (n_crit < 0 || n_negl < 0 || window_tokens < 0) return SLA_ERR_RANGE;
  const int64_t rows = int64_t(B) * Hs * nqb;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int M = 1;
  while (M * kWave < nkb) M *= 2;
#define SLA_DISPATCH_M(KERNEL, GRID, ...)                                    \
  switch (M) {                                                               \
    case 1: KERNEL<1><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 2: KERNEL<2><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 4: KERNEL<4><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 8: KERNEL<8><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 16: KERNEL<16><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 32: KERNEL<32><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    default: KERNEL<64><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
  }
  if (!causal) {
    if (n_crit + n_negl > nkb) return SLA_ERR_RANGE;
    const int64_t nm = nkb - n_crit - n_negl;
    if ((marg_rowptr == nullptr) != (marg_idx == nullptr)) return SLA_ERR_NULL;
    if (crit_cap < rows * n_crit || (marg_idx != nullptr && marg_cap < rows * nm)) return SLA_ERR_CAPACITY;
    if (rows * n_crit > INT32_MAX || rows * nm > INT32_MAX) return SLA_ERR_CAPACITY;
    SLA_DISPATCH_M(classify_kernel, dim3(uint32_t(rows)), scores, nkb, n_crit, n_negl, rows, crit_rowptr,
                   crit_idx, crit_flags, marg_rowptr, marg_idx, marg_bits, row_counts);
    return launch_status();
  }
  if (nqb != nkb) return SLA_ERR_SHAPE;
  if (marg_bits != nullptr) return SLA_ERR_UNSUPPORTED;   // causal maps have no marginal class
  const int64_t cap = sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, 1, window_tokens, 0);
  if (crit_cap < cap || cap > INT32_MAX) return SLA_ERR_CAPACITY;
  const size_t need = sla_block_map_workspace_bytes(B, Hs, nqb, nkb, n_crit, 1, window_tokens);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
  const int reach = window_reach(window_tokens);
  const int row_cap = n_crit + reach + 1;
  int* pad_idx = static_cast<int*>(workspace);
  uint8_t* pad_flags =
      static_cast<uint8_t*>(workspace) + (rows * row_cap * 4 + 255) / 256 * 256;
  SLA_DISPATCH_M(select_causal_kernel, dim3(uint32_t(rows)), scores, nkb, n_crit, reach, row_cap, pad_idx,
                 pad_flags, row_counts);
#undef SLA_DISPATCH_M
  rowptr_scan_kernel<<<1, 1024, 0, st>>>(row_counts, rows, crit_rowptr, marg_rowptr);
  compact_rows_kernel<<<dim3(uint32_t(rows)), 64, 0, st>>>(crit_rowptr, pad_idx, pad_flags, row_cap, crit_idx,
                                                          crit_flags);
  return launch_status();
}
