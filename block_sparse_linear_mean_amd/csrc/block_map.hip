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
#include <mutex>

#include "sla_device.h"
#include "sla_host.h"

namespace sla {

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;                     // -0 equals +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of the wave-wide mask m in the lanes below this one (v_mbcnt_lo / _hi: two
// instructions, no per-lane mask arithmetic).
__device__ __forceinline__ int bits_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Inclusive prefix sum over the 64 lanes of a wavefront, in lane order, without LDS: a
// Hillis-Steele scan inside each row of 16 lanes (DPP row shifts by 1, 2, 4, 8), then the row
// totals carried forward by the row broadcasts of lanes 15 and 31 (gfx9 DPP).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

// For each selection q: T[q] = the largest key such that at least n[q] candidates (j < ncand)
// have key >= T[q], i.e. the key of the n[q]-th most important candidate, and take[q] = how many
// candidates with key == T[q] belong to the top n[q] (n[q] clamped to 1 .. ncand; callers handle
// the degenerate cases).  MSB-first 8-bit radix select over LDS histograms (hist: at least
// max(kSub1, NS) x 256 words), the NS selections side by side so that their dependent LDS round
// trips overlap; the first digit's histogram has no prefix filter and serves every selection.
// The first digit (sign and exponent bits) is shared by most keys of a row, so its histogram is
// split into kSub1 copies (lane % kSub1), which cuts the serialisation of same-address atomics;
// the bin counts are the sums over the copies.  Scans run on DPP, broadcasts by readlane.
constexpr int kSub1 = 4;
constexpr int kHistWords = kSub1 * 256;   // histogram words; 64 more follow, one per lane, that take
                                          // the atomics of keys a pass does not count (branch-free)

// One radix pass over digit DGT (bits 8 DGT .. 8 DGT + 7): histogram of the keys that match each
// selection's prefix so far, then per selection the bin where its remaining count is reached.
// Straight-line code per pass; the keys a pass does not count go to the lane's dummy word.
template <int M, int NS, int DGT>
__device__ __forceinline__ void radix_pass(const uint32_t (&key)[M], const bool (&valid)[M], uint32_t* hist,
                                           uint32_t (&prefix)[NS], int (&rem)[NS]) {
  constexpr int shift = 8 * DGT;
  const int lane = threadIdx.x;
  const uint32_t dummy = kHistWords + lane;
  // selections whose prefixes agree so far share one histogram (always in the first pass)
  bool shared = true;
  if constexpr (DGT < 3) {
#pragma unroll
    for (int q = 1; q < NS; ++q) shared = shared && (prefix[q] >> (shift + 8)) == (prefix[0] >> (shift + 8));
  }
#pragma unroll
  for (int c = 0; c < (DGT == 3 ? kSub1 : NS); ++c)
    *reinterpret_cast<uint4*>(hist + 256 * c + 4 * lane) = uint4{0u, 0u, 0u, 0u};
  __syncthreads();
  if constexpr (DGT == 3) {
#pragma unroll
    for (int m = 0; m < M; ++m) atomicAdd(&hist[valid[m] ? 256 * (lane % kSub1) + (key[m] >> 24) : dummy], 1u);
  } else if (shared) {
    const uint32_t p0 = prefix[0] >> (shift + 8);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const bool match = valid[m] & ((key[m] >> (shift + 8)) == p0);
      atomicAdd(&hist[match ? (key[m] >> shift) & 255u : dummy], 1u);
    }
  } else if constexpr (NS == 2) {
    // two different prefixes: a key matches at most one of them, so one atomic per key
    const uint32_t p0 = prefix[0] >> (shift + 8), p1 = prefix[1] >> (shift + 8);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t hi = key[m] >> (shift + 8), dig = (key[m] >> shift) & 255u;
      const uint32_t at = hi == p0 ? dig : (hi == p1 ? 256u + dig : dummy);
      atomicAdd(&hist[valid[m] ? at : dummy], 1u);
    }
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const bool match = valid[m] & ((key[m] >> (shift + 8)) == (prefix[q] >> (shift + 8)));
        atomicAdd(&hist[match ? 256 * q + ((key[m] >> shift) & 255u) : dummy], 1u);
      }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    // lane l owns bins 255-4l .. 252-4l (descending), so lane order is key order
    const int lo = 252 - 4 * lane;               // bins lo .. lo + 3, c[e] = bin lo + 3 - e
    uint4 w4;
    if constexpr (DGT == 3) {
      w4 = *reinterpret_cast<const uint4*>(hist + lo);
#pragma unroll
      for (int sub = 1; sub < kSub1; ++sub) {
        const uint4 x = *reinterpret_cast<const uint4*>(hist + 256 * sub + lo);
        w4.x += x.x; w4.y += x.y; w4.z += x.z; w4.w += x.w;
      }
    } else {
      w4 = *reinterpret_cast<const uint4*>(hist + 256 * (shared ? 0 : q) + lo);
    }
    const uint32_t c[4] = {w4.w, w4.z, w4.y, w4.x};
    const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(lsum);
    const uint32_t excl = incl - lsum;
    const uint32_t rq = uint32_t(rem[q]);
    const bool hit = excl < rq && rq <= incl;
    // in the hit lane: the first of its bins whose cumulative count reaches rq (branch-free)
    const uint32_t a1 = excl + c[0], a2 = a1 + c[1], a3 = a2 + c[2];
    const uint32_t s1 = a1 < rq ? ~0u : 0u, s2 = a2 < rq ? ~0u : 0u, s3 = a3 < rq ? ~0u : 0u;  // bins passed
    const int bin = lo + 3 - int((s1 & 1u) + (s2 & 1u) + (s3 & 1u));
    const uint32_t above = excl + (c[0] & s1) + (c[1] & s2) + (c[2] & s3);
    const uint64_t hm = __ballot(hit);
    const int src = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<unsigned long long>(hm)) - 1);
    prefix[q] |= uint32_t(__builtin_amdgcn_readlane(bin, src)) << shift;
    rem[q] -= int(__builtin_amdgcn_readlane(above, src));
  }
  __syncthreads();
}

template <int M, int NS>
__device__ void radix_thresholds(const uint32_t (&key)[M], int ncand, const int (&n)[NS], uint32_t* hist,
                                 uint32_t (&T)[NS], int (&take)[NS]) {
  static_assert(NS <= kSub1, "one histogram per selection");
  const int lane = threadIdx.x;
  bool valid[M];
#pragma unroll
  for (int m = 0; m < M; ++m) valid[m] = lane + kWave * m < ncand;
  uint32_t prefix[NS];
  int rem[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) {
    prefix[q] = 0;
    rem[q] = min(max(n[q], 1), ncand);
  }
  radix_pass<M, NS, 3>(key, valid, hist, prefix, rem);
  radix_pass<M, NS, 2>(key, valid, hist, prefix, rem);
  radix_pass<M, NS, 1>(key, valid, hist, prefix, rem);
  radix_pass<M, NS, 0>(key, valid, hist, prefix, rem);
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
    // bitwise & and | (no short-circuit branches)
    const bool valid = lane + kWave * m < ncand;
    const bool eq = valid & (key[m] == T);
    const uint64_t em = __ballot(eq);
    const int before = seen + bits_below(em);
    in[m] = valid & ((key[m] > T) | (eq & (before < take)));
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
    const int at = pos + bits_below(bm);
    if (sel[m] & (at < limit)) {
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
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords + kWave];
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const float* s = scores + r * nkb;
  uint32_t key[M];
  float x[M];
#pragma unroll
  for (int m = 0; m < M; ++m) x[m] = s[min(lane + kWave * m, nkb - 1)];   // in bounds for every slot
  // the empty asm makes each value live here, after all loads are issued, so the compiler cannot
  // move a load under the j < nkb condition (where each load would wait for the one before)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    asm volatile("" : "+v"(x[m]));
    key[m] = order_key(x[m]) & (lane + kWave * m < nkb ? ~0u : 0u);
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
    for (int m = 0; m < M; ++m) marg[m] = keep[m] & !crit[m];
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
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords + kWave];
  const int64_t r = blockIdx.x;
  const int i = int(r % nb);
  const int lane = threadIdx.x;
  const int ncand = i + 1;
  const float* s = scores + r * nb;
  uint32_t key[M];
  float x[M];
#pragma unroll
  for (int m = 0; m < M; ++m) x[m] = s[min(lane + kWave * m, ncand - 1)];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    asm volatile("" : "+v"(x[m]));
    key[m] = order_key(x[m]) & (lane + kWave * m < ncand ? ~0u : 0u);
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

// Validation and launches of one block map; the causal path stages its padded per-row lists in
// `workspace` (a caller buffer, or this file's device scratch array for the allocation-free entry).
static sla_status block_map_impl(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                                 int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                                 int32_t* crit_rowptr, int32_t* crit_idx, uint8_t* crit_flags, int64_t crit_cap,
                                 int32_t* marg_rowptr, int32_t* marg_idx, int64_t marg_cap, uint32_t* marg_bits,
                                 int32_t* row_counts, void* workspace, size_t workspace_bytes, hipStream_t st) {
  const int64_t rows = int64_t(B) * Hs * nqb;
  // key slots per lane: the smallest instantiated M with 64 M >= nkb
  static constexpr int kSlots[] = {1, 2, 4, 8, 12, 16, 20, 24, 32, 40, 48, 64};
  int M = 64;
  for (int c : kSlots)
    if (c * kWave >= nkb) { M = c; break; }
#define SLA_DISPATCH_M(KERNEL, GRID, ...)                                    \
  switch (M) {                                                               \
    case 1: KERNEL<1><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 2: KERNEL<2><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 4: KERNEL<4><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 8: KERNEL<8><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;              \
    case 12: KERNEL<12><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 16: KERNEL<16><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 20: KERNEL<20><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 24: KERNEL<24><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 32: KERNEL<32><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 40: KERNEL<40><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    case 48: KERNEL<48><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
    default: KERNEL<64><<<GRID, 64, 0, st>>>(__VA_ARGS__); break;            \
  }
  if (!causal) {
    SLA_DISPATCH_M(classify_kernel, dim3(uint32_t(rows)), scores, nkb, n_crit, n_negl, rows, crit_rowptr,
                   crit_idx, crit_flags, marg_rowptr, marg_idx, marg_bits, row_counts);
    return launch_status();
  }
  const int reach = window_reach(window_tokens);
  const int row_cap = n_crit + reach + 1;
  int* pad_idx = static_cast<int*>(workspace);
  uint8_t* pad_flags =
      static_cast<uint8_t*>(workspace) + (rows * row_cap * 4 + 255) / 256 * 256;
  (void)workspace_bytes;
  SLA_DISPATCH_M(select_causal_kernel, dim3(uint32_t(rows)), scores, nkb, n_crit, reach, row_cap, pad_idx,
                 pad_flags, row_counts);
#undef SLA_DISPATCH_M
  rowptr_scan_kernel<<<1, 1024, 0, st>>>(row_counts, rows, crit_rowptr, marg_rowptr);
  compact_rows_kernel<<<dim3(uint32_t(rows)), 64, 0, st>>>(crit_rowptr, pad_idx, pad_flags, row_cap, crit_idx,
                                                          crit_flags);
  return launch_status();
}

// Host-side checks shared by both entry points (no HIP call).  need_ws: workspace bytes the
// causal path needs (0 for non-causal maps).
static sla_status block_map_check(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                                  int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                                  const int32_t* crit_rowptr, const int32_t* crit_idx, int64_t crit_cap,
                                  const int32_t* marg_rowptr, const int32_t* marg_idx, int64_t marg_cap,
                                  const uint32_t* marg_bits, const int32_t* row_counts, size_t* need_ws) {
  *need_ws = 0;
  if (scores == nullptr || crit_rowptr == nullptr || crit_idx == nullptr || row_counts == nullptr)
    return SLA_ERR_NULL;
  if (B < 1 || Hs < 1 || nqb < 1 || nkb < 1) return SLA_ERR_SHAPE;
  if (nkb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  if (n_crit < 0 || n_negl < 0 || window_tokens < 0) return SLA_ERR_RANGE;
  const int64_t rows = int64_t(B) * Hs * nqb;
  if (rows > INT32_MAX) return SLA_ERR_SHAPE;
  if (!causal) {
    if (n_crit + n_negl > nkb) return SLA_ERR_RANGE;
    const int64_t nm = nkb - n_crit - n_negl;
    if ((marg_rowptr == nullptr) != (marg_idx == nullptr)) return SLA_ERR_NULL;
    if (crit_cap < rows * n_crit || (marg_idx != nullptr && marg_cap < rows * nm)) return SLA_ERR_CAPACITY;
    if (rows * n_crit > INT32_MAX || rows * nm > INT32_MAX) return SLA_ERR_CAPACITY;
    return SLA_OK;
  }
  if (nqb != nkb) return SLA_ERR_SHAPE;
  if (marg_bits != nullptr) return SLA_ERR_UNSUPPORTED;   // causal maps have no marginal class
  const int64_t cap = sla_block_map_capacity(B, Hs, nqb, nkb, n_crit, n_negl, 1, window_tokens, 0);
  if (crit_cap < cap || cap > INT32_MAX) return SLA_ERR_CAPACITY;
  *need_ws = sla_block_map_workspace_bytes(B, Hs, nqb, nkb, n_crit, 1, window_tokens);
  return SLA_OK;
}

// ---- allocation-free variant: the causal path's scratch lives in a static device array

// Largest causal workspace the allocation-free entry point serves (rows * row_cap * 5 bytes plus
// alignment: e.g. 8 GQA groups x 16384 query blocks at 16 selected blocks and a 512-token window).
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on each device, looked up once per device (with that device
// current) on the entry point's first call there.  In host code the array's name is only a
// host-side stand-in; kernels get this address.
static void* g_scratch_dev[kScratchDevices] = {};
static std::mutex g_scratch_mu;

static sla_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SLA_ERR_HIP;
  if (dev >= kScratchDevices) return SLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SLA_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SLA_OK;
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
  size_t need = 0;
  const sla_status s = block_map_check(scores, B, Hs, nqb, nkb, n_crit, n_negl, causal, window_tokens,
                                       crit_rowptr, crit_idx, crit_cap, marg_rowptr, marg_idx, marg_cap, marg_bits,
                                       row_counts, &need);
  if (s != SLA_OK) return s;
  if (causal && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))) return SLA_ERR_WORKSPACE;
  return block_map_impl(scores, B, Hs, nqb, nkb, n_crit, n_negl, causal, window_tokens, crit_rowptr, crit_idx,
                        crit_flags, crit_cap, marg_rowptr, marg_idx, marg_cap, marg_bits, row_counts, workspace,
                        workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" sla_status sla_block_map_noalloc(const float* scores, int32_t B, int32_t Hs, int32_t nqb, int32_t nkb,
                                            int32_t n_crit, int32_t n_negl, int32_t causal, int32_t window_tokens,
                                            int32_t* crit_rowptr, int32_t* crit_idx, uint8_t* crit_flags,
                                            int64_t crit_cap, int32_t* marg_rowptr, int32_t* marg_idx,
                                            int64_t marg_cap, uint32_t* marg_bits, int32_t* row_counts,
                                            void* stream) {
  using namespace sla;
  size_t need = 0;
  const sla_status s = block_map_check(scores, B, Hs, nqb, nkb, n_crit, n_negl, causal, window_tokens,
                                       crit_rowptr, crit_idx, crit_cap, marg_rowptr, marg_idx, marg_cap, marg_bits,
                                       row_counts, &need);
  if (s != SLA_OK) return s;
  if (need > kScratchBytes) return SLA_ERR_WORKSPACE;
  void* ws = nullptr;
  const sla_status a = scratch_address(&ws);
  if (a != SLA_OK) return a;
  // Nothing in the scratch needs clearing: each row's padded list is written in full up to its count
  // by this call before the compaction reads it.
  return block_map_impl(scores, B, Hs, nqb, nkb, n_crit, n_negl, causal, window_tokens, crit_rowptr, crit_idx,
                        crit_flags, crit_cap, marg_rowptr, marg_idx, marg_cap, marg_bits, row_counts, ws, kScratchBytes,
                        static_cast<hipStream_t>(stream));
}
