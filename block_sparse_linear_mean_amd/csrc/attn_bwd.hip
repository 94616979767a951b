// Backward of the SLA layer: dQ, dK, dV of O = O_sparse + O_linear for a fixed block map.
//
// Method: the pages fine-tune SLA (SLA analysis page for arXiv 2509.24006: the Proj layer and
// the linear path are learned), so the layer needs the exact gradient of its forward.  The
// block map is piecewise constant in Q and K and is held fixed; the gradient flows through
//  * the critical branch (block-sparse softmax attention): with P = exp(scale q.k - lse),
//    dP = dO V^T, D_t = dO_t . O_sparse_t and dS = P (dP - D):
//    dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO over the critical pairs only;
//  * the marginal linear branch O_l = phi(q)^T S_i / (phi(q) . u_i) with S_i = sum of H_j and
//    u_i = sum of z_j over the marginal blocks j of query block i, H_j = phi(K_j)^T V_j:
//    dn = dO / den, dden = -(dO . O_l) / den, dphi(q) = S_i dn + u_i dden,
//    dS_i = phi(Q_i)^T dN_i, du_i = phi(Q_i)^T dden; dH_j and dz_j are the sums of dS_i, du_i
//    over the query blocks i that have j marginal (a 0/1-mask product with the mask
//    transposed); dphi(k) = dH_j v + dz_j, dV += phi(K_j) dH_j.
// O_sparse = O - O_l uses the forward's output; P uses the forward's log-sum-exp.
//
// Design (gfx950, wave64): every kernel runs 4 wavefronts of 16 rows (queries or keys) on
// 16x16x32 bf16 matrix cores with fp32 accumulation.  64-row tiles are staged in LDS in the
// layout of the transposing read (16-byte chunk c of row r at c ^ 2 (r % 4)), so an operand
// can be read along rows (16 contiguous bytes per lane) or across them (two transposing
// reads).  Contractions over the rows of an accumulator pair two 16-row tiles: the lane's
// 4 + 4 accumulator rows are the k-slots of one 32-deep product, and the other operand reads
// the same rows.  The query-stationary kernels (linear dQ and sparse dQ) iterate over a
// row's lists; the key-stationary ones (linear dK/dV and sparse dK/dV) over the transposed
// lists, kept as one bit per (key block, query block); no atomics on gradients, so results
// are deterministic.
#include <type_traits>

#include "attn_tiles.h"
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

sla_status launch_marginal_states(const u16* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const uint32_t* bits, u16* S, float* u, hipStream_t st);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  int64_t qsB, qsH, qsN, ksB, ksH, ksN, vsB, vsH, vsN, osB, osH, osN, dsB, dsH, dsN;
  int B, H, N, nb, n_valid, wq;   // wq: 32-bit words per transposed bit row, ceil(nb / 32)
  int Hkv, G, Hs, group_map;      // KV heads, query heads per KV head, map heads, maps shared by a group
  int window;                     // causal maps: key s of a window block is allowed iff t - s < window
  int overwrite;                  // no linear branch: the sparse kernels write dQ, dK, dV (else add)
  int gated;                      // SALAD: one linear state per head (all keys), gated by sigmoid(q . w_gate)
  int hsplit;                     // dK/dV workgroups per key block: each takes G / hsplit of the group's heads
  float* part_k;                  // hsplit > 1: [hsplit][B, Hkv, N, d] partial dK (scaled) and dV per subset
  float* part_v;
  float scale, scale_log2;
  const float* lse;               // [B, H, N] natural log-sum-exp of the forward's sparse branch
  const int* crit_rowptr;
  const int* crit_idx;
  const uint8_t* crit_flags;      // causal maps: bit 0 = selected block (else a window block)
  const uint32_t* critT_sel;      // causal maps: [map rows][wq], the selected bits of critT
  const float* Sf;                // SALAD: H_all fp32 [B, H][c][r] (S, u then unused; u = z_all)
  const float* w_gate;            // SALAD: [H][d]
  float* gpart;                   // SALAD: [B, H, nb][d] partial gradients of w_gate per query block
  const u16* S;                   // per-row marginal sums, bf16 [rows][c][r]
  const float* u;                 // [rows][r]
  float* D;                       // [B, H, N]: dO . O_sparse
  u16* dS;                        // [rows][c][r] bf16: gradient of S_i
  float* du;                      // [rows][r]
  const u16* dH;                  // [B, H, nb][c][r] bf16: gradient of H_j
  const float* dz;                // [B, H, nb][r]
  const uint32_t* critT;          // [map rows][wq]: bit i of row (b, m, j) = block j is critical for query block i
  const int* kv_order;            // [B * H * nb]: key-block rows, most-used first (dK/dV dispatch order)
  const float* k_shift;           // smooth-K: [B, H, d] key mean of the forward, or null
  const float* dk_mean;           // smooth-K: [B, H, d] mean over valid rows of the linear-branch dK
  const float* proj_w;            // Proj weight [heads][d][d] fp32 or null (identity)
  const float* proj_b;            // Proj bias [heads][d] or null
  int64_t proj_sH;                // elements between consecutive heads' weights (0: shared)
  u16* xlin;                      // Proj: [B, H, N, d] bf16, the linear-branch output O_l per row
  float* dq;                      // [B, H, N, d] fp32
  float* dk;
  float* dv;
};

constexpr int kBwWaves = 4;
constexpr int kBwThreads = kWave * kBwWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxKeyBlocksBwd = SLA_MAX_KEY_BLOCKS;

template <int D>
__device__ __forceinline__ int tpos(int r, int c8) {
  return v_pos<D>(r, c8);      // the layout the direct-to-LDS tile copies write
}

// Byte offset, in a tpos tile, of the transposing read that gives lane l (group g = l / 16,
// i = l % 16) rows row_g .. row_g + 3 of column col0 + i; row_g is the caller's row for the
// lane's group.
template <int D>
__device__ __forceinline__ int tr_addr(int row_g, int col0, int lane) {
  const int i = lane % 16;
  return tpos<D>(row_g + i / 4, col0 / 8 + (i % 4) / 2) + 8 * (i % 2);
}

// With the linear key side in the dK/dV epilogue, dK tiles use a permuted feature order: tile ct
// holds, in lane group g, the 4 consecutive features
// kcol(ct, g) .. + 3 = 32 (ct / 2) + 8 g + 4 (ct % 2) + 0..3 — the features that the 8-feature
// operand chunk 32 kc + 8 g of a lane holds (kc = ct / 2), so the key values the linear branch's dK
// needs at its output positions are already in the lane's K operand.  tr_addr_kperm is the
// transposing read of tile ct's features in that order (its 16 lanes point at 4 rows x 4 pieces of
// 4 features; output lane i gets piece i / 4, element i % 4 of each row).
__device__ __forceinline__ int kcol(int ct, int g) { return 32 * (ct / 2) + 8 * g + 4 * (ct % 2); }
template <int D>
__device__ __forceinline__ int tr_addr_kperm(int row_g, int ct, int lane) {
  const int i = lane % 16;
  return tpos<D>(row_g + i / 4, 4 * (ct / 2) + i % 4) + 8 * (ct % 2);
}

__device__ __forceinline__ bf16x8 join(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ bf16x4 cvt4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

template <typename T>
__device__ __forceinline__ f32x4 load4_f32(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xffff0000u)};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

// dO as the matrix-core products see it: fp32 inputs are rounded to bf16 for dP = dO V^T, so
// D = dO . O is formed from the same rounded values and dP - D cancels exactly where it must
// (a row whose softmax has a single key); bf16 inputs are unchanged.
template <typename T>
__device__ __forceinline__ float as_operand(float x) {
  if constexpr (sizeof(T) == 2) return x;
  else return static_cast<float>(static_cast<__bf16>(x));
}

// sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float group4_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Stage rows row0 .. row0 + 63 of X (row stride sN) into a tpos tile as bf16; rows at or past
// n_rows are written as zeros (and never read from X).
template <typename T, int D>
__device__ __forceinline__ void stage64(const T* __restrict__ X, int64_t sN, int row0, int n_rows, lds_u8* tile) {
  constexpr int kChunks = D / 8, kPer = kBlock * kChunks / kBwThreads;
  bf16x8 x[kPer];                    // every load of the thread in flight together
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = threadIdx.x + kBwThreads * u, r = e / kChunks, c = e % kChunks;
    x[u] = row0 + r < n_rows ? In<T>::load8(X + int64_t(row0 + r) * sN + 8 * c) : zero8();
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = threadIdx.x + kBwThreads * u;
    lds_store16(tile + tpos<D>(e / kChunks, e % kChunks), x[u]);
  }
}

// ------------------------------------------------------------------ transposed bit masks

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e < n) p[e] = v;
}

// One wavefront per map row (b, s, i), one lane per listed block j: set bit i of row (b, s, j) of
// the transposed critical mask, and of its selected mask when the entry's flag has bit 0 (causal
// maps; flags NULL: none), by atomic OR (the result does not depend on the order), so every
// entry's atomics are in flight at once.  Also counts, per key-block row (b, g, j) of the KV head g
// that map head s reads (s with shared maps, s / G otherwise), the listing entries (the dK/dV
// workload of that row, up to a factor G with shared maps).
__global__ __launch_bounds__(256) void crit_transpose_kernel(const int* __restrict__ rowptr, const int* __restrict__ idx,
                                                             const uint8_t* __restrict__ flags, int rows, int nb,
                                                             int wq, int Hs, int Hkv, int kv_div,
                                                             uint32_t* __restrict__ critT,
                                                             uint32_t* __restrict__ critT_sel,
                                                             int* __restrict__ counts) {
  const int r = blockIdx.x * 4 + int(threadIdx.x) / kWave;
  if (r >= rows) return;
  const int bs = r / nb, i = r % nb, b = bs / Hs, sh = bs % Hs;
  const int64_t kvrow0 = (int64_t(b) * Hkv + sh / kv_div) * nb;
  for (int e = rowptr[r] + int(threadIdx.x) % kWave; e < rowptr[r + 1]; e += kWave) {
    const int j = idx[e];
    if (unsigned(j) < unsigned(nb)) {
      const uint32_t bit = 1u << (i % 32);
      const int64_t word = (int64_t(bs) * nb + j) * wq + i / 32;
      // a repeated entry (a malformed list) is counted once
      if ((atomicOr(critT + word, bit) & bit) == 0u) atomicAdd(counts + kvrow0 + j, 1);
      if (flags != nullptr && (flags[e] & 1u) != 0u) atomicOr(critT_sel + word, bit);
    }
  }
}

// One thread per (map row, mask word): the marginal bit masks [rows][wk], transposed.
__global__ __launch_bounds__(256) void marg_transpose_kernel(const uint32_t* __restrict__ bits, int rows, int nb,
                                                             int wk, int wq, uint32_t* __restrict__ margT) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(rows) * wk) return;
  const int r = int(e / wk), word = int(e % wk);
  const int bh = r / nb, i = r % nb;
  uint32_t m = bits[e];
  while (m != 0u) {
    const int j = 32 * word + __builtin_ctz(m);
    m &= m - 1u;
    if (j < nb) atomicOr(margT + (int64_t(bh) * nb + j) * wq + i / 32, 1u << (i % 32));
  }
}

// ------------------------------------------------------------------ linear branch, query side

__device__ __forceinline__ bf16x4 lds_load8(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x4*>(p);
}

// LDS the linear query side works in: St the row's state as the [c][r] tile (D rows of 2 D bytes),
// Pq and Dn 64-row tiles (phi(Q_i) [t][r], dN_i [t][c]), Wt the Proj weight [o][c] (PROJ), us D
// floats, dden_s and dlog_s 64 floats, gred the gate-gradient row-group sums (GATED, kRg x D).
struct LinQLds {
  lds_u8* St;
  lds_u8* Pq;
  lds_u8* Dn;
  lds_u8* Wt;
  float* us;
  float* dden_s;
  float* dlog_s;
  float* gred;
};

// Linear branch, query side, of query block i of head h (wavefront w owns query rows
// 64 i + 16 w + l % 16): writes D_t and the per-row gradients dS_i ([c][r], bf16) and du_i, and
// returns the lane's linear dQ (dql[rt][e]: feature 16 rt + 4 g + e of its row; 0 on padded rows)
// and its row's D_t.
// PROJ: O = O_s + O_l W^T + b, so O_s = O - O_l W^T - b, the gradient reaching O_l is dO W, and
// O_l is written out (bf16) for the weight gradient.
// GATED (SALAD): the state is the head's sum over all keys (H_all, z_all, fp32) and
// O_l = sigmoid(q . w_g) phi(q)^T H_all / (phi(q) . z_all); the gate adds dlogit w_g to dq and
// dlogit q to the gate weights' gradient (a partial per query block), dlogit = (dO . y) g (1 - g)
// with y the ungated term.
template <typename T, int D, bool PROJ, bool GATED>
__device__ __forceinline__ void lin_q_side(const BwdParams& p, int b, int h, int i, const LinQLds& L,
                                           f32x4 (&dql)[D / 16], float& Dt) {
  constexpr int kKc = D / 32;     // 32-deep k-steps over features
  constexpr int kCt = D / 16;     // 16-wide feature tiles
  lds_u8* St = L.St;
  lds_u8* Pq = L.Pq;
  lds_u8* Dn = L.Dn;
  float* us = L.us;
  float* dden_s = L.dden_s;
  float* dlog_s = L.dlog_s;

  const int bh = b * p.H + h;
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  const int64_t row = int64_t(bh) * p.nb + i;
  // the state: the KV head's over all keys (gated), or the map row's marginal sum (the map row is
  // the query row: a linear branch takes per-head maps)
  const int64_t srow = GATED ? int64_t(b) * p.Hkv + h / p.G : row;
  constexpr int kPer = D * D / 8 / kBwThreads;   // 16-byte chunks of a d x d tile per thread
  if constexpr (GATED) {
    // the KV head's fp32 state, converted to bf16 through registers, the thread's loads in flight
    // together
    const float* Sg = p.Sf + srow * D * D;
    bf16x8 x[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) x[u] = In<float>::load8(Sg + 8 * (t + kBwThreads * u));
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = t + kBwThreads * u;
      lds_store16(St + tpos<D>(e / (D / 8), e % (D / 8)), x[u]);
    }
  } else {
    // the row's bf16 sums straight from global memory to LDS (64-row tile copies)
    const bf16raw* Sg = reinterpret_cast<const bf16raw*>(p.S + row * D * D);
    const StageOff<D, kBwWaves> off = stage_offsets<D, false, kBwWaves>(D);
    stage_tile<bf16raw, D, false, kBwWaves>(Sg, D, 0, St, off);
    if constexpr (D > kBlock) stage_tile<bf16raw, D, false, kBwWaves>(Sg, D, 1, St + AttnTile<D>::kTileB, off);
  }
  for (int e = t; e < D; e += kBwThreads) us[e] = p.u[srow * D + e];
  SLA_WAIT_VMCNT(0);
  __syncthreads();

  const int tq = kBlock * i + 16 * w + l16;
  const bool qv = tq < p.n_valid;
  const T* Qr = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH + int64_t(tq) * p.qsN;
  const T* Or = static_cast<const T*>(p.o) + int64_t(b) * p.osB + int64_t(h) * p.osH + int64_t(tq) * p.osN;
  const T* Gr = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH + int64_t(tq) * p.dsN;

  // phi(q) of this lane's row: B operands (features 32 kc + 8 g .. + 7) and the fp32 denominator
  bf16x8 pqf[kKc];
  float den = 0.f, glog = 0.f;
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    float x[8];
    if (qv) In<T>::load8_f32(Qr + 32 * kc + 8 * g, x);
    else for (int m = 0; m < 8; ++m) x[m] = 0.f;
    f32x8 ph;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      ph[m] = qv ? phi(x[m]) : 0.f;           // padded rows take no part
      den += ph[m] * us[32 * kc + 8 * g + m];
      if constexpr (GATED) glog += x[m] * p.w_gate[int64_t(h) * D + 32 * kc + 8 * g + m];
    }
    pqf[kc] = cvt8(ph);
    lds_store16(Pq + tpos<D>(16 * w + l16, 4 * kc + g), pqf[kc]);
  }
  den = group4_sum(den);
  const float inv_den = (qv && den > 0.f) ? 1.f / den : 0.f;
  float gate = 1.f;
  if constexpr (GATED) gate = qv ? 1.f / (1.f + __expf(-group4_sum(glog))) : 0.f;

  // O_l^T = S_i^T phi(q)^T: lane holds O_l[t][c = 16 ct + 4 g + e]
  f32x4 xl[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) acc = mfma16(lds_load16(St + tpos<D>(16 * ct + l16, 4 * kc + g)), pqf[kc], acc);
    xl[ct] = acc * inv_den;
  }
  // D_t = dO . O_s; a = the gradient reaching O_l; dn = a / den; dden = -(a . O_l) / den
  float dsum = 0.f, ax = 0.f;
  f32x4 go[kCt], ga[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) go[ct] = qv ? load4_f32(Gr + 16 * ct + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (PROJ) {
    lds_u8* Wt = L.Wt;
    const float* Wg = p.proj_w + int64_t(h) * p.proj_sH;
    bf16x8 wx[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) wx[u] = In<float>::load8(Wg + 8 * (t + kBwThreads * u));
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = t + kBwThreads * u;
      lds_store16(Wt + tpos<D>(e / (D / 8), e % (D / 8)), wx[u]);
    }
    __syncthreads();
    const float* bias = p.proj_b != nullptr ? p.proj_b + int64_t(h) * (p.proj_sH != 0 ? D : 0) : nullptr;
#pragma unroll
    for (int ot = 0; ot < kCt; ++ot) {
      // Y^T[o][t] = sum_c W[o][c] O_l[t][c]: k-slots c = 32 kc + 4 g + {0..3} and + 16 (the lane's O_l)
      f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < kKc; ++kc) {
        const int o = 16 * ot + l16;
        const bf16x8 a = join(lds_load8(Wt + tpos<D>(o, 4 * kc + g / 2) + 8 * (g % 2)),
                              lds_load8(Wt + tpos<D>(o, 4 * kc + 2 + g / 2) + 8 * (g % 2)));
        y = mfma16(a, join(cvt4(xl[2 * kc]), cvt4(xl[2 * kc + 1])), y);
      }
      const int o0 = 16 * ot + 4 * g;        // lane holds Y[t][o0 + e]
      const f32x4 oo = qv ? load4_f32(Or + o0) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 bb = bias != nullptr ? *reinterpret_cast<const f32x4*>(bias + o0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += as_operand<T>(go[ot][e]) * (oo[e] - y[e] - bb[e]);
    }
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      // a^T[c][t] = sum_o W[o][c] dO[t][o]: A = W^T (transposing reads of rows o), B = the lane's dO
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ko = 0; ko < kKc; ++ko) {
        const bf16x8 a = join(lds_read_tr4(Wt + tr_addr<D>(32 * ko + 4 * g, 16 * ct, lane)),
                              lds_read_tr4(Wt + tr_addr<D>(32 * ko + 16 + 4 * g, 16 * ct, lane)));
        acc = mfma16(a, join(cvt4(go[2 * ko]), cvt4(go[2 * ko + 1])), acc);
      }
      ga[ct] = acc;
      *reinterpret_cast<bf16x4*>(p.xlin + (int64_t(bh) * p.N + tq) * D + 16 * ct + 4 * g) = cvt4(xl[ct]);
    }
  } else {
    // ungated: O_l = y; gated: O_l = gate y, the gradient reaching y is gate dO
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      const f32x4 oo = qv ? load4_f32(Or + 16 * ct + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += as_operand<T>(go[ct][e]) * (oo[e] - gate * xl[ct][e]);
      ga[ct] = go[ct] * gate;
    }
  }
  float dlogit = 0.f;
  if constexpr (GATED) {
    float gy = 0.f;                  // dO . y
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) gy += go[ct][e] * xl[ct][e];
    dlogit = group4_sum(gy) * gate * (1.f - gate);
  }
  f32x4 dn[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    const int c = 16 * ct + 4 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) ax += ga[ct][e] * xl[ct][e];
    dn[ct] = ga[ct] * inv_den;
    // dN tile [t][c]: 4 consecutive c = 8 bytes
    *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(Dn + tpos<D>(16 * w + l16, c / 8) + 2 * (c % 8)) =
        cvt4(dn[ct]);
  }
  dsum = group4_sum(dsum);
  ax = group4_sum(ax);
  const float dden = -ax * inv_den;
  Dt = qv ? dsum : 0.f;
  if (g == 0) {
    p.D[int64_t(bh) * p.N + tq] = Dt;
    dden_s[16 * w + l16] = dden;
    if constexpr (GATED) dlog_s[16 * w + l16] = qv ? dlogit : 0.f;
  }

  // dphi(q)^T[r][t] = sum_c S[r][c] dn[t][c] (+ u[r] dden): A = S (transposing reads of the
  // [c][r] tile, rows c paired as 16 (2 kc) + 4 g .. and 16 (2 kc + 1) + 4 g ..), B = dn
  const T* Qb = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) {
      const bf16x8 a = join(lds_read_tr4(St + tr_addr<D>(32 * kc + 4 * g, 16 * rt, lane)),
                            lds_read_tr4(St + tr_addr<D>(32 * kc + 16 + 4 * g, 16 * rt, lane)));
      acc = mfma16(a, join(cvt4(dn[2 * kc]), cvt4(dn[2 * kc + 1])), acc);
    }
    // lane holds dphi(q)^T[r = 16 rt + 4 g + e][t = 16 w + l16]
    const int r0 = 16 * rt + 4 * g;
    const f32x4 qx = qv ? load4_f32(Qb + int64_t(tq) * p.qsN + r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[e] = qv ? (acc[e] + us[r0 + e] * dden) * dphi(qx[e]) : 0.f;
      if constexpr (GATED) out[e] += qv ? dlogit * p.w_gate[int64_t(h) * D + r0 + e] : 0.f;
    }
    dql[rt] = out;
  }
  __syncthreads();                // phi(Q_i), dN_i and dden complete in LDS
  if constexpr (GATED) {
    // the gate weights' partial gradient of this query block: sum over its rows of dlogit_t q_t.
    // Thread t takes the 8-feature chunk t % kCh of rows t / kCh + kRg u (all its loads in flight
    // at once), then the kRg row groups are summed through LDS in a fixed order.
    constexpr int kCh = D / 8, kRg = kBwThreads / kCh, kPer = kBlock / kRg;
    const int ch = t % kCh, rg = t / kCh;
    float x[kPer][8];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      In<T>::load8_f32(Qb + int64_t(min(kBlock * i + rg + kRg * u, p.n_valid - 1)) * p.qsN + 8 * ch, x[u]);
    float s8[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) s8[m] = 0.f;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (kBlock * i + rg + kRg * u < p.n_valid) {
#pragma unroll
        for (int m = 0; m < 8; ++m) s8[m] += dlog_s[rg + kRg * u] * x[u][m];
      }
#pragma unroll
    for (int m = 0; m < 8; ++m) L.gred[rg * D + 8 * ch + m] = s8[m];
    __syncthreads();
    for (int r = t; r < D; r += kBwThreads) {
      float s = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < kRg; ++g2) s += L.gred[g2 * D + r];
      p.gpart[row * D + r] = s;
    }
  }

  // dS_i[r][c] = sum_t phi(q_t)[r] dn_t[c], stored [c][r]: wave w covers (rt, ct) tiles
  // n = w, w + 4, ... of the kCt x kCt grid; the k steps run over the 64 query rows
  u16* dSg = p.dS + row * D * D;
#pragma unroll
  for (int m = 0; m < kCt * kCt / kBwWaves; ++m) {
    const int n = w + kBwWaves * m, rt = n / kCt, ct = n % kCt;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 a = join(lds_read_tr4(Pq + tr_addr<D>(32 * kt + 8 * g, 16 * rt, lane)),
                            lds_read_tr4(Pq + tr_addr<D>(32 * kt + 8 * g + 4, 16 * rt, lane)));
      const bf16x8 bb = join(lds_read_tr4(Dn + tr_addr<D>(32 * kt + 8 * g, 16 * ct, lane)),
                             lds_read_tr4(Dn + tr_addr<D>(32 * kt + 8 * g + 4, 16 * ct, lane)));
      acc = mfma16(a, bb, acc);
    }
    // lane holds dS[r = 16 rt + 4 g + e][c = 16 ct + l16]: 4 consecutive r of row c of [c][r]
    *reinterpret_cast<bf16x4*>(dSg + int64_t(16 * ct + l16) * D + 16 * rt + 4 * g) = cvt4(acc);
  }
  // du_i[r] = sum_t phi(q_t)[r] dden_t
  for (int r = t; r < D; r += kBwThreads) {
    float s = 0.f;
    for (int tt = 0; tt < kBlock; ++tt) {
      const u16 bits = *reinterpret_cast<const __attribute__((address_space(3))) u16*>(
          Pq + tpos<D>(tt, r / 8) + 2 * (r % 8));
      s += bf16_to_f32(bits) * dden_s[tt];
    }
    p.du[row * D + r] = s;
  }
}

// One workgroup per (query block i, head): the linear query side as a pass of its own (with Proj,
// whose weight needs the LDS the dQ kernel uses for its tiles), writing the linear dQ of every row.
template <typename T, int D, bool PROJ, bool GATED>
__global__ __launch_bounds__(kBwThreads) void bwd_lin_q_kernel(BwdParams p) {
  constexpr int RB = 2 * D;
  constexpr int kCt = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char w_sm[PROJ ? D * RB : 16];  // W: [o][c]
  __shared__ __attribute__((aligned(1024))) unsigned char st_sm[D * RB];      // S_i^T: [c][r]
  __shared__ __attribute__((aligned(1024))) unsigned char pq_sm[kBlock * RB]; // phi(Q_i): [t][r]
  __shared__ __attribute__((aligned(1024))) unsigned char dn_sm[kBlock * RB]; // dN_i: [t][c]
  __shared__ float us[D];
  __shared__ float dden_s[kBlock];
  __shared__ float dlog_s[GATED ? kBlock : 1];
  __shared__ float gred[GATED ? kBwThreads / (D / 8) * D : 1];   // gate-gradient row-group sums
  const LinQLds L{to_lds(st_sm), to_lds(pq_sm), to_lds(dn_sm), to_lds(w_sm), us, dden_s, dlog_s, gred};
  const int i = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  f32x4 dql[kCt];
  float Dt;
  lin_q_side<T, D, PROJ, GATED>(p, b, h, i, L, dql, Dt);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int tq = kBlock * i + 16 * w + lane % 16;
  float* dqr = p.dq + (int64_t(bh) * p.N + tq) * D;
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) *reinterpret_cast<f32x4*>(dqr + 16 * rt + 4 * (lane / 16)) = dql[rt];
}

// ------------------------------------------------------------------ linear branch, key side

// The linear part of dK and dV for key block j of KV head g, wavefront w owning keys
// 64 j + 16 w + l % 16: dphi(k) = dH_j v + dz_j, dv = dH_j^T phi(k); with smooth-K, phi and its
// derivative at the shifted key k - mean.  dH_j and dz_j are summed over the query heads that read
// KV head g (one per head: each head has its own map and queries; SALAD: every key block reads its
// heads' one all-key state gradient).  The dK/dV kernel adds this in its epilogue; with smooth-K it
// runs as a pass of its own (bwd_lin_k_kernel).
__device__ __forceinline__ int64_t lin_k_srow(const BwdParams& p, int b, int h, int j) {
  const int64_t hrow = int64_t(b) * p.H + h;
  return p.gated ? hrow : hrow * p.nb + j;
}

// dH_j as the [c][r] tile of D rows (2 D bytes each) in two 64-row halves: rows c < 64 at lo, the
// others at hi (D = 64: lo only).  One query head per KV head: straight from global memory to LDS
// (the caller waits on vmcnt before its barrier); several: summed in fp32 through registers, every
// load of one head in flight together.
template <int D>
__device__ __forceinline__ void lin_k_stage_dh(const BwdParams& p, int b, int gk, int j, lds_u8* lo, lds_u8* hi) {
  const int h0 = gk * p.G;
  if (p.G == 1) {
    const bf16raw* src = reinterpret_cast<const bf16raw*>(p.dH + lin_k_srow(p, b, h0, j) * D * D);
    const StageOff<D, kBwWaves> off = stage_offsets<D, false, kBwWaves>(D);
    stage_tile<bf16raw, D, false, kBwWaves>(src, D, 0, lo, off);
    if constexpr (D > kBlock) stage_tile<bf16raw, D, false, kBwWaves>(src, D, 1, hi, off);
    return;
  }
  constexpr int kPer = D * D / 8 / kBwThreads;    // 16-byte chunks per thread
  const int t = threadIdx.x;
  float acc[kPer][8];
  for (int hh = 0; hh < p.G; ++hh) {
    const bf16raw* src = reinterpret_cast<const bf16raw*>(p.dH + lin_k_srow(p, b, h0 + hh, j) * D * D);
    float x[kPer][8];
#pragma unroll
    for (int u = 0; u < kPer; ++u) In<bf16raw>::load8_f32(src + 8 * (t + kBwThreads * u), x[u]);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[u][m] = hh == 0 ? x[u][m] : acc[u][m] + x[u][m];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int e = t + kBwThreads * u, c = e / (D / 8), r8 = e % (D / 8);
    f32x8 a8;
#pragma unroll
    for (int m = 0; m < 8; ++m) a8[m] = acc[u][m];
    lds_store16((c < kBlock ? lo : hi) + tpos<D>(c % kBlock, r8), cvt8(a8));
  }
}

// dz_j[r] for thread r < D (0 for the others)
__device__ __forceinline__ float lin_k_dz(const BwdParams& p, int b, int gk, int j, int D) {
  const int r = threadIdx.x;
  float z = 0.f;
  if (r < D)
    for (int hh = 0; hh < p.G; ++hh) z += p.dz[lin_k_srow(p, b, gk * p.G + hh, j) * D + r];
  return z;
}

// The linear branch's dK (with respect to the shifted key when smooth-K) and dV of this lane's key
// row s (Kr its row of K; kf, vf its K and V rows as the B operands; kv: s < n_valid), from the
// staged dH tile (lo, hi) and dzs: lk[rt][e] is column kcol(rt, g) + e of dK, lv[ct][e] column
// 16 ct + 4 g + e of dV; rows past n_valid get 0.
template <typename T, int D>
__device__ __forceinline__ void lin_k_grads(const BwdParams& p, int bh, const T* Kr, bool kv,
                                            const bf16x8 (&kf)[D / 32], const bf16x8 (&vf)[D / 32], lds_u8* lo,
                                            lds_u8* hi, const float* dzs, f32x4 (&lk)[D / 16],
                                            f32x4 (&lv)[D / 16]) {
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  const int lane = threadIdx.x % kWave, l16 = lane % 16, g = lane / 16;
  auto half = [&](int r) { return r < kBlock ? lo : hi; };   // the half that holds tile row r
  bf16x8 pkf[kKc];
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    float x[8];
    if constexpr (sizeof(T) == 2) {  // bf16 keys: the lane's K operand holds them exactly
#pragma unroll
      for (int m = 0; m < 8; ++m) x[m] = static_cast<float>(kf[kc][m]);
    } else if (kv) {
      In<T>::load8_f32(Kr + 32 * kc + 8 * g, x);
    }
    f32x8 ph;
#pragma unroll
    for (int m = 0; m < 8; ++m) ph[m] = kv ? phi(x[m] - (p.k_shift ? p.k_shift[int64_t(bh) * D + 32 * kc + 8 * g + m] : 0.f)) : 0.f;
    pkf[kc] = cvt8(ph);
  }
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) {
    // dphi(k)^T[r][s] = sum_c dH[r][c] v[s][c]: A = dH rows r (transposing reads of [c][r]), the
    // features r of tile rt in the kcol order
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) {
      const int c0 = 32 * kc + 8 * g;                 // rows c0 .. c0 + 7 lie in one half
      lds_u8* Hh = half(c0);
      const bf16x8 a = join(lds_read_tr4(Hh + tr_addr_kperm<D>(c0 % kBlock, rt, lane)),
                            lds_read_tr4(Hh + tr_addr_kperm<D>(c0 % kBlock + 4, rt, lane)));
      acc = mfma16(a, vf[kc], acc);
    }
    const int r0 = kcol(rt, g);       // lane holds features r0 .. r0 + 3 = elements 4 (rt % 2) .. of kf[rt / 2]
    f32x4 kx;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) kx[e] = static_cast<float>(kf[rt / 2][4 * (rt % 2) + e]);
    } else {
      kx = kv ? load4_f32(Kr + r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (p.k_shift != nullptr) kx -= *reinterpret_cast<const f32x4*>(p.k_shift + int64_t(bh) * D + r0);
#pragma unroll
    for (int e = 0; e < 4; ++e) lk[rt][e] = kv ? (acc[e] + dzs[r0 + e]) * dphi(kx[e]) : 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    // dv^T[c][s] = sum_r dH[r][c] phi(k)[s][r]: A = rows c of the [c][r] tile
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int c = 16 * ct + l16;
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) acc = mfma16(lds_load16(half(c) + tpos<D>(c % kBlock, 4 * kc + g)), pkf[kc], acc);
    lv[ct] = kv ? acc : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// The linear key side as a pass of its own (used with smooth-K, whose dK mean needs every row's
// linear dK before the sparse branch adds its part): one WG per (key block, KV head) writes dK, dV.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void bwd_lin_k_kernel(BwdParams p) {
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  constexpr int RB = 2 * D;
  __shared__ __attribute__((aligned(1024))) unsigned char dh_sm[D * RB];   // dH_j: [c][r]
  __shared__ float dzs[D];
  lds_u8* lo = to_lds(dh_sm);
  lds_u8* hi = lo + AttnTile<D>::kTileB;

  const int j = blockIdx.x, bh = blockIdx.y, b = bh / p.Hkv, gk = bh % p.Hkv;
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  lin_k_stage_dh<D>(p, b, gk, j, lo, hi);
  const float z = lin_k_dz(p, b, gk, j, D);
  if (t < D) dzs[t] = z;
  SLA_WAIT_VMCNT(0);
  SLA_WAIT_LGKM0();
  SLA_BARRIER();

  const int s = kBlock * j + 16 * w + l16;
  const bool kv = s < p.n_valid;
  const T* Kr = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(gk) * p.ksH + int64_t(s) * p.ksN;
  const T* Vr = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(gk) * p.vsH + int64_t(s) * p.vsN;
  bf16x8 kf[kKc], vf[kKc];
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    kf[kc] = kv ? In<T>::load8(Kr + 32 * kc + 8 * g) : zero8();
    vf[kc] = kv ? In<T>::load8(Vr + 32 * kc + 8 * g) : zero8();
  }
  f32x4 lk[kCt], lv[kCt];
  lin_k_grads<T, D>(p, bh, Kr, kv, kf, vf, lo, hi, dzs, lk, lv);
  float* dkr = p.dk + (int64_t(bh) * p.N + s) * D;
  float* dvr = p.dv + (int64_t(bh) * p.N + s) * D;
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    *reinterpret_cast<f32x4*>(dkr + kcol(ct, g)) = lk[ct];
    *reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g) = lv[ct];
  }
}

// ------------------------------------------------------------------ Proj weight gradient

// Partial dW[o][c] = sum_t dO[t][o] O_l[t][c] and db[o] = sum_t dO[t][o] over one chunk of 16
// query blocks of one (batch, head): grid x = chunk (of the rows that share weight y), y = weight.
// Rows past n_valid take no part.  Partials are summed by proj_reduce_kernel in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void proj_grad_kernel(BwdParams p, int per_head, int chunks_per_bh,
                                                               float* __restrict__ partW, float* __restrict__ partB) {
  constexpr int kCt = D / 16;
  constexpr int kTiles = kCt * kCt / kBwWaves;   // 16 x 16 output tiles per wavefront
  __shared__ __attribute__((aligned(1024))) unsigned char g_sm[kBlock * 2 * D];   // dO: [t][o]
  __shared__ __attribute__((aligned(1024))) unsigned char x_sm[kBlock * 2 * D];   // O_l: [t][c]
  lds_u8* Gt = to_lds(g_sm);
  lds_u8* Xt = to_lds(x_sm);
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, g = lane / 16;
  const int y = blockIdx.y, x = blockIdx.x;
  const int bh_idx = x / chunks_per_bh, chunk = x % chunks_per_bh;
  const int b = per_head ? bh_idx : bh_idx / p.H, h = per_head ? y : bh_idx % p.H;
  const int bh = b * p.H + h;
  const T* G = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH;
  const bf16raw* X = reinterpret_cast<const bf16raw*>(p.xlin) + int64_t(bh) * p.N * D;
  f32x4 acc[kTiles];
#pragma unroll
  for (int n = 0; n < kTiles; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float bsum = 0.f;
  const int i0 = chunk * 16, i1 = min(p.nb, i0 + 16);
  for (int i = i0; i < i1; ++i) {
    __syncthreads();
    stage64<T, D>(G, p.dsN, kBlock * i, p.n_valid, Gt);
    stage64<bf16raw, D>(X, D, kBlock * i, p.n_valid, Xt);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kTiles; ++n) {
      const int tile = w * kTiles + n, ot = tile / kCt, ct = tile % kCt;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = join(lds_read_tr4(Gt + tr_addr<D>(32 * kt + 8 * g, 16 * ot, lane)),
                              lds_read_tr4(Gt + tr_addr<D>(32 * kt + 8 * g + 4, 16 * ot, lane)));
        const bf16x8 bb = join(lds_read_tr4(Xt + tr_addr<D>(32 * kt + 8 * g, 16 * ct, lane)),
                               lds_read_tr4(Xt + tr_addr<D>(32 * kt + 8 * g + 4, 16 * ct, lane)));
        acc[n] = mfma16(a, bb, acc[n]);
      }
    }
    if (t < D) {
      for (int tt = 0; tt < kBlock; ++tt)
        bsum += bf16_to_f32(*reinterpret_cast<const __attribute__((address_space(3))) u16*>(
            Gt + tpos<D>(tt, t / 8) + 2 * (t % 8)));
    }
  }
  const int64_t part = int64_t(y) * gridDim.x + x;
#pragma unroll
  for (int n = 0; n < kTiles; ++n) {
    const int tile = w * kTiles + n, ot = tile / kCt, ct = tile % kCt;
    // lane holds dW[o = 16 ot + 4 g + e][c = 16 ct + lane % 16]
#pragma unroll
    for (int e = 0; e < 4; ++e) partW[(part * D + 16 * ot + 4 * g + e) * D + 16 * ct + lane % 16] = acc[n][e];
  }
  if (t < D) partB[part * D + t] = bsum;
}

// s += x[0] + ... + x[n - 1] in this order, x[q] = p[q * stride]: loads issued 8 at a time, all in
// flight before their adds (one at a time would expose a memory latency per term).
__device__ __forceinline__ float ordered_sum(const float* __restrict__ p, int n, int64_t stride, float s) {
  constexpr int kU = 8;
  for (int q0 = 0; q0 < n; q0 += kU) {
    float x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = p[int64_t(min(q0 + u, n - 1)) * stride];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (q0 + u < n) s += x[u];
  }
  return s;
}

// out[y][e] = sum over the parts of weight y, in order.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const float* __restrict__ part, int parts, int len,
                                                          float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x, y = blockIdx.y;
  if (e >= len) return;
  out[int64_t(y) * len + e] = ordered_sum(part + int64_t(y) * parts * len + e, parts, len, 0.f);
}

// Smooth-K: the mean over the valid rows of the linear-branch dK of each head (the gradient that
// flows back through the key mean).  One workgroup per (8 features, head), strided fp32 sums then
// a fixed-order LDS tree.
__global__ __launch_bounds__(256) void dk_mean_kernel(const float* __restrict__ dk, int N, int d, int n_valid,
                                                      float* __restrict__ mean) {
  const int bh = blockIdx.y, r0 = 8 * blockIdx.x, t = threadIdx.x;
  float s[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) s[m] = 0.f;
  // rows t, t + 256, ...: 4 rows' loads in flight at a time, added in row order
  for (int row0 = t; row0 < n_valid; row0 += 4 * 256) {
    f32x4 a[4], b4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* src = dk + (int64_t(bh) * N + min(row0 + 256 * u, n_valid - 1)) * d + r0;
      a[u] = *reinterpret_cast<const f32x4*>(src);
      b4[u] = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (row0 + 256 * u < n_valid) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          s[m] += a[u][m];
          s[4 + m] += b4[u][m];
        }
      }
  }
  __shared__ float red[256][9];
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
  if (t < 8) mean[int64_t(bh) * d + r0 + t] = n_valid > 0 ? red[0][t] / float(n_valid) : 0.f;
}

// ------------------------------------------------------------------ sparse branch, dQ

// Zero rows r0 .. 63 of a tile (the padded rows of a partial block; a direct copy brings whatever
// the caller's padding holds).
template <int D>
__device__ __forceinline__ void zero_rows(lds_u8* tile, int r0) {
  constexpr int kChunks = D / 8;
  for (int e = threadIdx.x; e < (kBlock - r0) * kChunks; e += kBwThreads)
    lds_store16(tile + tpos<D>(r0 + e / kChunks, e % kChunks), zero8());
}

// One workgroup per (query block i, query head h); wavefront w owns query rows 64 i + 16 w + l % 16.
// Over the blocks of the row's map (the head's own, or its GQA group's): S^T = K Q^T,
// dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T, with K and V of the group's KV head.
// CAUSAL (NSA-style maps): key s of block j is allowed iff s <= t and (j is a selected block or
// t - s < window).  K and V tiles are double-buffered: the next block's direct-to-LDS copies run
// during this one.
// LINQ (1: row states, 2: gated): the linear query side (lin_q_side) runs first in the same
// workgroup, in the tile buffers, and gives the rows' D and linear dQ; dQ is then written once.
template <typename T, int D, bool CAUSAL, int LINQ>
__global__ __launch_bounds__(kBwThreads) void bwd_dq_kernel(BwdParams p) {
  using Tl = AttnTile<D>;
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char k_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char v_sm[2][Tl::kTileB];
  __shared__ float lq_us[LINQ ? D : 1];
  __shared__ float lq_dden[LINQ ? kBlock : 1];
  __shared__ float lq_dlog[LINQ == 2 ? kBlock : 1];
  __shared__ float lq_gred[LINQ == 2 ? kBwThreads / (D / 8) * D : 1];

  const int i = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int gk = h / p.G;                          // KV head
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  const int64_t row = (int64_t(b) * p.Hs + (p.group_map ? gk : h)) * p.nb + i;   // map row
  const int tq = kBlock * i + 16 * w + l16;
  const bool qv = tq < p.n_valid;
  const T* Qr = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH + int64_t(tq) * p.qsN;
  const T* Gr = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH + int64_t(tq) * p.dsN;
  const T* K = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(gk) * p.ksH;
  const T* V = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(gk) * p.vsH;
  const StageOff<D, kBwWaves> koff = stage_offsets<D, false, kBwWaves>(p.ksN);
  const StageOff<D, kBwWaves> voff = stage_offsets<D, false, kBwWaves>(p.vsN);

  const int cbeg = p.crit_rowptr[row], cend = p.crit_rowptr[row + 1];
  // the row's next valid block index at or after list position e (or -1), wave-uniform; sel: its
  // selected flag (causal maps)
  auto next_block = [&](int& e, bool& sel) -> int {
    while (e < cend) {
      const int jraw = __builtin_amdgcn_readfirstlane(p.crit_idx[e]);
      if constexpr (CAUSAL) sel = (__builtin_amdgcn_readfirstlane(int(p.crit_flags[e])) & 1) != 0;
      ++e;
      if (unsigned(jraw) < unsigned(p.nb)) return jraw;   // malformed entries are skipped
    }
    return -1;
  };
  f32x4 dql[kCt];
  float Dt_lin = 0.f;
  if constexpr (LINQ != 0) {         // St in the K buffers (D rows of 2 D bytes), Pq and Dn in the V buffers
    const LinQLds L{to_lds(k_sm[0]), to_lds(v_sm[0]), to_lds(v_sm[1]), nullptr, lq_us, lq_dden, lq_dlog, lq_gred};
    lin_q_side<T, D, false, LINQ == 2>(p, b, h, i, L, dql, Dt_lin);
    SLA_WAIT_LGKM0();
    SLA_BARRIER();                   // the tile buffers are free again
  }
  int epos = cbeg;
  bool sel_cur = true, sel_nxt = true;
  int cur = next_block(epos, sel_cur);
  if (cur >= 0) {
    stage_tile<T, D, false, kBwWaves>(K, p.ksN, cur, to_lds(k_sm[0]), koff);
    stage_tile<T, D, false, kBwWaves>(V, p.vsN, cur, to_lds(v_sm[0]), voff);
  }
  bf16x8 qf[kKc], gf[kKc];
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    qf[kc] = qv ? In<T>::load8(Qr + 32 * kc + 8 * g) : zero8();
    gf[kc] = qv ? In<T>::load8(Gr + 32 * kc + 8 * g) : zero8();
  }
  const float lse_raw = qv ? p.lse[int64_t(bh) * p.N + tq] : -__builtin_inff();
  const bool has = qv && lse_raw > -__builtin_inff();
  const float lse2 = has ? lse_raw * kLog2e : 0.f;
  const float Dt = LINQ != 0 ? Dt_lin : (qv ? p.D[int64_t(bh) * p.N + tq] : 0.f);
  const float c2 = p.scale_log2;

  f32x4 acc[kCt];
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int buf = 0;
  while (cur >= 0) {
    const int nxt = next_block(epos, sel_nxt);
    lds_u8* Kt = to_lds(k_sm[buf]);
    lds_u8* Vt = to_lds(v_sm[buf]);
    SLA_WAIT_VMCNT(0);               // this block's copies have landed ...
    SLA_WAIT_LGKM0();
    SLA_BARRIER();                   // ... for every wavefront, and the other buffer is free
    const int rv = p.n_valid - kBlock * cur;
    if (rv < kBlock) {               // padded keys: zero their K and V rows
      zero_rows<D>(Kt, rv);
      zero_rows<D>(Vt, rv);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
    }
    if (nxt >= 0) {
      stage_tile<T, D, false, kBwWaves>(K, p.ksN, nxt, to_lds(k_sm[buf ^ 1]), koff);
      stage_tile<T, D, false, kBwWaves>(V, p.vsN, nxt, to_lds(v_sm[buf ^ 1]), voff);
    }
    bf16x4 dsb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < kKc; ++kc) {
        sacc = mfma16(lds_load16(Kt + tpos<D>(16 * st + l16, 4 * kc + g)), qf[kc], sacc);
        pacc = mfma16(lds_load16(Vt + tpos<D>(16 * st + l16, 4 * kc + g)), gf[kc], pacc);
      }
      // lane holds S^T[s = 16 st + 4 g + e][t]
      f32x4 ds;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bool ok = has && 16 * st + 4 * g + e4 < rv;
        if constexpr (CAUSAL) {
          const int sk = kBlock * cur + 16 * st + 4 * g + e4;
          ok = ok && sk <= tq && (sel_cur || tq - sk < p.window);
        }
        const float pr = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e4], c2, -lse2)) : 0.f;
        ds[e4] = ok ? pr * (pacc[e4] - Dt) : 0.f;
      }
      dsb[st] = cvt4(ds);
    }
    // dQ^T[r][t] += sum_s K[s][r] dS^T[s][t]: k-slots = keys 16 st + 4 g + 0..3 of a pair of tiles
#pragma unroll
    for (int rt = 0; rt < kCt; ++rt)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const bf16x8 a = join(lds_read_tr4(Kt + tr_addr<D>(32 * pr + 4 * g, 16 * rt, lane)),
                              lds_read_tr4(Kt + tr_addr<D>(32 * pr + 16 + 4 * g, 16 * rt, lane)));
        acc[rt] = mfma16(a, join(dsb[2 * pr], dsb[2 * pr + 1]), acc[rt]);
      }
    cur = nxt;
    sel_cur = sel_nxt;
    buf ^= 1;
  }
  // lane holds dQ^T[r = 16 rt + 4 g + e][t]: added to the linear part, or written (no linear branch;
  // padded rows then get their zeros here)
  float* dqr = p.dq + (int64_t(bh) * p.N + tq) * D;
  if constexpr (LINQ != 0) {         // linear part + sparse part, every row written (padded: 0)
#pragma unroll
    for (int rt = 0; rt < kCt; ++rt)
      *reinterpret_cast<f32x4*>(dqr + 16 * rt + 4 * g) = qv ? dql[rt] + acc[rt] * p.scale : f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (p.overwrite) {
#pragma unroll
    for (int rt = 0; rt < kCt; ++rt)
      *reinterpret_cast<f32x4*>(dqr + 16 * rt + 4 * g) = qv ? acc[rt] * p.scale : f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (qv) {
#pragma unroll
    for (int rt = 0; rt < kCt; ++rt) {
      f32x4* q4 = reinterpret_cast<f32x4*>(dqr + 16 * rt + 4 * g);
      *q4 = *q4 + acc[rt] * p.scale;
    }
  }
}

// ------------------------------------------------------------------ sparse branch, dK and dV

// Dispatch order of the dK/dV workgroups: key-block rows sorted by how many query blocks list them
// (counted by crit_transpose_kernel), most-used first, so the longest workgroups start first and
// the round-robin dispatch spreads them over the XCDs.  One workgroup: a histogram of the counts in
// LDS, a descending scan (one wavefront: per-lane runs, then a wave scan of the run sums), a scatter (the order within one count is arbitrary; results do not depend
// on the order).  Counts above max_count <= 4096 rank as max_count.
__global__ __launch_bounds__(1024) void kv_order_kernel(const int* __restrict__ counts, int rows, int max_count,
                                                        int* __restrict__ order) {
  __shared__ int hist[kMaxKeyBlocksBwd + 2];
  const int t = threadIdx.x;
  for (int c = t; c <= max_count + 1; c += 1024) hist[c] = 0;
  __syncthreads();
  for (int r = t; r < rows; r += 1024) atomicAdd(&hist[min(counts[r], max_count)], 1);
  __syncthreads();
  if (t < kWave) {                                // exclusive scan from the largest count down:
    const int n = max_count + 1;                  // lane l takes descending positions l*per .. l*per+per-1
    const int per = (n + kWave - 1) / kWave;      // (count = max_count - position)
    int sum = 0;
    for (int k = 0; k < per; ++k) {
      const int pos = t * per + k;
      if (pos < n) sum += hist[max_count - pos];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (t >= off) incl += y;
    }
    int run = incl - sum;
    for (int k = 0; k < per; ++k) {
      const int pos = t * per + k;
      if (pos < n) {
        const int c = max_count - pos;
        const int h = hist[c];
        hist[c] = run;
        run += h;
      }
    }
  }
  __syncthreads();
  for (int r = t; r < rows; r += 1024) order[atomicAdd(&hist[min(counts[r], max_count)], 1)] = r;
}

// One workgroup per (key block j, KV head g); wavefront w owns keys 64 j + 16 w + l % 16.  Over
// the query heads h of the group and, for each, the query blocks i whose map row lists j:
// S = Q K^T, dP = dO V^T, dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.  Q, dO tiles and the
// rows' log-sum-exp and D are double-buffered: the next (head, query block)'s direct-to-LDS copies
// run during this one.  CAUSAL: the masks of the dQ kernel (s <= t and (selected or t - s < window)).
// LIN: the linear branch's key side (lin_k_stage_dh / lin_k_grads; not with smooth-K) is added in
// this kernel's epilogue, so dK and dV are written once; dH_j and dz_j are requested during the
// last listed block.
template <typename T, int D, bool CAUSAL, bool LIN>
__global__ __launch_bounds__(kBwThreads) void bwd_dkdv_kernel(BwdParams p) {
  using Tl = AttnTile<D>;
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char q_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char g_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(256))) float lse_s[2][kBlock];
  __shared__ __attribute__((aligned(256))) float d_s[2][kBlock];

  const int krow = p.kv_order[blockIdx.x / p.hsplit];   // (b, g, j), most-used key blocks first
  const int hs = blockIdx.x % p.hsplit;                  // this workgroup's subset of the group's heads
  const int j = krow % p.nb, bk = krow / p.nb, b = bk / p.Hkv, gk = bk % p.Hkv;
  const int t = threadIdx.x, lane = t % kWave, l16 = lane % 16, g = lane / 16;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);
  const int s = kBlock * j + 16 * w + l16;
  const bool kv = s < p.n_valid;
  const T* Kr = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(gk) * p.ksH + int64_t(s) * p.ksN;
  const T* Vr = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(gk) * p.vsH + int64_t(s) * p.vsN;
  const StageOff<D, kBwWaves> qoff = stage_offsets<D, false, kBwWaves>(p.qsN);
  const StageOff<D, kBwWaves> goff = stage_offsets<D, false, kBwWaves>(p.dsN);
  const int Gs = p.G / p.hsplit;                         // heads per subset
  const int h0 = gk * p.G + hs * Gs;

  // the (head, query block) pairs that list j, heads ascending (the subset's), then query blocks
  // ascending: a wave-uniform scan of the transposed bit rows (the group's one row per head with
  // shared maps)
  int hh = 0, word = 0;
  uint32_t m = 0u, msel = 0u;
  auto next_block = [&](int& head, bool& sel) -> int {
    while (m == 0u) {
      if (word >= p.wq) {
        if (hh + 1 >= Gs) return -1;
        ++hh;
        word = 0;
        continue;
      }
      const int64_t brow = (int64_t(b) * p.Hs + (p.group_map ? gk : h0 + hh)) * p.nb + j;
      m = __builtin_amdgcn_readfirstlane(p.critT[brow * p.wq + word]);
      if constexpr (CAUSAL) msel = __builtin_amdgcn_readfirstlane(p.critT_sel[brow * p.wq + word]);
      ++word;
    }
    const int bit = __builtin_ctz(m);
    m &= m - 1u;
    head = h0 + hh;
    if constexpr (CAUSAL) sel = ((msel >> bit) & 1u) != 0u;
    return 32 * (word - 1) + bit;
  };
  // copies of query block i of head h into buffer bf: Q and dO tiles by every wavefront, the 64
  // rows' log-sum-exp and D (256 bytes each) by wavefront 0
  auto stage = [&](int i, int h, int bf) {
    const T* Q = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
    const T* G = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH;
    stage_tile<T, D, false, kBwWaves>(Q, p.qsN, i, to_lds(q_sm[bf]), qoff);
    stage_tile<T, D, false, kBwWaves>(G, p.dsN, i, to_lds(g_sm[bf]), goff);
    if (w == 0) {
      const int64_t r0 = (int64_t(b) * p.H + h) * p.N + kBlock * i;
      load_lds4_sbase(p.lse + r0, uint32_t(4 * lane), to_lds(lse_s[bf]));
      load_lds4_sbase(p.D + r0, uint32_t(4 * lane), to_lds(d_s[bf]));
    }
  };
  int h_cur = h0, h_nxt = h0;
  bool sel_cur = true, sel_nxt = true;
  int cur = next_block(h_cur, sel_cur);
  if (cur >= 0) stage(cur, h_cur, 0);

  bf16x8 kf[kKc], vf[kKc];
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    kf[kc] = kv ? In<T>::load8(Kr + 32 * kc + 8 * g) : zero8();
    vf[kc] = kv ? In<T>::load8(Vr + 32 * kc + 8 * g) : zero8();
  }
  const float c2 = p.scale_log2;
  f32x4 dk[kCt], dv[kCt];
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    dk[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the first of the 4 dK features a lane holds in tile ct: the kcol order with the linear epilogue
  // (faster there, and the epilogue needs it), the plain order otherwise (2% faster for NSA-style maps)
  auto dcol = [&](int ct) { return LIN ? kcol(ct, g) : 16 * ct + 4 * g; };
  int buf = 0;
  int dh_buf = -1;                   // LIN: the buffer pair that received dH_j during the last block
  float dzv = 0.f;                   // LIN: dz_j[t], requested before the loop
  if constexpr (LIN) {
    if (hs == 0) dzv = lin_k_dz(p, b, gk, j, D);
  }
  while (cur >= 0) {
    const int nxt = next_block(h_nxt, sel_nxt);
    lds_u8* Qt = to_lds(q_sm[buf]);
    lds_u8* Gt = to_lds(g_sm[buf]);
    SLA_WAIT_VMCNT(0);               // this block's copies have landed ...
    SLA_WAIT_LGKM0();
    SLA_BARRIER();                   // ... for every wavefront, and the other buffer is free
    const int rq = p.n_valid - kBlock * cur;     // valid query rows of this block
    if (rq < kBlock) {               // padded queries: zero their Q and dO rows
      zero_rows<D>(Qt, rq);
      zero_rows<D>(Gt, rq);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
    }
    if (nxt >= 0) {
      stage(nxt, h_nxt, buf ^ 1);
    } else if constexpr (LIN) {      // last block: the linear part's dH_j and dz_j into the free buffers
      if (hs == 0 && p.G == 1) {
        lin_k_stage_dh<D>(p, b, gk, j, to_lds(q_sm[buf ^ 1]), to_lds(g_sm[buf ^ 1]));
        dh_buf = buf ^ 1;
      }
    }
    bf16x4 pb[4], db[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f}, pacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < kKc; ++kc) {
        sacc = mfma16(lds_load16(Qt + tpos<D>(16 * tt + l16, 4 * kc + g)), kf[kc], sacc);
        pacc = mfma16(lds_load16(Gt + tpos<D>(16 * tt + l16, 4 * kc + g)), vf[kc], pacc);
      }
      // lane holds S[t = 16 tt + 4 g + e][s]; rows without allowed keys or past n_valid get P = 0
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse_s[buf][16 * tt + 4 * g]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&d_s[buf][16 * tt + 4 * g]);
      f32x4 pr, ds;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bool ok = kv && 16 * tt + 4 * g + e4 < rq && l4[e4] > -__builtin_inff();
        if constexpr (CAUSAL) {
          const int tq = kBlock * cur + 16 * tt + 4 * g + e4;
          ok = ok && s <= tq && (sel_cur || tq - s < p.window);
        }
        pr[e4] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e4], c2, -l4[e4] * kLog2e)) : 0.f;
        ds[e4] = ok ? pr[e4] * (pacc[e4] - d4[e4]) : 0.f;
      }
      pb[tt] = cvt4(pr);
      db[tt] = cvt4(ds);
    }
    // dV^T[c][s] += sum_t dO[t][c] P[t][s]; dK^T[r][s] += sum_t Q[t][r] dS[t][s] (LIN: r in the kcol order)
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const bf16x8 ag = join(lds_read_tr4(Gt + tr_addr<D>(32 * pr + 4 * g, 16 * ct, lane)),
                               lds_read_tr4(Gt + tr_addr<D>(32 * pr + 16 + 4 * g, 16 * ct, lane)));
        dv[ct] = mfma16(ag, join(pb[2 * pr], pb[2 * pr + 1]), dv[ct]);
        bf16x8 aq;
        if constexpr (LIN)
          aq = join(lds_read_tr4(Qt + tr_addr_kperm<D>(32 * pr + 4 * g, ct, lane)),
                    lds_read_tr4(Qt + tr_addr_kperm<D>(32 * pr + 16 + 4 * g, ct, lane)));
        else
          aq = join(lds_read_tr4(Qt + tr_addr<D>(32 * pr + 4 * g, 16 * ct, lane)),
                    lds_read_tr4(Qt + tr_addr<D>(32 * pr + 16 + 4 * g, 16 * ct, lane)));
        dk[ct] = mfma16(aq, join(db[2 * pr], db[2 * pr + 1]), dk[ct]);
      }
    cur = nxt;
    h_cur = h_nxt;
    sel_cur = sel_nxt;
    buf ^= 1;
  }
  float* dkr = p.dk + (int64_t(bk) * p.N + s) * D;
  float* dvr = p.dv + (int64_t(bk) * p.N + s) * D;
  f32x4 lk[kCt], lv[kCt];
  if constexpr (LIN) {
    if (hs == 0) {                   // once per key row: the first head subset's workgroup
      lds_u8* lo = to_lds(dh_buf >= 0 ? q_sm[dh_buf] : q_sm[0]);
      lds_u8* hi = to_lds(dh_buf >= 0 ? g_sm[dh_buf] : q_sm[1]);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();                 // every wavefront is done with the last block's tiles and lse_s
      if (dh_buf < 0) lin_k_stage_dh<D>(p, b, gk, j, lo, hi);   // several query heads, or no listing block
      float* dzs = &lse_s[0][0];     // D floats
      if (t < D) dzs[t] = dzv;
      SLA_WAIT_VMCNT(0);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
      lin_k_grads<T, D>(p, bk, Kr, kv, kf, vf, lo, hi, dzs, lk, lv);
    }
  }
  if (p.hsplit > 1) {                // a subset's partial sums, added up by dkdv_combine_kernel
    if constexpr (LIN) {
      if (hs == 0) {                 // the linear part is written first; the combine adds the partials
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) {
          *reinterpret_cast<f32x4*>(dkr + kcol(ct, g)) = lk[ct];
          *reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g) = lv[ct];
        }
      }
    }
    const int64_t off = ((int64_t(hs) * p.B * p.Hkv + bk) * p.N + s) * D;
    float* pk = p.part_k + off;
    float* pv = p.part_v + off;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      *reinterpret_cast<f32x4*>(pk + dcol(ct)) = kv ? dk[ct] * p.scale : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(pv + 16 * ct + 4 * g) = kv ? dv[ct] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  if constexpr (LIN) {               // linear part + sparse part, every row written (padded: 0)
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      *reinterpret_cast<f32x4*>(dkr + kcol(ct, g)) = kv ? lk[ct] + dk[ct] * p.scale : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g) = kv ? lv[ct] + dv[ct] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  } else if (p.overwrite) {          // no linear branch: this kernel writes every row (padded: 0)
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      *reinterpret_cast<f32x4*>(dkr + dcol(ct)) = kv ? dk[ct] * p.scale : f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g) = kv ? dv[ct] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  } else if (kv) {
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      f32x4* k4 = reinterpret_cast<f32x4*>(dkr + dcol(ct));
      f32x4* v4 = reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g);
      f32x4 add = dk[ct] * p.scale;
      // smooth-K: the linear branch saw k - mean(k), so its dK loses its own mean over the valid rows
      if (p.dk_mean != nullptr) add -= *reinterpret_cast<const f32x4*>(p.dk_mean + int64_t(bk) * D + dcol(ct));
      *k4 = *k4 + add;
      *v4 = *v4 + dv[ct];
    }
  }
}

// D_t = dO_t . O_t for every row (no linear branch: O_sparse = O): 16 lanes per row, fp32 sums.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dot_kernel(BwdParams p, int rows) {
  const int r = blockIdx.x * 16 + int(threadIdx.x) / 16, l = int(threadIdx.x) % 16;
  if (r >= rows) return;
  const int tq = r % p.N, bh = r / p.N, b = bh / p.H, h = bh % p.H;
  float acc = 0.f;
  if (tq < p.n_valid) {
    const T* Or = static_cast<const T*>(p.o) + int64_t(b) * p.osB + int64_t(h) * p.osH + int64_t(tq) * p.osN;
    const T* Gr = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH + int64_t(tq) * p.dsN;
#pragma unroll
    for (int c = 8 * l; c < D; c += 128) {
      float x[8], y[8];
      In<T>::load8_f32(Or + c, x);
      In<T>::load8_f32(Gr + c, y);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc += x[m] * as_operand<T>(y[m]);
    }
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off);
  if (l == 0) p.D[r] = acc;
}

// SALAD: dw_gate[h][r] = sum over b and the query blocks i of gpart[(b, h, i)][r].  One workgroup
// per (head, 8 features): thread t sums the rows (b, i) with b nb + i = t, t + 256, ... (4 rows'
// loads in flight at a time), then a fixed-order LDS tree over the threads (deterministic).
__global__ __launch_bounds__(256) void gate_reduce_kernel(const float* __restrict__ gpart, int B, int H, int nb, int d,
                                                          float* __restrict__ out) {
  const int h = blockIdx.y, r0 = 8 * blockIdx.x, t = threadIdx.x;
  const int rows = B * nb;
  float s[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) s[m] = 0.f;
  for (int q0 = t; q0 < rows; q0 += 4 * 256) {
    f32x4 a[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = min(q0 + 256 * u, rows - 1), b = q / nb, i = q % nb;
      const float* src = gpart + ((int64_t(b) * H + h) * nb + i) * d + r0;
      a[u] = *reinterpret_cast<const f32x4*>(src);
      c[u] = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (q0 + 256 * u < rows) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          s[m] += a[u][m];
          s[4 + m] += c[u][m];
        }
      }
  }
  __shared__ float red[256][9];
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
  if (t < 8) out[int64_t(h) * d + r0 + t] = red[0][t];
}

// dK and dV from the head subsets' partials (hsplit > 1): summed in subset order, then written (no
// linear branch) or added to the linear part (valid rows; with smooth-K minus the mean of that
// part), as the dK/dV kernel does without a split.  One thread per 4 features of a row.
__global__ __launch_bounds__(256) void dkdv_combine_kernel(BwdParams p, int D) {
  const int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t total = int64_t(p.B) * p.Hkv * p.N * D;
  if (e >= total) return;
  const int64_t rowi = e / D;
  const int bk = int(rowi / p.N), s = int(rowi % p.N), c = int(e % D);
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int hs = 0; hs < p.hsplit; ++hs) {
    sk += *reinterpret_cast<const f32x4*>(p.part_k + hs * total + e);
    sv += *reinterpret_cast<const f32x4*>(p.part_v + hs * total + e);
  }
  f32x4* k4 = reinterpret_cast<f32x4*>(p.dk + e);
  f32x4* v4 = reinterpret_cast<f32x4*>(p.dv + e);
  if (p.overwrite) {
    *k4 = sk;                        // padded rows: the partials are 0
    *v4 = sv;
  } else if (s < p.n_valid) {
    if (p.dk_mean != nullptr) sk -= *reinterpret_cast<const f32x4*>(p.dk_mean + int64_t(bk) * D + c);
    *k4 = *k4 + sk;
    *v4 = *v4 + sv;
  }
}

// One bit per query block of every row: word w of a row holds blocks 32 w .. 32 w + 31 below nb.
__global__ __launch_bounds__(256) void ones_bits_kernel(uint32_t* __restrict__ bits, int rows, int nb, int wq) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= int64_t(rows) * wq) return;
  const int word = int(e % wq), n = min(32, nb - 32 * word);
  bits[e] = n >= 32 ? ~0u : (1u << n) - 1u;
}

struct BwdWs {
  float* D;
  u16* dS;
  float* du;
  u16* dH;
  float* dz;
  uint32_t* critT;
  uint32_t* critT_sel;
  uint32_t* margT;
  int* kv_counts;
  int* kv_order;
  float* dk_mean;
  u16* xlin;
  float* partW;
  float* partB;
  float* gpart;
  float* part_k;
  float* part_v;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// dK/dV workgroups per key block.  A key block's work is every (head, query block) pair that lists
// it, G heads per KV head: with few key-block rows (one wave of workgroups or less) the most-listed
// block alone sets the kernel's time (at the NSA prefill: 114 listing query blocks x 16 heads against
// 24 x 16 on average), so the group's heads are split over 2 or 4 workgroups whose partial sums a
// second kernel adds up in a fixed order.
static int bwd_hsplit(int B, int Hq, int Hkv, int nb) {
  const int G = Hq / Hkv;
  if (G < 2 || int64_t(B) * Hkv * nb >= 2048) return 1;
  return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
}

constexpr int kProjChunk = 16;   // query blocks per partial of the Proj weight gradient

// The shapes a backward call works on: B, Hq query heads, Hkv KV heads, Hs map heads, N, d.
struct BwdShape {
  int B, Hq, Hkv, Hs, N, d, lin, causal, proj;
};

static size_t bwd_ws_layout(const BwdShape& sh, BwdWs* ws, void* base) {
  const int64_t nb = sh.N / kBlock, wq = (nb + 31) / 32;
  const int64_t qrows = int64_t(sh.B) * sh.Hq * nb;          // query-head rows (b, h, i)
  const int64_t mrows = int64_t(sh.B) * sh.Hs * nb;          // map rows
  const int64_t krows = int64_t(sh.B) * sh.Hkv * nb;         // key-block rows (b, g, j)
  const bool lin = sh.lin != SLA_LIN_NONE, gated = sh.lin == SLA_LIN_GLOBAL_GATED;
  const int64_t hrows = gated ? int64_t(sh.B) * sh.Hq : qrows;   // rows of dH, dz
  const int64_t parts = sh.proj ? int64_t(sh.B) * sh.Hq * ((nb + kProjChunk - 1) / kProjChunk) : 0;
  const size_t d = size_t(sh.d);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t oD = take(size_t(sh.B) * sh.Hq * sh.N * 4);
  const size_t odS = take(lin ? size_t(qrows) * d * d * 2 : 0);
  const size_t odu = take(lin ? size_t(qrows) * d * 4 : 0);
  const size_t odH = take(lin ? size_t(hrows) * d * d * 2 : 0);
  const size_t odz = take(lin ? size_t(hrows) * d * 4 : 0);
  const size_t oc = take(size_t(mrows) * wq * 4);
  const size_t ocs = take(sh.causal ? size_t(mrows) * wq * 4 : 0);
  // transposed marginal masks, or (gated) the all-ones masks of the per-head state sums
  const size_t om = take(sh.lin == SLA_LIN_ROW_STATES ? size_t(qrows) * wq * 4
                                                      : gated ? size_t(sh.B) * sh.Hq * wq * 4 : 0);
  const size_t okc = take(size_t(krows) * 4);
  const size_t oko = take(size_t(krows) * 4);
  const size_t okm = take(lin ? size_t(sh.B) * sh.Hkv * d * 4 : 0);
  const size_t ox = take(sh.proj ? size_t(sh.B) * sh.Hq * sh.N * d * 2 : 0);
  const size_t opw = take(size_t(parts) * d * d * 4);
  const size_t opb = take(size_t(parts) * d * 4);
  const size_t og = take(gated ? size_t(qrows) * d * 4 : 0);
  const int hsplit = bwd_hsplit(sh.B, sh.Hq, sh.Hkv, int(nb));
  const size_t npart = hsplit > 1 ? size_t(hsplit) * sh.B * sh.Hkv * sh.N * d : 0;
  const size_t opk = take(npart * 4);
  const size_t opv = take(npart * 4);
  if (ws != nullptr) {
    unsigned char* p = static_cast<unsigned char*>(base);
    ws->D = reinterpret_cast<float*>(p + oD);
    ws->dS = reinterpret_cast<u16*>(p + odS);
    ws->du = reinterpret_cast<float*>(p + odu);
    ws->dH = reinterpret_cast<u16*>(p + odH);
    ws->dz = reinterpret_cast<float*>(p + odz);
    ws->critT = reinterpret_cast<uint32_t*>(p + oc);
    ws->critT_sel = reinterpret_cast<uint32_t*>(p + ocs);
    ws->margT = reinterpret_cast<uint32_t*>(p + om);
    ws->kv_counts = reinterpret_cast<int*>(p + okc);
    ws->kv_order = reinterpret_cast<int*>(p + oko);
    ws->dk_mean = reinterpret_cast<float*>(p + okm);
    ws->xlin = reinterpret_cast<u16*>(p + ox);
    ws->partW = reinterpret_cast<float*>(p + opw);
    ws->partB = reinterpret_cast<float*>(p + opb);
    ws->gpart = reinterpret_cast<float*>(p + og);
    ws->part_k = reinterpret_cast<float*>(p + opk);
    ws->part_v = reinterpret_cast<float*>(p + opv);
  }
  return off;
}

// The query side: with a linear branch and no Proj, the dQ kernel that also does the linear query
// side (dQ complete after it); with Proj, the linear query side as a pass of its own (the dQ kernel
// follows with the key side); without a linear branch, D = dO . O.
template <typename T, int D>
static void launch_bwd_q_side(const BwdParams& p, int B, hipStream_t st) {
  const dim3 grid(p.nb, B * p.H);
  if (p.gated) bwd_dq_kernel<T, D, false, 2><<<grid, kBwThreads, 0, st>>>(p);
  else if (p.proj_w != nullptr) bwd_lin_q_kernel<T, D, true, false><<<grid, kBwThreads, 0, st>>>(p);
  else if (p.S != nullptr) bwd_dq_kernel<T, D, false, 1><<<grid, kBwThreads, 0, st>>>(p);
  else {
    const int rows = B * p.H * p.N;
    bwd_dot_kernel<T, D><<<dim3((rows + 15) / 16), 256, 0, st>>>(p, rows);
  }
}

template <typename T, int D>
static void launch_bwd_k_side(const BwdParams& p, int B, bool lin, hipStream_t st) {
  const int BK = B * p.Hkv;
  // with smooth-K the linear dK's mean over all rows is needed before the sparse part is added, so
  // the linear key side runs first as a pass of its own; otherwise the dK/dV kernel adds it
  const bool fused = lin && p.dk_mean == nullptr;
  if (lin && !fused) {
    bwd_lin_k_kernel<T, D><<<dim3(p.nb, BK), kBwThreads, 0, st>>>(p);
    dk_mean_kernel<<<dim3(D / 8, BK), 256, 0, st>>>(p.dk, p.N, D, p.n_valid, const_cast<float*>(p.dk_mean));
  }
  const dim3 qgrid(p.nb, B * p.H);
  const dim3 kgrid(p.nb * BK * p.hsplit);
  if (p.critT_sel != nullptr) {
    bwd_dq_kernel<T, D, true, 0><<<qgrid, kBwThreads, 0, st>>>(p);
    bwd_dkdv_kernel<T, D, true, false><<<kgrid, kBwThreads, 0, st>>>(p);
  } else {
    // with a linear branch and no Proj the query side's kernel has written dQ already
    if (!lin || p.proj_w != nullptr) bwd_dq_kernel<T, D, false, 0><<<qgrid, kBwThreads, 0, st>>>(p);
    if (fused) bwd_dkdv_kernel<T, D, false, true><<<kgrid, kBwThreads, 0, st>>>(p);
    else bwd_dkdv_kernel<T, D, false, false><<<kgrid, kBwThreads, 0, st>>>(p);
  }
  if (p.hsplit > 1) {
    const int64_t quads = int64_t(B) * p.Hkv * p.N * D / 4;
    dkdv_combine_kernel<<<dim3(uint32_t((quads + 255) / 256)), 256, 0, st>>>(p, D);
  }
}

// dW (and db) of the Proj layer: partials over chunks of query blocks, then their ordered sums.
template <typename T, int D>
static void launch_proj_grad(const BwdParams& p, int B, int per_head, const BwdWs& ws, float* dw, float* db,
                             hipStream_t st) {
  const int chunks = (p.nb + kProjChunk - 1) / kProjChunk;
  const int weights = per_head ? p.H : 1;
  const int parts = (per_head ? B : B * p.H) * chunks;
  proj_grad_kernel<T, D><<<dim3(parts, weights), kBwThreads, 0, st>>>(p, per_head, chunks, ws.partW, ws.partB);
  proj_reduce_kernel<<<dim3((D * D + 255) / 256, weights), 256, 0, st>>>(ws.partW, parts, D * D, dw);
  if (db != nullptr) proj_reduce_kernel<<<dim3(1, weights), 256, 0, st>>>(ws.partB, parts, D, db);
}

template <typename F>
static void by_type(int dtype, int d, F&& f) {
  // f is a generic lambda called with (T{}, integral_constant<D>)
  if (d == 128) {
    if (dtype == SLA_BF16) f(bf16raw{}, std::integral_constant<int, 128>{});
    else f(float{}, std::integral_constant<int, 128>{});
  } else {
    if (dtype == SLA_BF16) f(bf16raw{}, std::integral_constant<int, 64>{});
    else f(float{}, std::integral_constant<int, 64>{});
  }
}

static bool bwd_shape_of(int B, int Hq, int Hkv, int N, int d, int lin, int causal, int group_map, int proj_heads,
                         BwdShape* sh) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < kBlock || N % kBlock != 0 || (d != 64 && d != 128))
    return false;
  if (N / kBlock > SLA_MAX_KEY_BLOCKS) return false;
  if (lin != SLA_LIN_NONE && lin != SLA_LIN_ROW_STATES && lin != SLA_LIN_GLOBAL_GATED) return false;
  if (lin != SLA_LIN_NONE && (causal || group_map)) return false;
  if (proj_heads != 0 && (lin != SLA_LIN_ROW_STATES || (proj_heads != 1 && proj_heads != Hq))) return false;
  *sh = BwdShape{B, Hq, Hkv, group_map ? Hkv : Hq, N, d, lin, causal ? 1 : 0, proj_heads != 0 ? 1 : 0};
  return true;
}

}  // namespace sla

extern "C" size_t sla_attn_bwd_ext_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t N, int32_t d,
                                                   int32_t lin_mode, int32_t causal, int32_t group_map,
                                                   int32_t proj_heads) {
  sla::BwdShape sh{};
  if (!sla::bwd_shape_of(B, Hq, Hkv, N, d, lin_mode, causal, group_map, proj_heads, &sh)) return 0;
  return sla::bwd_ws_layout(sh, nullptr, nullptr);
}

extern "C" size_t sla_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d, int32_t proj_heads) {
  if (proj_heads != 0 && proj_heads != 1 && proj_heads != H) return 0;
  return sla_attn_bwd_ext_workspace_bytes(B, H, H, N, d, SLA_LIN_ROW_STATES, 0, 0, proj_heads);
}

extern "C" sla_status sla_attn_bwd_ext(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v,
                                       const sla_tensor* o, const sla_tensor* dout, const float* lse,
                                       int32_t n_valid, float scale, int32_t lin_mode, int32_t causal,
                                       int32_t window_tokens, int32_t group_map, const int32_t* crit_rowptr,
                                       const int32_t* crit_idx, const uint8_t* crit_flags,
                                       const uint32_t* marg_bits, const void* S, const float* u,
                                       const float* H_all, const float* z_all, const float* w_gate,
                                       const float* k_shift, const float* proj_w, const float* proj_b,
                                       int32_t proj_heads, float* dq, float* dk, float* dv, float* dproj_w,
                                       float* dproj_b, float* dw_gate, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if ((st = check_tensor(o)) != SLA_OK) return st;
  if ((st = check_tensor(dout)) != SLA_OK) return st;
  if (!same_geometry(q, k) || !same_geometry(k, v) || !same_geometry(q, o) || !same_geometry(q, dout))
    return SLA_ERR_SHAPE;
  if (v->H != k->H || o->H != q->H || dout->H != q->H || q->H % k->H != 0) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale)) return SLA_ERR_RANGE;
  if (lin_mode != SLA_LIN_NONE && lin_mode != SLA_LIN_ROW_STATES && lin_mode != SLA_LIN_GLOBAL_GATED)
    return SLA_ERR_UNSUPPORTED;
  if (lin_mode != SLA_LIN_NONE && (causal != 0 || group_map != 0)) return SLA_ERR_UNSUPPORTED;
  if (causal != 0 && crit_flags == nullptr) return SLA_ERR_NULL;
  if (causal != 0 && window_tokens < 0) return SLA_ERR_RANGE;
  if (lse == nullptr || crit_rowptr == nullptr || crit_idx == nullptr || dq == nullptr || dk == nullptr ||
      dv == nullptr)
    return SLA_ERR_NULL;
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return SLA_ERR_ALIGN;
  const bool rowst = lin_mode == SLA_LIN_ROW_STATES, gated = lin_mode == SLA_LIN_GLOBAL_GATED;
  if (rowst && (marg_bits == nullptr || S == nullptr || u == nullptr)) return SLA_ERR_NULL;
  if (rowst && (!aligned16(S) || !aligned16(u))) return SLA_ERR_ALIGN;
  if (gated && (H_all == nullptr || z_all == nullptr || w_gate == nullptr || dw_gate == nullptr)) return SLA_ERR_NULL;
  if (gated && (!aligned16(H_all) || !aligned16(z_all) || !aligned16(w_gate) || !aligned16(dw_gate)))
    return SLA_ERR_ALIGN;
  if (!gated && dw_gate != nullptr) return SLA_ERR_NULL;
  const bool proj = proj_w != nullptr;
  if (!proj && (proj_b != nullptr || dproj_w != nullptr || dproj_b != nullptr)) return SLA_ERR_NULL;
  if (proj) {
    if (!rowst) return SLA_ERR_UNSUPPORTED;
    if (dproj_w == nullptr) return SLA_ERR_NULL;
    if (proj_heads != 1 && proj_heads != q->H) return SLA_ERR_SHAPE;
    if (!aligned16(proj_w) || !aligned16(dproj_w) || (proj_b != nullptr && !aligned16(proj_b)) ||
        (dproj_b != nullptr && !aligned16(dproj_b)))
      return SLA_ERR_ALIGN;
  }
  if (k_shift != nullptr && (lin_mode == SLA_LIN_NONE)) return SLA_ERR_UNSUPPORTED;
  if (k_shift != nullptr && !aligned16(k_shift)) return SLA_ERR_ALIGN;
  const int d = q->d, B = q->B, Hq = q->H, Hkv = k->H, N = q->N, nb = N / kBlock;
  if (nb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  BwdShape sh{};
  if (!bwd_shape_of(B, Hq, Hkv, N, d, lin_mode, causal, group_map, proj ? proj_heads : 0, &sh))
    return SLA_ERR_UNSUPPORTED;
  const size_t need = bwd_ws_layout(sh, nullptr, nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
  BwdWs ws{};
  bwd_ws_layout(sh, &ws, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);

  BwdParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr; p.o = o->ptr; p.dout = dout->ptr;
  p.qsB = q->sB; p.qsH = q->sH; p.qsN = q->sN;
  p.ksB = k->sB; p.ksH = k->sH; p.ksN = k->sN;
  p.vsB = v->sB; p.vsH = v->sH; p.vsN = v->sN;
  p.osB = o->sB; p.osH = o->sH; p.osN = o->sN;
  p.dsB = dout->sB; p.dsH = dout->sH; p.dsN = dout->sN;
  p.B = B; p.H = Hq; p.N = N; p.nb = nb; p.n_valid = n_valid; p.wq = (nb + 31) / 32;
  p.hsplit = bwd_hsplit(B, Hq, Hkv, nb);
  p.part_k = ws.part_k;
  p.part_v = ws.part_v;
  p.Hkv = Hkv; p.G = Hq / Hkv; p.Hs = sh.Hs; p.group_map = group_map ? 1 : 0;
  p.window = causal ? window_tokens : 0;
  p.overwrite = lin_mode == SLA_LIN_NONE ? 1 : 0;
  p.gated = gated ? 1 : 0;
  p.scale = scale; p.scale_log2 = scale * kLog2e;
  p.lse = lse; p.crit_rowptr = crit_rowptr; p.crit_idx = crit_idx;
  p.crit_flags = causal ? crit_flags : nullptr;
  p.critT_sel = causal ? ws.critT_sel : nullptr;
  if (rowst) {
    p.S = static_cast<const u16*>(S);
    p.u = u;
  }
  if (gated) {
    p.Sf = H_all;
    p.u = z_all;
    p.w_gate = w_gate;
    p.gpart = ws.gpart;
  }
  p.D = ws.D; p.dS = ws.dS; p.du = ws.du; p.dH = ws.dH; p.dz = ws.dz; p.critT = ws.critT;
  p.kv_order = ws.kv_order;
  p.k_shift = k_shift;
  p.dk_mean = k_shift != nullptr ? ws.dk_mean : nullptr;
  if (proj) {
    p.proj_w = proj_w; p.proj_b = proj_b;
    p.proj_sH = proj_heads != 1 ? int64_t(d) * d : 0;
    p.xlin = ws.xlin;
  }
  p.dq = dq; p.dk = dk; p.dv = dv;

  // transposed masks (cleared by a fill kernel, then set by atomic OR) and the dK/dV order
  const int mrows = B * sh.Hs * nb, qrows = B * Hq * nb, krows = B * Hkv * nb;
  const int64_t nbits = int64_t(mrows) * p.wq;
  auto fill = [&](uint32_t* ptr, int64_t n, uint32_t val) {
    fill_u32_kernel<<<dim3(uint32_t((n + 255) / 256)), 256, 0, s>>>(ptr, n, val);
  };
  fill(ws.critT, nbits, 0u);
  if (causal) fill(ws.critT_sel, nbits, 0u);
  fill(reinterpret_cast<uint32_t*>(ws.kv_counts), krows, 0u);
  crit_transpose_kernel<<<dim3((mrows + 3) / 4), 256, 0, s>>>(crit_rowptr, crit_idx, p.crit_flags, mrows, nb, p.wq,
                                                              sh.Hs, Hkv, group_map ? 1 : p.G, ws.critT,
                                                              ws.critT_sel, ws.kv_counts);
  if (rowst) {
    fill(ws.margT, int64_t(qrows) * p.wq, 0u);
    const int wk = (nb + 31) / 32;
    marg_transpose_kernel<<<dim3(uint32_t((int64_t(qrows) * wk + 255) / 256)), 256, 0, s>>>(marg_bits, qrows, nb, wk,
                                                                                           p.wq, ws.margT);
  } else if (gated) {
    ones_bits_kernel<<<dim3(uint32_t((int64_t(B) * Hq * p.wq + 255) / 256)), 256, 0, s>>>(ws.margT, B * Hq, nb, p.wq);
  }
  const int max_count = min(nb * (group_map ? 1 : p.G), kMaxKeyBlocksBwd);
  kv_order_kernel<<<1, 1024, 0, s>>>(ws.kv_counts, krows, max_count, ws.kv_order);

  // 1. query side: linear dQ, D, dS_i, du_i (and O_l with Proj; the gate weights' partials when
  //    gated) — without Proj inside the dQ kernel, which then writes the whole dQ — or D alone
  //    without a linear branch
  by_type(q->dtype, d, [&](auto tv, auto dv_) { launch_bwd_q_side<decltype(tv), decltype(dv_)::value>(p, B, s); });
  if (proj) {
    const int per_head = proj_heads != 1;
    by_type(q->dtype, d, [&](auto tv, auto dv_) {
      launch_proj_grad<decltype(tv), decltype(dv_)::value>(p, B, per_head, ws, dproj_w, dproj_b, s);
    });
  }
  if (gated) gate_reduce_kernel<<<dim3(d / 8, Hq), 256, 0, s>>>(ws.gpart, B, Hq, nb, d, dw_gate);
  // 2. dH_j = sum of dS_i, dz_j = sum of du_i over the query blocks i with j marginal: the
  //    marginal aggregation with the mask transposed (rows = key blocks, summed items = query
  //    blocks); gated: one row per head whose mask holds every query block
  if (rowst) {
    if ((st = launch_marginal_states(ws.dS, ws.du, B, Hq, Hq, nb, nb, d, 0, ws.margT, ws.dH, ws.dz, s)) != SLA_OK)
      return st;
  } else if (gated) {
    if ((st = launch_marginal_states(ws.dS, ws.du, B, Hq, Hq, 1, nb, d, 0, ws.margT, ws.dH, ws.dz, s)) != SLA_OK)
      return st;
  }
  // 3. linear branch, key side (dK, dV written; with smooth-K the mean of that dK), then the sparse
  //    branch (dQ, dK, dV accumulated, or written without a linear branch)
  by_type(q->dtype, d, [&](auto tv, auto dv_) {
    launch_bwd_k_side<decltype(tv), decltype(dv_)::value>(p, B, lin_mode != SLA_LIN_NONE, s);
  });
  return launch_status();
}

extern "C" sla_status sla_attn_bwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v,
                                   const sla_tensor* o, const sla_tensor* dout, const float* lse, int32_t n_valid,
                                   float scale, const int32_t* crit_rowptr, const int32_t* crit_idx,
                                   const uint32_t* marg_bits, const void* S, const float* u, const float* k_shift,
                                   const float* proj_w, const float* proj_b, int32_t proj_heads, float* dq,
                                   float* dk, float* dv, float* dproj_w, float* dproj_b, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if (k->H != q->H) return SLA_ERR_UNSUPPORTED;  // one KV head per query head
  return sla_attn_bwd_ext(q, k, v, o, dout, lse, n_valid, scale, SLA_LIN_ROW_STATES, 0, 0, 0, crit_rowptr, crit_idx,
                          nullptr, marg_bits, S, u, nullptr, nullptr, nullptr, k_shift, proj_w, proj_b, proj_heads,
                          dq, dk, dv, dproj_w, dproj_b, nullptr, workspace, workspace_bytes, stream);
}
