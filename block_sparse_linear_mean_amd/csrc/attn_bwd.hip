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
  int H, N, nb, n_valid, wq;      // wq: 32-bit words per transposed bit row, ceil(nb / 32)
  float scale, scale_log2;
  const float* lse;               // [B, H, N] natural log-sum-exp of the forward's sparse branch
  const int* crit_rowptr;
  const int* crit_idx;
  const u16* S;                   // per-row marginal sums, bf16 [rows][c][r]
  const float* u;                 // [rows][r]
  float* D;                       // [B, H, N]: dO . O_sparse
  u16* dS;                        // [rows][c][r] bf16: gradient of S_i
  float* du;                      // [rows][r]
  const u16* dH;                  // [B, H, nb][c][r] bf16: gradient of H_j
  const float* dz;                // [B, H, nb][r]
  const uint32_t* critT;          // [B, H, nb][wq]: bit i of row j = block j is critical for query block i
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
  constexpr int kChunks = D / 8;
  for (int e = threadIdx.x; e < kBlock * kChunks; e += kBwThreads) {
    const int r = e / kChunks, c = e % kChunks;
    const bf16x8 x = row0 + r < n_rows ? In<T>::load8(X + int64_t(row0 + r) * sN + 8 * c) : zero8();
    lds_store16(tile + tpos<D>(r, c), x);
  }
}

// ------------------------------------------------------------------ transposed bit masks

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e < n) p[e] = v;
}

// One wavefront per map row (bh, i), one lane per listed block j: set bit i of row (bh, j) of the
// transposed critical mask (atomic OR: the result does not depend on the order), so every entry's
// atomics are in flight at once.  Also counts, per key-block row, the query blocks that list it
// (the dK/dV workload of that row).
__global__ __launch_bounds__(256) void crit_transpose_kernel(const int* __restrict__ rowptr, const int* __restrict__ idx,
                                                             int rows, int nb, int wq, uint32_t* __restrict__ critT,
                                                             int* __restrict__ counts) {
  const int r = blockIdx.x * 4 + int(threadIdx.x) / kWave;
  if (r >= rows) return;
  const int bh = r / nb, i = r % nb;
  for (int e = rowptr[r] + int(threadIdx.x) % kWave; e < rowptr[r + 1]; e += kWave) {
    const int j = idx[e];
    if (unsigned(j) < unsigned(nb)) {
      const uint32_t bit = 1u << (i % 32);
      // a repeated entry (a malformed list) is counted once
      if ((atomicOr(critT + (int64_t(bh) * nb + j) * wq + i / 32, bit) & bit) == 0u) atomicAdd(counts + bh * nb + j, 1);
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

// One workgroup per (query block i, head); wavefront w owns query rows 64 i + 16 w + l % 16.
// Writes dQ (linear part, all rows), D_t, and the per-row gradients dS_i ([c][r], bf16), du_i.
// PROJ: O = O_s + O_l W^T + b, so O_s = O - O_l W^T - b, the gradient reaching O_l is dO W, and
// O_l is written out (bf16) for the weight gradient.
template <typename T, int D, bool PROJ>
__global__ __launch_bounds__(kBwThreads) void bwd_lin_q_kernel(BwdParams p) {
  constexpr int kKc = D / 32;     // 32-deep k-steps over features
  constexpr int kCt = D / 16;     // 16-wide feature tiles
  constexpr int RB = 2 * D;
  __shared__ __attribute__((aligned(1024))) unsigned char w_sm[PROJ ? D * RB : 16];  // W: [o][c]
  __shared__ __attribute__((aligned(1024))) unsigned char st_sm[D * RB];      // S_i^T: [c][r]
  __shared__ __attribute__((aligned(1024))) unsigned char pq_sm[kBlock * RB]; // phi(Q_i): [t][r]
  __shared__ __attribute__((aligned(1024))) unsigned char dn_sm[kBlock * RB]; // dN_i: [t][c]
  __shared__ float us[D];
  __shared__ float dden_s[kBlock];
  lds_u8* St = to_lds(st_sm);
  lds_u8* Pq = to_lds(pq_sm);
  lds_u8* Dn = to_lds(dn_sm);

  const int i = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  const int64_t row = int64_t(bh) * p.nb + i;
  const u16* Sg = p.S + row * D * D;
  for (int e = t; e < D * D / 8; e += kBwThreads) {
    const int c = e / (D / 8), r8 = e % (D / 8);
    lds_store16(St + tpos<D>(c, r8), *reinterpret_cast<const bf16x8*>(Sg + int64_t(c) * D + 8 * r8));
  }
  for (int e = t; e < D; e += kBwThreads) us[e] = p.u[row * D + e];
  __syncthreads();

  const int tq = kBlock * i + 16 * w + l16;
  const bool qv = tq < p.n_valid;
  const T* Qr = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH + int64_t(tq) * p.qsN;
  const T* Or = static_cast<const T*>(p.o) + int64_t(b) * p.osB + int64_t(h) * p.osH + int64_t(tq) * p.osN;
  const T* Gr = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH + int64_t(tq) * p.dsN;

  // phi(q) of this lane's row: B operands (features 32 kc + 8 g .. + 7) and the fp32 denominator
  bf16x8 pqf[kKc];
  float den = 0.f;
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
    }
    pqf[kc] = cvt8(ph);
    lds_store16(Pq + tpos<D>(16 * w + l16, 4 * kc + g), pqf[kc]);
  }
  den = group4_sum(den);
  const float inv_den = (qv && den > 0.f) ? 1.f / den : 0.f;

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
    lds_u8* Wt = to_lds(w_sm);
    const float* Wg = p.proj_w + int64_t(h) * p.proj_sH;
    for (int e = t; e < D * D / 8; e += kBwThreads) {
      const int o = e / (D / 8), c8 = e % (D / 8);
      lds_store16(Wt + tpos<D>(o, c8), In<float>::load8(Wg + int64_t(o) * D + 8 * c8));
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
      for (int e = 0; e < 4; ++e) dsum += go[ot][e] * (oo[e] - y[e] - bb[e]);
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
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      const f32x4 oo = qv ? load4_f32(Or + 16 * ct + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += go[ct][e] * (oo[e] - xl[ct][e]);
      ga[ct] = go[ct];
    }
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
  if (g == 0) {
    p.D[int64_t(bh) * p.N + tq] = qv ? dsum : 0.f;
    dden_s[16 * w + l16] = dden;
  }

  // dphi(q)^T[r][t] = sum_c S[r][c] dn[t][c] (+ u[r] dden): A = S (transposing reads of the
  // [c][r] tile, rows c paired as 16 (2 kc) + 4 g .. and 16 (2 kc + 1) + 4 g ..), B = dn
  const T* Qb = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
  float* dqr = p.dq + (int64_t(bh) * p.N + tq) * D;
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
    for (int e = 0; e < 4; ++e) out[e] = qv ? (acc[e] + us[r0 + e] * dden) * dphi(qx[e]) : 0.f;
    *reinterpret_cast<f32x4*>(dqr + r0) = out;
  }
  __syncthreads();                // phi(Q_i), dN_i and dden complete in LDS

  // dS_i[r][c] = sum_t phi(q_t)[r] dn_t[c], stored [c][r]: wave w covers (rt, ct) tiles
  // n = w, w + 4, ... of the kCt x kCt grid; the k steps run over the 64 query rows
  u16* dSg = p.dS + row * D * D;
#pragma unroll
  for (int n = w; n < kCt * kCt; n += kBwWaves) {
    const int rt = n / kCt, ct = n % kCt;
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

// ------------------------------------------------------------------ linear branch, key side

// One workgroup per (key block j, head); wavefront w owns keys 64 j + 16 w + l % 16.
// Writes dK and dV (linear part, all rows): dphi(k) = dH_j v + dz_j, dv = dH_j^T phi(k); with
// smooth-K, phi and its derivative at the shifted key k - mean.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void bwd_lin_k_kernel(BwdParams p) {
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  constexpr int RB = 2 * D;
  __shared__ __attribute__((aligned(1024))) unsigned char dh_sm[D * RB];   // dH_j: [c][r]
  __shared__ float dzs[D];
  lds_u8* Ht = to_lds(dh_sm);

  const int j = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  const int64_t row = int64_t(bh) * p.nb + j;
  const u16* Hg = p.dH + row * D * D;
  for (int e = t; e < D * D / 8; e += kBwThreads) {
    const int c = e / (D / 8), r8 = e % (D / 8);
    lds_store16(Ht + tpos<D>(c, r8), *reinterpret_cast<const bf16x8*>(Hg + int64_t(c) * D + 8 * r8));
  }
  for (int e = t; e < D; e += kBwThreads) dzs[e] = p.dz[row * D + e];
  __syncthreads();

  const int s = kBlock * j + 16 * w + l16;
  const bool kv = s < p.n_valid;
  const T* Kr = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(h) * p.ksH + int64_t(s) * p.ksN;
  const T* Vr = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(h) * p.vsH + int64_t(s) * p.vsN;
  bf16x8 vf[kKc], pkf[kKc];
#pragma unroll
  for (int kc = 0; kc < kKc; ++kc) {
    vf[kc] = kv ? In<T>::load8(Vr + 32 * kc + 8 * g) : zero8();
    float x[8];
    if (kv) In<T>::load8_f32(Kr + 32 * kc + 8 * g, x);
    f32x8 ph;
#pragma unroll
    for (int m = 0; m < 8; ++m) ph[m] = kv ? phi(x[m] - (p.k_shift ? p.k_shift[int64_t(bh) * D + 32 * kc + 8 * g + m] : 0.f)) : 0.f;
    pkf[kc] = cvt8(ph);
  }
  float* dkr = p.dk + (int64_t(bh) * p.N + s) * D;
  float* dvr = p.dv + (int64_t(bh) * p.N + s) * D;
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) {
    // dphi(k)^T[r][s] = sum_c dH[r][c] v[s][c]: A = dH rows r (transposing reads of [c][r])
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) {
      const bf16x8 a = join(lds_read_tr4(Ht + tr_addr<D>(32 * kc + 8 * g, 16 * rt, lane)),
                            lds_read_tr4(Ht + tr_addr<D>(32 * kc + 8 * g + 4, 16 * rt, lane)));
      acc = mfma16(a, vf[kc], acc);
    }
    const int r0 = 16 * rt + 4 * g;
    f32x4 kx = kv ? load4_f32(Kr + r0) : f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.k_shift != nullptr) kx -= *reinterpret_cast<const f32x4*>(p.k_shift + int64_t(bh) * D + r0);
    f32x4 out;                       // the gradient with respect to the (shifted) key of the linear branch
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = kv ? (acc[e] + dzs[r0 + e]) * dphi(kx[e]) : 0.f;
    *reinterpret_cast<f32x4*>(dkr + r0) = out;
  }
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) {
    // dv^T[c][s] = sum_r dH[r][c] phi(k)[s][r]: A = rows c of the [c][r] tile
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKc; ++kc) acc = mfma16(lds_load16(Ht + tpos<D>(16 * ct + l16, 4 * kc + g)), pkf[kc], acc);
    const int c0 = 16 * ct + 4 * g;
    *reinterpret_cast<f32x4*>(dvr + c0) = kv ? acc : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ------------------------------------------------------------------ Proj weight gradient

// Partial dW[o][c] = sum_t dO[t][o] O_l[t][c] and db[o] = sum_t dO[t][o] over one chunk of 16
// query blocks of one (batch, head): grid x = chunk (of the rows that share weight y), y = weight.
// Rows past n_valid take no part.  Partials are summed by proj_reduce_kernel in a fixed order.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void proj_grad_kernel(BwdParams p, int B, int per_head, int chunks_per_bh,
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

// out[y][e] = sum over the parts of weight y, in order.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const float* __restrict__ part, int parts, int len,
                                                          float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x, y = blockIdx.y;
  if (e >= len) return;
  float s = 0.f;
  for (int q = 0; q < parts; ++q) s += part[(int64_t(y) * parts + q) * len + e];
  out[int64_t(y) * len + e] = s;
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
  for (int row = t; row < n_valid; row += 256) {
    const float* src = dk + (int64_t(bh) * N + row) * d + r0;
    const f32x4 a = *reinterpret_cast<const f32x4*>(src), b4 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      s[m] += a[m];
      s[4 + m] += b4[m];
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

// One workgroup per (query block i, head); wavefront w owns query rows 64 i + 16 w + l % 16.
// Over the row's critical blocks: S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
// K and V tiles are double-buffered: the next block's direct-to-LDS copies run during this one.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void bwd_dq_kernel(BwdParams p) {
  using Tl = AttnTile<D>;
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char k_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char v_sm[2][Tl::kTileB];

  const int i = blockIdx.x, bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t % kWave, w = t / kWave, l16 = lane % 16, g = lane / 16;
  const int64_t row = int64_t(bh) * p.nb + i;
  const int tq = kBlock * i + 16 * w + l16;
  const bool qv = tq < p.n_valid;
  const T* Qr = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH + int64_t(tq) * p.qsN;
  const T* Gr = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH + int64_t(tq) * p.dsN;
  const T* K = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(h) * p.ksH;
  const T* V = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(h) * p.vsH;
  const StageOff<D, kBwWaves> koff = stage_offsets<D, false, kBwWaves>(p.ksN);
  const StageOff<D, kBwWaves> voff = stage_offsets<D, false, kBwWaves>(p.vsN);

  const int cbeg = p.crit_rowptr[row], cend = p.crit_rowptr[row + 1];
  // the row's next valid block index at or after list position e (or -1), wave-uniform
  auto next_block = [&](int& e) -> int {
    while (e < cend) {
      const int jraw = __builtin_amdgcn_readfirstlane(p.crit_idx[e]);
      ++e;
      if (unsigned(jraw) < unsigned(p.nb)) return jraw;   // malformed entries are skipped
    }
    return -1;
  };
  int epos = cbeg;
  int cur = next_block(epos);
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
  const float Dt = qv ? p.D[int64_t(bh) * p.N + tq] : 0.f;
  const float c2 = p.scale_log2;

  f32x4 acc[kCt];
#pragma unroll
  for (int rt = 0; rt < kCt; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int buf = 0;
  while (cur >= 0) {
    const int nxt = next_block(epos);
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
        const bool ok = has && 16 * st + 4 * g + e4 < rv;
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
    buf ^= 1;
  }
  // lane holds dQ^T[r = 16 rt + 4 g + e][t]: add to the linear part
  if (qv) {
    float* dqr = p.dq + (int64_t(bh) * p.N + tq) * D;
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
// on the order).  Counts are at most nb <= 4096.
__global__ __launch_bounds__(1024) void kv_order_kernel(const int* __restrict__ counts, int rows, int max_count,
                                                        int* __restrict__ order) {
  __shared__ int hist[kMaxKeyBlocksBwd + 2];
  const int t = threadIdx.x;
  for (int c = t; c <= max_count + 1; c += 1024) hist[c] = 0;
  __syncthreads();
  for (int r = t; r < rows; r += 1024) atomicAdd(&hist[counts[r]], 1);
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
  for (int r = t; r < rows; r += 1024) order[atomicAdd(&hist[counts[r]], 1)] = r;
}

// One workgroup per (key block j, head); wavefront w owns keys 64 j + 16 w + l % 16.  Over the
// query blocks i that list j as critical: S = Q K^T, dP = dO V^T, dS = P (dP - D),
// dV^T += dO^T P, dK^T += Q^T dS.  Q, dO tiles and the rows' log-sum-exp and D are
// double-buffered: the next query block's direct-to-LDS copies run during this one.
template <typename T, int D>
__global__ __launch_bounds__(kBwThreads) void bwd_dkdv_kernel(BwdParams p) {
  using Tl = AttnTile<D>;
  constexpr int kKc = D / 32;
  constexpr int kCt = D / 16;
  __shared__ __attribute__((aligned(1024))) unsigned char q_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char g_sm[2][Tl::kTileB];
  __shared__ __attribute__((aligned(256))) float lse_s[2][kBlock];
  __shared__ __attribute__((aligned(256))) float d_s[2][kBlock];

  const int krow = p.kv_order[blockIdx.x];        // (bh, j), most-used key blocks first
  const int j = krow % p.nb, bh = krow / p.nb, b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t % kWave, l16 = lane % 16, g = lane / 16;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);
  const int s = kBlock * j + 16 * w + l16;
  const bool kv = s < p.n_valid;
  const T* Kr = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(h) * p.ksH + int64_t(s) * p.ksN;
  const T* Vr = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(h) * p.vsH + int64_t(s) * p.vsN;
  const T* Q = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
  const T* G = static_cast<const T*>(p.dout) + int64_t(b) * p.dsB + int64_t(h) * p.dsH;
  const float* lse_h = p.lse + int64_t(bh) * p.N;
  const float* D_h = p.D + int64_t(bh) * p.N;
  const StageOff<D, kBwWaves> qoff = stage_offsets<D, false, kBwWaves>(p.qsN);
  const StageOff<D, kBwWaves> goff = stage_offsets<D, false, kBwWaves>(p.dsN);

  // the query blocks that list j, ascending: a wave-uniform scan of the transposed bit row
  const uint32_t* bits = p.critT + (int64_t(bh) * p.nb + j) * p.wq;
  int word = 0;
  uint32_t m = 0u;
  auto next_block = [&]() -> int {
    while (m == 0u) {
      if (word >= p.wq) return -1;
      m = __builtin_amdgcn_readfirstlane(bits[word]);
      ++word;
    }
    const int i = 32 * (word - 1) + __builtin_ctz(m);
    m &= m - 1u;
    return i;
  };
  // copies of query block i into buffer bf: Q and dO tiles by every wavefront, the 64 rows'
  // log-sum-exp and D (256 bytes each) by wavefront 0
  auto stage = [&](int i, int bf) {
    stage_tile<T, D, false, kBwWaves>(Q, p.qsN, i, to_lds(q_sm[bf]), qoff);
    stage_tile<T, D, false, kBwWaves>(G, p.dsN, i, to_lds(g_sm[bf]), goff);
    if (w == 0) {
      load_lds4_sbase(lse_h + kBlock * i, uint32_t(4 * lane), to_lds(lse_s[bf]));
      load_lds4_sbase(D_h + kBlock * i, uint32_t(4 * lane), to_lds(d_s[bf]));
    }
  };
  int cur = next_block();
  if (cur >= 0) stage(cur, 0);

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

  int buf = 0;
  while (cur >= 0) {
    const int nxt = next_block();
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
    if (nxt >= 0) stage(nxt, buf ^ 1);
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
        const bool ok = kv && 16 * tt + 4 * g + e4 < rq && l4[e4] > -__builtin_inff();
        pr[e4] = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[e4], c2, -l4[e4] * kLog2e)) : 0.f;
        ds[e4] = ok ? pr[e4] * (pacc[e4] - d4[e4]) : 0.f;
      }
      pb[tt] = cvt4(pr);
      db[tt] = cvt4(ds);
    }
    // dV^T[c][s] += sum_t dO[t][c] P[t][s]; dK^T[r][s] += sum_t Q[t][r] dS[t][s]
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const bf16x8 ag = join(lds_read_tr4(Gt + tr_addr<D>(32 * pr + 4 * g, 16 * ct, lane)),
                               lds_read_tr4(Gt + tr_addr<D>(32 * pr + 16 + 4 * g, 16 * ct, lane)));
        dv[ct] = mfma16(ag, join(pb[2 * pr], pb[2 * pr + 1]), dv[ct]);
        const bf16x8 aq = join(lds_read_tr4(Qt + tr_addr<D>(32 * pr + 4 * g, 16 * ct, lane)),
                               lds_read_tr4(Qt + tr_addr<D>(32 * pr + 16 + 4 * g, 16 * ct, lane)));
        dk[ct] = mfma16(aq, join(db[2 * pr], db[2 * pr + 1]), dk[ct]);
      }
    cur = nxt;
    buf ^= 1;
  }
  if (kv) {
    float* dkr = p.dk + (int64_t(bh) * p.N + s) * D;
    float* dvr = p.dv + (int64_t(bh) * p.N + s) * D;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) {
      f32x4* k4 = reinterpret_cast<f32x4*>(dkr + 16 * ct + 4 * g);
      f32x4* v4 = reinterpret_cast<f32x4*>(dvr + 16 * ct + 4 * g);
      f32x4 add = dk[ct] * p.scale;
      // smooth-K: the linear branch saw k - mean(k), so its dK loses its own mean over the valid rows
      if (p.dk_mean != nullptr) add -= *reinterpret_cast<const f32x4*>(p.dk_mean + int64_t(bh) * D + 16 * ct + 4 * g);
      *k4 = *k4 + add;
      *v4 = *v4 + dv[ct];
    }
  }
}

struct BwdWs {
  float* D;
  u16* dS;
  float* du;
  u16* dH;
  float* dz;
  uint32_t* critT;
  uint32_t* margT;
  int* kv_counts;
  int* kv_order;
  float* dk_mean;
  u16* xlin;
  float* partW;
  float* partB;
};

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

constexpr int kProjChunk = 16;   // query blocks per partial of the Proj weight gradient

static size_t bwd_ws_layout(int B, int H, int N, int d, bool proj, BwdWs* ws, void* base) {
  const int64_t nb = N / kBlock, rows = int64_t(B) * H * nb, wq = (nb + 31) / 32;
  const int64_t parts = proj ? int64_t(B) * H * ((nb + kProjChunk - 1) / kProjChunk) : 0;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t oD = take(size_t(B) * H * N * 4);
  const size_t odS = take(size_t(rows) * d * d * 2);
  const size_t odu = take(size_t(rows) * d * 4);
  const size_t odH = take(size_t(rows) * d * d * 2);
  const size_t odz = take(size_t(rows) * d * 4);
  const size_t oc = take(size_t(rows) * wq * 4);
  const size_t om = take(size_t(rows) * wq * 4);
  const size_t okc = take(size_t(rows) * 4);
  const size_t oko = take(size_t(rows) * 4);
  const size_t okm = take(size_t(B) * H * d * 4);
  const size_t ox = take(proj ? size_t(B) * H * N * d * 2 : 0);
  const size_t opw = take(size_t(parts) * d * d * 4);
  const size_t opb = take(size_t(parts) * d * 4);
  if (ws != nullptr) {
    unsigned char* p = static_cast<unsigned char*>(base);
    ws->D = reinterpret_cast<float*>(p + oD);
    ws->dS = reinterpret_cast<u16*>(p + odS);
    ws->du = reinterpret_cast<float*>(p + odu);
    ws->dH = reinterpret_cast<u16*>(p + odH);
    ws->dz = reinterpret_cast<float*>(p + odz);
    ws->critT = reinterpret_cast<uint32_t*>(p + oc);
    ws->margT = reinterpret_cast<uint32_t*>(p + om);
    ws->kv_counts = reinterpret_cast<int*>(p + okc);
    ws->kv_order = reinterpret_cast<int*>(p + oko);
    ws->dk_mean = reinterpret_cast<float*>(p + okm);
    ws->xlin = reinterpret_cast<u16*>(p + ox);
    ws->partW = reinterpret_cast<float*>(p + opw);
    ws->partB = reinterpret_cast<float*>(p + opb);
  }
  return off;
}

template <typename T, int D>
static void launch_bwd_kernels(const BwdParams& p, int BH, hipStream_t st) {
  const dim3 grid(p.nb, BH);
  if (p.proj_w != nullptr) bwd_lin_q_kernel<T, D, true><<<grid, kBwThreads, 0, st>>>(p);
  else bwd_lin_q_kernel<T, D, false><<<grid, kBwThreads, 0, st>>>(p);
}

template <typename T, int D>
static void launch_bwd_k_side(const BwdParams& p, int BH, hipStream_t st) {
  const dim3 grid(p.nb, BH);
  bwd_lin_k_kernel<T, D><<<grid, kBwThreads, 0, st>>>(p);
  if (p.dk_mean != nullptr)
    dk_mean_kernel<<<dim3(D / 8, BH), 256, 0, st>>>(p.dk, p.N, D, p.n_valid, const_cast<float*>(p.dk_mean));
  bwd_dq_kernel<T, D><<<grid, kBwThreads, 0, st>>>(p);
  bwd_dkdv_kernel<T, D><<<dim3(p.nb * BH), kBwThreads, 0, st>>>(p);
}

// dW (and db) of the Proj layer: partials over chunks of query blocks, then their ordered sums.
template <typename T, int D>
static void launch_proj_grad(const BwdParams& p, int B, int per_head, const BwdWs& ws, float* dw, float* db,
                             hipStream_t st) {
  const int chunks = (p.nb + kProjChunk - 1) / kProjChunk;
  const int weights = per_head ? p.H : 1;
  const int parts = (per_head ? B : B * p.H) * chunks;
  proj_grad_kernel<T, D><<<dim3(parts, weights), kBwThreads, 0, st>>>(p, B, per_head, chunks, ws.partW, ws.partB);
  proj_reduce_kernel<<<dim3((D * D + 255) / 256, weights), 256, 0, st>>>(ws.partW, parts, D * D, dw);
  if (db != nullptr) proj_reduce_kernel<<<dim3(1, weights), 256, 0, st>>>(ws.partB, parts, D, db);
}

}  // namespace sla

extern "C" size_t sla_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d, int32_t proj_heads) {
  if (B < 1 || H < 1 || N < sla::kBlock || N % sla::kBlock != 0 || (d != 64 && d != 128)) return 0;
  if (proj_heads != 0 && proj_heads != 1 && proj_heads != H) return 0;
  return sla::bwd_ws_layout(B, H, N, d, proj_heads != 0, nullptr, nullptr);
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
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if ((st = check_tensor(o)) != SLA_OK) return st;
  if ((st = check_tensor(dout)) != SLA_OK) return st;
  if (!same_geometry(q, k) || !same_geometry(k, v) || !same_geometry(q, o) || !same_geometry(q, dout))
    return SLA_ERR_SHAPE;
  if (k->H != q->H || v->H != q->H || o->H != q->H || dout->H != q->H) return SLA_ERR_UNSUPPORTED;  // MHA only
  if (o->dtype != q->dtype || dout->dtype != q->dtype) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale)) return SLA_ERR_RANGE;
  if (lse == nullptr || crit_rowptr == nullptr || crit_idx == nullptr || marg_bits == nullptr || S == nullptr ||
      u == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return SLA_ERR_NULL;
  if (!aligned16(S) || !aligned16(u) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return SLA_ERR_ALIGN;
  const bool proj = proj_w != nullptr;
  if (!proj && (proj_b != nullptr || dproj_w != nullptr || dproj_b != nullptr)) return SLA_ERR_NULL;
  if (proj) {
    if (dproj_w == nullptr) return SLA_ERR_NULL;
    if (proj_heads != 1 && proj_heads != q->H) return SLA_ERR_SHAPE;
    if (!aligned16(proj_w) || !aligned16(dproj_w) || (proj_b != nullptr && !aligned16(proj_b)) ||
        (dproj_b != nullptr && !aligned16(dproj_b)))
      return SLA_ERR_ALIGN;
  }
  if (k_shift != nullptr && !aligned16(k_shift)) return SLA_ERR_ALIGN;
  const int d = q->d, B = q->B, H = q->H, N = q->N, nb = N / kBlock;
  if (nb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  const size_t need = bwd_ws_layout(B, H, N, d, proj, nullptr, nullptr);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
  BwdWs ws{};
  bwd_ws_layout(B, H, N, d, proj, &ws, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);

  BwdParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr; p.o = o->ptr; p.dout = dout->ptr;
  p.qsB = q->sB; p.qsH = q->sH; p.qsN = q->sN;
  p.ksB = k->sB; p.ksH = k->sH; p.ksN = k->sN;
  p.vsB = v->sB; p.vsH = v->sH; p.vsN = v->sN;
  p.osB = o->sB; p.osH = o->sH; p.osN = o->sN;
  p.dsB = dout->sB; p.dsH = dout->sH; p.dsN = dout->sN;
  p.H = H; p.N = N; p.nb = nb; p.n_valid = n_valid; p.wq = (nb + 31) / 32;
  p.scale = scale; p.scale_log2 = scale * kLog2e;
  p.lse = lse; p.crit_rowptr = crit_rowptr; p.crit_idx = crit_idx;
  p.S = static_cast<const u16*>(S); p.u = u;
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

  // transposed masks (cleared by a fill kernel, then set by atomic OR)
  const int rows = B * H * nb;
  const int64_t nbits = int64_t(rows) * p.wq;
  fill_u32_kernel<<<dim3(uint32_t((nbits + 255) / 256)), 256, 0, s>>>(ws.critT, nbits, 0u);
  fill_u32_kernel<<<dim3(uint32_t((nbits + 255) / 256)), 256, 0, s>>>(ws.margT, nbits, 0u);
  fill_u32_kernel<<<dim3(uint32_t((rows + 255) / 256)), 256, 0, s>>>(reinterpret_cast<uint32_t*>(ws.kv_counts),
                                                                     rows, 0u);
  crit_transpose_kernel<<<dim3((rows + 3) / 4), 256, 0, s>>>(crit_rowptr, crit_idx, rows, nb, p.wq, ws.critT,
                                                             ws.kv_counts);
  const int wk = (nb + 31) / 32;
  marg_transpose_kernel<<<dim3(uint32_t((int64_t(rows) * wk + 255) / 256)), 256, 0, s>>>(marg_bits, rows, nb, wk,
                                                                                        p.wq, ws.margT);
  kv_order_kernel<<<1, 1024, 0, s>>>(ws.kv_counts, rows, nb, ws.kv_order);
  const bool bf = q->dtype == SLA_BF16;
  // 1. linear branch, query side: dQ (linear part), D, dS_i, du_i (and O_l with Proj)
  if (d == 128) {
    if (bf) launch_bwd_kernels<bf16raw, 128>(p, B * H, s);
    else launch_bwd_kernels<float, 128>(p, B * H, s);
  } else {
    if (bf) launch_bwd_kernels<bf16raw, 64>(p, B * H, s);
    else launch_bwd_kernels<float, 64>(p, B * H, s);
  }
  if (proj) {
    const int per_head = proj_heads != 1;
    if (d == 128) {
      if (bf) launch_proj_grad<bf16raw, 128>(p, B, per_head, ws, dproj_w, dproj_b, s);
      else launch_proj_grad<float, 128>(p, B, per_head, ws, dproj_w, dproj_b, s);
    } else {
      if (bf) launch_proj_grad<bf16raw, 64>(p, B, per_head, ws, dproj_w, dproj_b, s);
      else launch_proj_grad<float, 64>(p, B, per_head, ws, dproj_w, dproj_b, s);
    }
  }
  // 2. dH_j = sum of dS_i, dz_j = sum of du_i over the query blocks i with j marginal: the
  //    marginal aggregation with the mask transposed (rows = key blocks, summed items = query blocks)
  if ((st = launch_marginal_states(ws.dS, ws.du, B, H, H, nb, nb, d, 0, ws.margT, ws.dH, ws.dz, s)) != SLA_OK)
    return st;
  // 3. linear branch, key side (dK, dV written; with smooth-K the mean of that dK), then the sparse
  //    branch (dQ, dK, dV accumulated)
  if (d == 128) {
    if (bf) launch_bwd_k_side<bf16raw, 128>(p, B * H, s);
    else launch_bwd_k_side<float, 128>(p, B * H, s);
  } else {
    if (bf) launch_bwd_k_side<bf16raw, 64>(p, B * H, s);
    else launch_bwd_k_side<float, 64>(p, B * H, s);
  }
  return launch_status();
}
