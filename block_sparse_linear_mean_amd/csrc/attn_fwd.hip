// Attention step: exact block-sparse softmax attention over each query block's critical
// key blocks, with the linear branch fused into the output epilogue.
//
// Method: critical (query block, key block) pairs get exact softmax attention, i.e.
// FlashAttention restricted to the listed blocks, and marginal pairs linear attention;
// the outputs are summed (SLA analysis page for arXiv 2509.24006: FlashAttn + linear
// attention per block pair, O = O_s + Proj(O_l) with Proj zero-initialised and here
// the identity).  SALAD gates a linear branch over all keys by an input-dependent
// gate (SALAD page, method framework).  The NSA-style variant attends to selected
// blocks plus a sliding window under a causal mask, and the query heads of a GQA
// group share the selection ("Sparse Attention 方法综述", section 2 NSA).
//
// Design (gfx950, wave64, 16x16x32 bf16 matrix cores):
//  * one workgroup = one 64-row query block of one head, 4 wavefronts x 16 query rows;
//  * the query fragment stays in registers for the whole block list;
//  * per critical key block, K is staged in LDS row-major and V transposed
//    ([feature][token]); scores are computed transposed (S^T = K Q^T), so each lane
//    owns one query column and 16 keys: the row max needs two cross-lane steps and
//    the online-softmax rescale of the (transposed) output accumulators is per lane;
//  * P^T feeds the P.V product directly from registers: the 32-key contraction uses a
//    fixed permutation of keys that matches how the S^T tiles sit in the lanes, and
//    V^T is read from LDS in the same permuted order (two 8-byte reads per operand);
//  * exp2 with scale*log2(e) folded in; fp32 running max / sum / accumulators;
//  * epilogue: 1/l normalisation, then the linear term phi(q)^T S / (phi(q) . u)
//    as one more matrix-core product against S^T staged in LDS as bf16.
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

sla_status launch_marginal_states(const float* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const int* rowptr, const int* idx, float* S, float* u,
                                  hipStream_t st);

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t qsB, qsH, qsN, ksB, ksH, ksN, vsB, vsH, vsN;
  int Hq, Hkv, Hs, N, nqb, n_valid, window, group_map;
  float scale_log2;
  const int* crit_rowptr;
  const int* crit_idx;
  const uint8_t* crit_flags;
  const float* S;       // SLA: per map row d x d ([r][c]); SALAD: per KV head H_all
  const float* u;       // SLA: per map row d;         SALAD: per KV head z_all
  const float* w_gate;  // SALAD: [Hq][d]
  void* out;
  int out_f32;
};

template <int D>
struct AttnSmem {
  static constexpr int kKs = kBlock * (D + 8);     // K block, row-major, padded rows
  static constexpr int kVt = D * (kBlock + 8);     // V block, transposed, padded rows
  static constexpr int kSt = D * (D + 8);          // epilogue: S^T (bf16)
  static constexpr int kElems = (kKs + kVt) > kSt ? (kKs + kVt) : kSt;
};

template <typename T, int D, bool CAUSAL, int LIN>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
  constexpr int kQs = D / 32;      // 32-wide feature steps of the Q.K contraction
  constexpr int kDt = D / 16;      // 16-wide feature tiles of the output
  constexpr int kTpt = D / 32;     // tokens per thread in the V transpose
  constexpr int kTg = kBlock / kTpt;
  constexpr int kVs = kBlock + 8;  // Vt row stride
  constexpr int kKsS = D + 8;      // Ks row stride
  __shared__ __attribute__((aligned(16))) u16 smem[AttnSmem<D>::kElems];
  __shared__ float lin_u[D];
  u16* Ks = smem;
  u16* Vt = smem + AttnSmem<D>::kKs;

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int g = h / G;
  const int smap = p.group_map ? g : h;
  const int64_t mrow = (int64_t(b) * p.Hs + smap) * p.nqb + i;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave, l16 = lane % 16, lg = lane / 16;
  const T* Q = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
  const T* K = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(g) * p.ksH;
  const T* V = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(g) * p.vsH;

  const int tq = kBlock * i + 16 * w + l16;       // this lane's query row
  const bool qvalid = tq < p.n_valid;
  bf16x8 qf[kQs];
#pragma unroll
  for (int ks = 0; ks < kQs; ++ks)
    qf[ks] = qvalid ? In<T>::load8(Q + int64_t(tq) * p.qsN + 32 * ks + 8 * lg) : zero8();

  f32x4 oacc[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int cbeg = p.crit_rowptr[mrow], cend = p.crit_rowptr[mrow + 1];
  for (int pi = cbeg; pi < cend; ++pi) {
    const int j = p.crit_idx[pi];
    const int flag = CAUSAL ? int(p.crit_flags[pi]) : 1;
    if (unsigned(j) >= unsigned(p.nqb)) continue;   // malformed list entry: never read outside K/V
    __syncthreads();
    // ---- stage K_j (row-major) and V_j (transposed) in LDS; padded keys are zero
#pragma unroll
    for (int u = 0; u < (kBlock * D / 8) / 256; ++u) {
      const int e = t + 256 * u;
      const int row = e / (D / 8), c8 = e % (D / 8);
      const int s = kBlock * j + row;
      const bf16x8 x = s < p.n_valid ? In<T>::load8(K + int64_t(s) * p.ksN + 8 * c8) : zero8();
      *reinterpret_cast<bf16x8*>(Ks + row * kKsS + 8 * c8) = x;
    }
    {
      const int tg = t % kTg, fg = t / kTg;
      bf16x8 vv[kTpt];
#pragma unroll
      for (int uu = 0; uu < kTpt; ++uu) {
        const int s = kBlock * j + kTpt * tg + uu;
        vv[uu] = s < p.n_valid ? In<T>::load8(V + int64_t(s) * p.vsN + 8 * fg) : zero8();
      }
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        u16* dst = Vt + (8 * fg + f) * kVs + kTpt * tg;
        if constexpr (kTpt == 4) {
          bf16x4 col = {vv[0][f], vv[1][f], vv[2][f], vv[3][f]};
          *reinterpret_cast<bf16x4*>(dst) = col;
        } else {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          bf16x2 col = {vv[0][f], vv[1][f]};
          *reinterpret_cast<bf16x2*>(dst) = col;
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane holds keys 16kt + 4lg + e (e < 4) for query column l16
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kQs; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (16 * kt + l16) * kKsS + 32 * ks + 8 * lg);
        sacc[kt] = mfma16(a, qf[ks], sacc[kt]);
      }
    }
    float x[4][4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = kBlock * j + 16 * kt + 4 * lg + e;
        bool ok = s < p.n_valid;
        if constexpr (CAUSAL) ok = ok && s <= tq && ((flag & 1) || tq - s < p.window);
        x[kt][e] = ok ? sacc[kt][e] * p.scale_log2 : -__builtin_inff();
        mx = fmaxf(mx, x[kt][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - base);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[kt][e] = __builtin_amdgcn_exp2f(x[kt][e] - base);
        l_run += x[kt][e];
      }

    // ---- O^T += V^T P^T over two 32-key steps; k-slot m of lane group lg holds key
    //      32 ks + 16 (m / 4) + 4 lg + m % 4 in both operands
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x8 pv = {x[2 * ks][0], x[2 * ks][1], x[2 * ks][2], x[2 * ks][3],
                        x[2 * ks + 1][0], x[2 * ks + 1][1], x[2 * ks + 1][2], x[2 * ks + 1][3]};
      const bf16x8 pb = cvt8(pv);
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const u16* row = Vt + (16 * dt + l16) * kVs + 32 * ks + 4 * lg;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[dt] = mfma16(a, pb, oacc[dt]);
      }
    }
  }

  // ---- normalise the sparse branch
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) oacc[dt] *= inv_l;

  // ---- linear branch: phi(q)^T S / (phi(q) . u), S^T staged in LDS as bf16
  if constexpr (LIN != SLA_LIN_NONE) {
    const float* Sg;
    const float* ug;
    if constexpr (LIN == SLA_LIN_MARGINAL) {
      Sg = p.S + mrow * D * D;
      ug = p.u + mrow * D;
    } else {
      Sg = p.S + (int64_t(b) * p.Hkv + g) * D * D;
      ug = p.u + (int64_t(b) * p.Hkv + g) * D;
    }
    __syncthreads();   // the last K/V tile is no longer read
    u16* St = smem;    // [c][r], row stride D + 8
    for (int blk = t; blk < (D / 4) * (D / 4); blk += 256) {
      const int r0 = 4 * (blk / (D / 4)), c0 = 4 * (blk % (D / 4));
      f32x4 rows4[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) rows4[rr] = *reinterpret_cast<const f32x4*>(Sg + (r0 + rr) * D + c0);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f32x4 col = {rows4[0][cc], rows4[1][cc], rows4[2][cc], rows4[3][cc]};
        *reinterpret_cast<bf16x4*>(St + (c0 + cc) * (D + 8) + r0) = __builtin_convertvector(col, bf16x4);
      }
    }
    if (t < D) lin_u[t] = ug[t];
    __syncthreads();

    bf16x8 pq[kQs];
    float den = 0.f, gdot = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQs; ++ks) {
      f32x8 ph;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int r = 32 * ks + 8 * lg + m;
        const float qv = float(qf[ks][m]);
        ph[m] = phi(qv);
        den += ph[m] * lin_u[r];
        if constexpr (LIN == SLA_LIN_GLOBAL_GATED) gdot += qv * p.w_gate[int64_t(h) * D + r];
      }
      pq[ks] = cvt8(ph);
    }
    den += __shfl_xor(den, 16);
    den += __shfl_xor(den, 32);
    float scale_lin = den > 0.f ? 1.f / den : 0.f;
    if constexpr (LIN == SLA_LIN_GLOBAL_GATED) {
      gdot += __shfl_xor(gdot, 16);
      gdot += __shfl_xor(gdot, 32);
      scale_lin *= 1.f / (1.f + __expf(-gdot));
    }
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kQs; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(St + (16 * dt + l16) * (D + 8) + 32 * ks + 8 * lg);
        num = mfma16(a, pq[ks], num);
      }
      oacc[dt] += num * scale_lin;
    }
  }

  // ---- store: lane holds O[tq][16 dt + 4 lg + e]; padded query rows are zero
  const int64_t obase = ((int64_t(b) * p.Hq + h) * p.N + tq) * D;
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) {
    f32x4 o = qvalid ? oacc[dt] : f32x4{0.f, 0.f, 0.f, 0.f};
    const int col = 16 * dt + 4 * lg;
    if (p.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + col) = o;
    } else {
      *reinterpret_cast<bf16x4*>(static_cast<u16*>(p.out) + obase + col) = __builtin_convertvector(o, bf16x4);
    }
  }
}

template <typename T, int D>
static void launch_attn(const AttnParams& p, int causal, int lin, dim3 grid, hipStream_t st) {
  if (causal) {
    attn_fwd_kernel<T, D, true, SLA_LIN_NONE><<<grid, 256, 0, st>>>(p);
  } else if (lin == SLA_LIN_MARGINAL || lin == SLA_LIN_ROW_STATES) {
    attn_fwd_kernel<T, D, false, SLA_LIN_MARGINAL><<<grid, 256, 0, st>>>(p);
  } else if (lin == SLA_LIN_GLOBAL_GATED) {
    attn_fwd_kernel<T, D, false, SLA_LIN_GLOBAL_GATED><<<grid, 256, 0, st>>>(p);
  } else {
    attn_fwd_kernel<T, D, false, SLA_LIN_NONE><<<grid, 256, 0, st>>>(p);
  }
}

}  // namespace sla

extern "C" sla_status sla_attn_fwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                                   float scale, int32_t causal, int32_t window_tokens, int32_t group_map,
                                   const int32_t* crit_rowptr, const int32_t* crit_idx, const uint8_t* crit_flags,
                                   const int32_t* marg_rowptr, const int32_t* marg_idx, int32_t lin_mode,
                                   const float* H, const float* z, const float* H_all, const float* z_all,
                                   const float* w_gate, void* out, int32_t out_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(q);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(k)) != SLA_OK) return st;
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if (!same_geometry(q, k) || !same_geometry(k, v) || k->H != v->H || q->H % k->H != 0) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, q->N)) != SLA_OK) return st;
  if (!(scale > 0.f) || !__builtin_isfinite(scale) || window_tokens < 0) return SLA_ERR_RANGE;
  if (out == nullptr || crit_rowptr == nullptr || crit_idx == nullptr) return SLA_ERR_NULL;
  if (!aligned16(out)) return SLA_ERR_ALIGN;
  if (out_dtype != SLA_BF16 && out_dtype != SLA_F32) return SLA_ERR_UNSUPPORTED;
  if (lin_mode < SLA_LIN_NONE || lin_mode > SLA_LIN_ROW_STATES) return SLA_ERR_UNSUPPORTED;
  if (causal && lin_mode != SLA_LIN_NONE) return SLA_ERR_UNSUPPORTED;
  if (causal && crit_flags == nullptr) return SLA_ERR_NULL;
  const int d = q->d, nqb = q->N / kBlock;
  const int Hs = group_map ? k->H : q->H;
  hipStream_t s = static_cast<hipStream_t>(stream);

  AttnParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr;
  p.qsB = q->sB; p.qsH = q->sH; p.qsN = q->sN;
  p.ksB = k->sB; p.ksH = k->sH; p.ksN = k->sN;
  p.vsB = v->sB; p.vsH = v->sH; p.vsN = v->sN;
  p.Hq = q->H; p.Hkv = k->H; p.Hs = Hs; p.N = q->N; p.nqb = nqb; p.n_valid = n_valid;
  p.window = window_tokens; p.group_map = group_map ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.crit_rowptr = crit_rowptr; p.crit_idx = crit_idx; p.crit_flags = crit_flags;
  p.out = out; p.out_f32 = out_dtype == SLA_F32;

  if (lin_mode == SLA_LIN_MARGINAL) {
    if (H == nullptr || z == nullptr || marg_rowptr == nullptr || marg_idx == nullptr) return SLA_ERR_NULL;
    const size_t need = sla_attn_workspace_bytes(q->B, Hs, nqb, d, lin_mode);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
    float* S = static_cast<float*>(workspace);
    float* u = S + int64_t(q->B) * Hs * nqb * d * d;
    if ((st = launch_marginal_states(H, z, q->B, q->H, k->H, nqb, nqb, d, p.group_map, marg_rowptr, marg_idx, S,
                                     u, s)) != SLA_OK)
      return st;
    p.S = S;
    p.u = u;
  } else if (lin_mode == SLA_LIN_ROW_STATES) {
    if (H == nullptr || z == nullptr) return SLA_ERR_NULL;
    if (!aligned16(H) || !aligned16(z)) return SLA_ERR_ALIGN;
    p.S = H;
    p.u = z;
  } else if (lin_mode == SLA_LIN_GLOBAL_GATED) {
    if (H_all == nullptr || z_all == nullptr || w_gate == nullptr) return SLA_ERR_NULL;
    p.S = H_all;
    p.u = z_all;
    p.w_gate = w_gate;
  }
  dim3 grid(nqb, q->H, q->B);
  const bool bf = q->dtype == SLA_BF16;
  if (d == 128) {
    if (bf) launch_attn<bf16raw, 128>(p, causal, lin_mode, grid, s);
    else launch_attn<float, 128>(p, causal, lin_mode, grid, s);
  } else {
    if (bf) launch_attn<bf16raw, 64>(p, causal, lin_mode, grid, s);
    else launch_attn<float, 64>(p, causal, lin_mode, grid, s);
  }
  return launch_status();
}
