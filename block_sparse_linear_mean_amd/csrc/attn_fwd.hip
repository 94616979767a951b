// Attention step: exact block-sparse softmax attention over each query block's critical
// key blocks, with the linear branch fused into the output epilogue.
//
// Method: critical (query block, key block) pairs get exact softmax attention, i.e.
// FlashAttention restricted to the listed blocks, and marginal pairs linear attention;
// the outputs are summed (SLA analysis page for arXiv 2509.24006: FlashAttn + linear
// attention per block pair, O = O_s + Proj(O_l) with Proj a learned, zero-initialised
// layer: the identity unless a weight is passed).  SALAD gates a linear branch over all
// keys by an input-dependent gate (SALAD page, method framework).  The NSA-style variant
// attends to selected blocks plus a sliding window under a causal mask, and the query
// heads of a GQA group share the selection ("Sparse Attention 方法综述", section 2 NSA).
//
// Design (gfx950, wave64, 32x32x16 bf16 matrix cores):
//  * one workgroup = one 64-row query block of one head (2 wavefronts x 32 query rows), or of
//    two heads of a GQA group that share a causal block map (4 wavefronts, each staged K/V tile
//    serving both); the heads of a group run on one XCD back to back (shared L2);
//  * the query fragment stays in registers for the whole block list;
//  * per critical key block, K and V tiles are copied global -> LDS by the direct-to-LDS
//    loads; scores are computed transposed (S^T = K Q^T), so each lane owns one query
//    column: the row max and sum need one half-wave swap, and the online-softmax
//    rescale of the (transposed) output accumulators is per lane;
//  * P^T feeds the P.V product directly from registers, V^T comes from the transposing
//    LDS read;
//  * each key block as two 32-key halves: the scores of one half and the P.V of the other are
//    issued among the half's softmax instructions (a wavefront's own VALU work runs in the shadow
//    of its matrix-core products; another wavefront's barely does);
//  * exp2 with scale*log2(e) folded in; fp32 running offset / sum / accumulators;
//  * epilogue: 1/l normalisation, then the linear term phi(q)^T S / (phi(q) . u)
//    as one more matrix-core product against S^T staged in LDS as bf16, and, with a
//    projection, one more product against the staged weight.
#include "attn_tiles.h"
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

sla_status launch_marginal_states(const u16* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const uint32_t* bits, u16* S, float* u, hipStream_t st);

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t qsB, qsH, qsN, ksB, ksH, ksN, vsB, vsH, vsN;
  int Hq, Hkv, Hs, N, nqb, n_valid, window, group_map;
  int nkb, n_keys;      // key blocks and valid keys (= nqb, n_valid unless the keys are compressed tokens)
  int cmp_block, cmp_stride;   // compressed keys (cmp_stride > 0): key m is visible to query t iff
                               // m * cmp_stride + cmp_block - 1 <= t; otherwise key s iff s <= t (causal)
  float scale_log2;
  const int* crit_rowptr;
  const int* crit_idx;
  const uint8_t* crit_flags;
  const void* S;        // SLA: per map row d x d bf16 [c][r]; SALAD: per KV head H_all fp32 [c][r]
  const float* u;       // SLA: per map row d;              SALAD: per KV head z_all
  const float* w_gate;  // SALAD: [Hq][d]
  const float* proj_w;  // SLA: Proj weight [heads][d (out)][d (in)] fp32, or null (identity)
  const float* proj_b;  // SLA: Proj bias [heads][d] fp32, or null
  int64_t proj_sH;      // elements between the weights of consecutive heads (0: one shared weight)
  float* lse;           // optional [B][Hq][N]: natural log-sum-exp of each row's sparse-branch logits
  void* out;
  int out_f32;
};

// Workgroup order.  Workgroups are dealt round-robin to the 8 XCDs, each with its own L2, so
// the hardware index is remapped: the workgroups one XCD receives form one contiguous range of
// the logical order, in which the query heads of a GQA group (same map row, same K/V blocks)
// come first, then neighbouring query blocks (largely the same critical blocks).
struct WgCoord {
  int i, h, b;
};
// Causal rows do work that grows with i: there (heavy_first) each XCD's range takes every 8th
// query block, largest i first, so the XCDs stay balanced and the longest blocks start first.
// hp: query heads per workgroup (consecutive heads of one GQA group; hp divides the group size).
__device__ __forceinline__ WgCoord wg_coord(int nqb, int Hq, int Hkv, bool heavy_first = false, int hp = 1) {
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int G = Hq / Hkv;
  const int hh = (logical % (G / hp)) * hp;
  const int rest = logical / (G / hp);
  int i = rest % nqb;
  if (heavy_first) {
    const int per = nqb / 8;
    i = (per > 0 && i < 8 * per) ? nqb - 1 - ((i % per) * 8 + i / per) : nqb - 1 - i;
  }
  const int bg = rest / nqb;
  const int g = bg % Hkv, b = bg / Hkv;
  return WgCoord{i, g * G + hh, b};
}

// One workgroup = one 64-row query block of one head: 2 wavefronts x 32 query rows, 32x32x16
// bf16 matrix cores; for causal maps shared by a GQA group, of two heads of the group (NW = 4:
// wavefronts 2 and 3 take the second head), which then share every staged K/V tile.  Per critical key block: S^T = K Q^T (lane = one query column, 32 keys),
// online softmax in registers, O^T += V^T P^T with P^T fed from registers and V^T from the
// transposing LDS read.  One 32 KB K+V stage per workgroup (four workgroups per CU; two of the
// 4-wavefront head pairs).  At the NSA prefill head pairs take the pass from 1.08 to 1.05 ms; four
// heads sharing each staged tile in one 8-wavefront workgroup measured slower, 1.31 ms (one
// workgroup per CU).
// Step k of NSTEP of the softmax of a 32-key half (scores sc, 16 per lane): elements
// E k .. E k + E - 1 (E = 16 / NSTEP) of P = exp2(c2 s - off); each time eight are done they are
// packed into a bf16 B operand (p0, then p1) and added to the row sum (of those bf16 values, two
// per dot instruction).
#define SOFTMAX_STEP(NSTEP, sc, k, pv, p0, p1, lsum, off)                                       \
  do {                                                                                          \
    constexpr int kE_ = 16 / (NSTEP);                                                           \
    _Pragma("unroll") for (int m_ = 0; m_ < kE_; ++m_)                                          \
      pv[(kE_ * (k) + m_) % 8] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kE_ * (k) + m_], c2, -(off))); \
    if ((kE_ * (k) + kE_) % 8 == 0) {                                                           \
      bf16x8& dst_ = kE_ * (k) < 8 ? (p0) : (p1);                                               \
      dst_ = cvt8(pv);                                                                          \
      lsum += sum8_bf16(dst_);                                                                  \
    }                                                                                           \
  } while (0)

template <typename T, int D, bool CAUSAL, int LIN, int NW, bool PROJ = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(AttnParams p) {
  using Tl = AttnTile<D>;
  constexpr int kQs = D / 16;      // 16-wide feature steps of the Q.K contraction
  constexpr int kDt = D / 32;      // 32-wide feature tiles of the output
  constexpr bool kDirect = sizeof(T) == 2;
  constexpr int kWaitK = kDirect ? Tl::kInst / NW : 0;  // loads of one tile per wavefront
  constexpr int kThreads = kWave * NW;
  __shared__ __attribute__((aligned(1024))) unsigned char ksm[Tl::kTileB];
  __shared__ __attribute__((aligned(1024))) unsigned char vsm[Tl::kTileB];
  __shared__ float lin_u[D];
  lds_u8* Kb = to_lds(ksm);
  lds_u8* Vb = to_lds(vsm);

  const int t = threadIdx.x, lane = t % kWave, l32 = lane % 32, lg = lane / 32;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);   // wave-uniform: head and K/V bases in SGPRs
  static_assert(NW == 2 || (NW == 4 && LIN == SLA_LIN_NONE),
                "one head per workgroup (two wavefronts of 32 query rows), or two heads without a linear branch");
  const WgCoord wc = wg_coord(p.nqb, p.Hq, p.Hkv, CAUSAL, NW / 2);
  const int i = wc.i, h = wc.h + w / 2, b = wc.b;  // this wavefront's head
  const int G = p.Hq / p.Hkv;
  const int g = h / G;
  const int smap = p.group_map ? g : h;
  const int64_t mrow = (int64_t(b) * p.Hs + smap) * p.nqb + i;
  const T* Q = static_cast<const T*>(p.q) + int64_t(b) * p.qsB + int64_t(h) * p.qsH;
  const T* K = static_cast<const T*>(p.k) + int64_t(b) * p.ksB + int64_t(g) * p.ksH;
  const T* V = static_cast<const T*>(p.v) + int64_t(b) * p.vsB + int64_t(g) * p.vsH;

  if constexpr (LIN == SLA_LIN_MARGINAL) {
    if (t < D) lin_u[t] = p.u[mrow * D + t];
  } else if constexpr (LIN != SLA_LIN_NONE) {
    if (t < D) lin_u[t] = p.u[(int64_t(b) * p.Hkv + g) * D + t];
  }
  const int tq = kBlock * i + 32 * (w % 2) + l32; // this lane's query row
  const bool qvalid = tq < p.n_valid;
  // causal limit: key s is visible iff s <= tlim (s <= tq; for compressed keys s * stride + block - 1 <= tq)
  const int tlim = !CAUSAL || p.cmp_stride <= 0 ? tq
                   : (tq >= p.cmp_block - 1 ? (tq - p.cmp_block + 1) / p.cmp_stride : -1);
  bf16x8 qf[kQs];
#pragma unroll
  for (int ks = 0; ks < kQs; ++ks)
    qf[ks] = qvalid ? In<T>::load8(Q + int64_t(tq) * p.qsN + 16 * ks + 8 * lg) : zero8();

  f32x16 oacc[kDt];
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
  // running row offset M in exp2 units (P = exp2(c2 s - M)), -inf until the row has seen a key
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c2 = p.scale_log2;

  // per-lane offsets, computed once: direct-load sources, K operand reads, V transposed reads
  const StageOff<D, NW> koff = stage_offsets<D, true, NW>(p.ksN);
  const StageOff<D, NW> voff = stage_offsets<D, false, NW>(p.vsN);
  int kread[kQs];                 // K row 32 kt + l32, chunk 2 ks + lg (+ 32 kt rows = kt * 8 KB)
#pragma unroll
  for (int ks = 0; ks < kQs; ++ks) kread[ks] = k_pos<D>(l32, 2 * ks + lg);
  const int sg = (lane / 16) % 2, kk = lane % 16;
  int vread[kDt];                 // V rows 16 u + 4 lg + kk / 4 (+ 8), 8-byte half kk % 2
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
    vread[dt] = v_pos<D>(4 * lg + kk / 4, 4 * dt + 2 * sg + (kk % 4) / 2) + 8 * (kk % 2);

  const int cbeg = p.crit_rowptr[mrow], cend = p.crit_rowptr[mrow + 1];
  // the row's list, 128 entries at a time in two registers per lane, read back with readlane
  int lj0 = 0, lj1 = 0, lf0 = 0, lf1 = 0;
  auto load_list = [&](int base) {
    const int e0 = base + lane, e1 = base + 64 + lane;
    lj0 = e0 < cend ? p.crit_idx[e0] : 0;
    lj1 = e1 < cend ? p.crit_idx[e1] : 0;
    if constexpr (CAUSAL) {
      lf0 = e0 < cend ? int(p.crit_flags[e0]) : 0;
      lf1 = e1 < cend ? int(p.crit_flags[e1]) : 0;
    }
  };
  int lbase = cbeg;
  load_list(lbase);
  auto entry = [&](int n, int v0, int v1) {   // n = position relative to lbase, 0 <= n < 128
    return n < 64 ? __builtin_amdgcn_readlane(v0, n) : __builtin_amdgcn_readlane(v1, n - 64);
  };
  auto safe_block = [&](int jraw) { return unsigned(jraw) < unsigned(p.nkb) ? jraw : 0; };
  // scores of keys that may not be attended (padded, malformed, causal, window) become -inf; key
  // s = rel + C with C = 32 kt + 8 (e / 4) + e % 4 a constant per slot, so every test compares C
  // with a per-lane bound and no per-slot key index has to live in registers
  auto mask_scores = [&](f32x16& sc, int kt, int j, bool jok, int flag) {
    const int rel = kBlock * j + 4 * lg;
    const int lim_valid = jok ? p.n_keys - rel : 0;    // s < n_keys       <=> C < lim_valid
    const int lim_causal = tlim - rel;                  // s <= tlim        <=> C <= lim_causal
    const int lim_win = tq - rel - p.window;            // tq - s < window  <=> C > lim_win
    const bool sel = flag & 1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int C = 32 * kt + 8 * (e / 4) + (e % 4);
      bool ok = C < lim_valid;
      if constexpr (CAUSAL) ok = ok && C <= lim_causal && (sel || C > lim_win);
      sc[e] = ok ? sc[e] : -__builtin_inff();
    }
  };
  // softmax of one 32-key half: P = exp2(c2 s - M) as two bf16 B operands and their row sum (of the
  // bf16 values the P.V product uses, two per dot instruction)
  auto half_probs = [&](const f32x16& sc, bf16x8& p0, bf16x8& p1, float off) {
    f32x8 a, b2;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      a[m] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[m], c2, -off));
      b2[m] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[8 + m], c2, -off));
    }
    p0 = cvt8(a);
    p1 = cvt8(b2);
    return sum8_bf16(p0) + sum8_bf16(p1);
  };
  // the running offset M moves only when the row has none yet or a half's P sum passes 2^16: then
  // the half's row max sets it, the accumulators are rescaled and the half's P recomputed.  Every P
  // stays below 2^16, far from overflow, without a row max per block.
  auto settle = [&](const f32x16& sc, bf16x8& p0, bf16x8& p1, float& lsum) {
    if (__any(m_run == -__builtin_inff() || !(lsum <= 65536.f))) {
      float mxs[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int e = 0; e < 16; ++e) mxs[e % 4] = fmaxf(mxs[e % 4], sc[e]);
      const float mx = xor32_max(fmaxf(fmaxf(mxs[0], mxs[1]), fmaxf(mxs[2], mxs[3]))) * c2;
      const float m_new = fmaxf(m_run, mx);          // -inf while the row has no key
      if (m_new != m_run) {
        const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
      }
      lsum = half_probs(sc, p0, p1, m_run == -__builtin_inff() ? 0.f : m_run);
    }
    l_run += lsum;
  };
  // O^T += V^T P^T over keys 16 u .. 16 u + 15: slot m of P holds key 16 u + 8 (m / 4) + 4 lg + m % 4;
  // each 16-lane group reads 4 consecutive keys of one 16-column strip with the transposing read
  // (row r0 + 8 has the same swizzle as r0, since both leave the same remainder mod 4)
  auto vop = [&](int u, int dt) {
    const bf16x4 lo = lds_read_tr4(Vb + vread[dt] + 16 * u * Tl::kRowB);
    const bf16x4 hi = lds_read_tr4(Vb + vread[dt] + (16 * u + 8) * Tl::kRowB);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // padded keys: zero the V rows r0 .. r1 - 1 (every wavefront waits for the others afterwards)
  auto zero_v_rows = [&](int r0, int r1) {
    for (int e = t; e < (r1 - r0) * Tl::kChunks; e += kThreads) {
      const int r = r0 + e / Tl::kChunks;
      lds_store16(Vb + v_pos<D>(r, e % Tl::kChunks), zero8());
    }
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
  };
  const bf16raw* Srow = reinterpret_cast<const bf16raw*>(static_cast<const u16*>(p.S)) + mrow * D * D;

  // Each key block is taken as two 32-key halves (h = 0, 1), and the matrix-core products of one
  // half are issued among the VALU work of the other: on gfx950 a wavefront's own independent
  // VALU instructions run largely in the shadow of its MFMAs, while another wavefront's barely do.
  //   R0: S0 = K[0:32] Q^T                          (K rows 0..31 then free: K_{j+1}[0:32] streams in)
  //   R1: S1 = K[32:64] Q^T  |  softmax(S0)         (K rows 32..63 free: K_{j+1}[32:64])
  //   R2: O += V[0:32] P0    |  softmax(S1)
  //   R3: O += V[32:64] P1                          (V free: V_{j+1} streams in)
  // K goes by half tiles (kHS direct loads per wavefront each), so each half has about a block's
  // time to land; V, needed only from R2 on, has R0 and R1.  The waits name how many of this
  // wavefront's copies may stay in flight.
  constexpr int kHS = HalfSteps<D, NW>::kSteps;
  const HalfSteps<D, NW> khs = half_steps<D, NW>(p.ksN);
  const HalfSteps<D, NW> vhs = half_steps<D, NW>(p.vsN);
  if (cbeg < cend) {
    const int j0 = safe_block(entry(0, lj0, lj1));
    stage_half<T, D, true, NW>(K, p.ksN, j0, 0, Kb, koff, khs);
    stage_half<T, D, true, NW>(K, p.ksN, j0, 1, Kb, koff, khs);
    stage_half<T, D, false, NW>(V, p.vsN, j0, 0, Vb, voff, vhs);
    stage_half<T, D, false, NW>(V, p.vsN, j0, 1, Vb, voff, vhs);
    if constexpr (kDirect) SLA_WAIT_VMCNT(2 * kHS);  // K_0 resident (V_0 may still be in flight)
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
  }
  for (int pi = cbeg; pi < cend; ++pi) {
    if (pi - lbase == 64) {                          // slide the list window (rare: > 64 entries)
      lbase += 64;
      lj0 = lj1;
      lf0 = lf1;
      const int e1 = lbase + 64 + lane;
      lj1 = e1 < cend ? p.crit_idx[e1] : 0;
      if constexpr (CAUSAL) lf1 = e1 < cend ? int(p.crit_flags[e1]) : 0;
    }
    const int jraw = entry(pi - lbase, lj0, lj1);
    const bool jok = unsigned(jraw) < unsigned(p.nkb);   // a malformed entry reads block 0, fully masked
    const int j = jok ? jraw : 0;
    const int flag = CAUSAL ? entry(pi - lbase, lf0, lf1) : 1;
    const bool more = pi + 1 < cend;
    const int jn = more ? safe_block(entry(pi + 1 - lbase, lj0, lj1)) : 0;
    const int rv = p.n_keys - kBlock * j;           // valid rows of this block (may exceed 64)
    const bool full = jok && rv >= kBlock && !CAUSAL;
    const int vz = jok ? max(rv, 0) : 0;             // V rows from vz on are padding

    // ---- R0: S0 = K rows 0..31 x Q^T (one accumulation chain, operands a step ahead)
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = 0.f;
      s1[e] = 0.f;
    }
    {
      bf16x8 ka[3];                                  // operands two steps ahead
      ka[0] = lds_load16(Kb + kread[0]);
      ka[1] = lds_load16(Kb + kread[1]);
#pragma unroll
      for (int ks = 0; ks < kQs; ++ks) {
        if (ks + 2 < kQs) ka[(ks + 2) % 3] = lds_load16(Kb + kread[ks + 2]);
        s0 = mfma32(ka[ks % 3], qf[ks], s0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    SLA_WAIT_LGKM0();
    SLA_BARRIER();                                   // A: every wavefront has read K rows 0..31
    if (more) stage_half<T, D, true, NW>(K, p.ksN, jn, 0, Kb, koff, khs);
    if (!full) mask_scores(s0, 0, j, jok, flag);

    // ---- R1: S1 = K rows 32..63 x Q^T among the softmax of S0
    bf16x8 pb[4];
    const float off1 = m_run == -__builtin_inff() ? 0.f : m_run;
    // step ks: one product, the next K operand and 1/8 of the softmax (scheduling barriers keep
    // the compiler from regrouping them)
    float lsum0 = 0.f;
    {
      f32x8 pv;
      bf16x8 kb3[3];                                 // operands two steps ahead
      kb3[0] = lds_load16(Kb + kread[0] + 32 * Tl::kRowB);
      kb3[1] = lds_load16(Kb + kread[1] + 32 * Tl::kRowB);
#pragma unroll
      for (int ks = 0; ks < kQs; ++ks) {
        if (ks + 2 < kQs) kb3[(ks + 2) % 3] = lds_load16(Kb + kread[ks + 2] + 32 * Tl::kRowB);
        s1 = mfma32(kb3[ks % 3], qf[ks], s1);
        SOFTMAX_STEP(kQs, s0, ks, pv, pb[0], pb[1], lsum0, off1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    settle(s0, pb[0], pb[1], lsum0);

    // ---- B: K rows 32..63 read by every wavefront; V_j resident (the copy after it: with a next
    // block, its K rows 0..31)
    if constexpr (kDirect) {
      if (more) SLA_WAIT_VMCNT(kHS);
      else SLA_WAIT_VMCNT(0);
    }
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
    if (more) {
      stage_half<T, D, true, NW>(K, p.ksN, jn, 1, Kb, koff, khs);
    } else if constexpr (LIN == SLA_LIN_MARGINAL) {
      // last block: the linear epilogue's S^T rows 0..63 stream into the free K buffer now
      stage_tile<bf16raw, D, true, NW>(Srow, D, 0, Kb, stage_offsets<D, true, NW>(D));
    }
    if (vz < kBlock) zero_v_rows(vz, kBlock);
    if (!full) mask_scores(s1, 1, j, jok, flag);

    // ---- R2: O += V rows 0..31 x P0 among the softmax of S1
    const float off2 = m_run == -__builtin_inff() ? 0.f : m_run;
    float lsum1 = 0.f;
    {
      static_assert(2 * kDt == kQs, "the P.V steps of a half pair with the softmax steps");
      f32x8 pv;
      bf16x8 va[3];                                  // operands two steps ahead
      va[0] = vop(0, 0);
      va[1] = vop(1 / kDt, 1 % kDt);
#pragma unroll
      for (int st = 0; st < 2 * kDt; ++st) {
        const int u = st / kDt, dt = st % kDt;
        if (st + 2 < 2 * kDt) va[(st + 2) % 3] = vop((st + 2) / kDt, (st + 2) % kDt);
        oacc[dt] = mfma32(va[st % 3], pb[u], oacc[dt]);
        SOFTMAX_STEP(2 * kDt, s1, st, pv, pb[2], pb[3], lsum1, off2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    settle(s1, pb[2], pb[3], lsum1);

    // ---- R3: O += V rows 32..63 x P1
    {
      constexpr int kSt = 2 * kDt;
      bf16x8 va[3];                                  // operands two steps ahead
      va[0] = vop(2, 0);
      va[1] = vop(2 + 1 / kDt, 1 % kDt);
#pragma unroll
      for (int st = 0; st < kSt; ++st) {
        const int u = 2 + st / kDt, dt = st % kDt;
        if (st + 2 < kSt) va[(st + 2) % 3] = vop(2 + (st + 2) / kDt, (st + 2) % kDt);
        oacc[dt] = mfma32(va[st % 3], pb[u], oacc[dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- D: V_j read by every wavefront; the next block's K resident (no copy after it)
    if constexpr (kDirect) {
      if (more) SLA_WAIT_VMCNT(0);
    }
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
    if (more) {
      stage_half<T, D, false, NW>(V, p.vsN, jn, 0, Vb, voff, vhs);
      stage_half<T, D, false, NW>(V, p.vsN, jn, 1, Vb, voff, vhs);
    } else if constexpr (LIN == SLA_LIN_MARGINAL && D == 128) {
      stage_tile<bf16raw, D, true, NW>(Srow, D, 1, Vb, stage_offsets<D, true, NW>(D));
    }
  }

  // ---- normalise the sparse branch
  const float l_tot = xor32_sum(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (p.lse != nullptr && lg == 0)   // ln sum_s exp(scale q.k_s) = (m c2 + log2 l) ln 2; -inf without keys
    p.lse[(int64_t(b) * p.Hq + h) * p.N + tq] =
        (qvalid && l_tot > 0.f) ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -__builtin_inff();
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt) oacc[dt] *= inv_l;

  // ---- linear branch: phi(q)^T S / (phi(q) . u) with S^T staged in LDS ([c][r], K layout)
  if constexpr (LIN != SLA_LIN_NONE) {
    // S^T rows (c) 0..63 go to the K buffer, rows 64..D-1 to the V buffer, both in the K layout
    // (for per-row states already issued during the last critical block, if the row has one)
    auto st_tile = [&](int r) { return r < kBlock ? Kb : Vb; };
    if (LIN != SLA_LIN_MARGINAL || cbeg >= cend) {
      SLA_WAIT_VMCNT(0);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
      if constexpr (LIN == SLA_LIN_MARGINAL) {
        const u16* Sg = static_cast<const u16*>(p.S) + mrow * D * D;
        const StageOff<D, NW> soff = stage_offsets<D, true, NW>(D);
        stage_tile<bf16raw, D, true, NW>(reinterpret_cast<const bf16raw*>(Sg), D, 0, Kb, soff);
        if constexpr (D == 128) stage_tile<bf16raw, D, true, NW>(reinterpret_cast<const bf16raw*>(Sg), D, 1, Vb, soff);
      } else {
        const float* Sg = static_cast<const float*>(p.S) + (int64_t(b) * p.Hkv + g) * D * D;
        for (int e = t; e < D * Tl::kChunks; e += kThreads) {
          const int r = e / Tl::kChunks, c = e % Tl::kChunks;
          const bf16x8 x = In<float>::load8(Sg + r * D + 8 * c);
          lds_store16(st_tile(r) + k_pos<D>(r % kBlock, c), x);
        }
      }
    }
    SLA_WAIT_VMCNT(0);
    SLA_WAIT_LGKM0();
    SLA_BARRIER();

    bf16x8 pq[kQs];
    float den = 0.f, gdot = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQs; ++ks) {
      f32x8 ph;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int r = 16 * ks + 8 * lg + m;
        const float qv = float(qf[ks][m]);
        ph[m] = phi(qv);
        den += ph[m] * lin_u[r];
        if constexpr (LIN == SLA_LIN_GLOBAL_GATED) gdot += qv * p.w_gate[int64_t(h) * D + r];
      }
      pq[ks] = cvt8(ph);
    }
    den = xor32_sum(den);
    float scale_lin = den > 0.f ? 1.f / den : 0.f;
    if constexpr (LIN == SLA_LIN_GLOBAL_GATED) {
      gdot = xor32_sum(gdot);
      scale_lin *= 1.f / (1.f + __expf(-gdot));
    }
    bf16x8 lb[PROJ ? kQs : 1];    // Proj: O_l^T as B operands
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) {
      f32x16 num = f32x16{};
      const int row = 32 * dt + l32;                 // c
#pragma unroll
      for (int ks = 0; ks < kQs; ++ks) {
        const bf16x8 a = lds_load16(st_tile(row) + k_pos<D>(row % kBlock, 2 * ks + lg));
        num = mfma32(a, pq[ks], num);
      }
      if constexpr (!PROJ) {
        oacc[dt] += num * scale_lin;
      } else {
        // Proj(O_l)^T = W O_l^T + b with O_l^T as the B operand.  For k-step ks the lane needs
        // O_l[tq][16 ks + 8 lg .. + 7]; it holds features 16 ks + 4 lg + {0..3} and
        // 16 ks + 8 + 4 lg + {0..3} (elements 8 (ks % 2) + {0..3, 4..7} of this dt's tile, dt =
        // ks / 2), so one half-wave swap per register pair trades the lower half-wave's second
        // group for the upper half-wave's first.
        num *= scale_lin;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          f32x8 x;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(num[8 * h2 + m]),
                                                            __float_as_uint(num[8 * h2 + 4 + m]), false, false);
            x[m] = __uint_as_float(r[0]);
            x[4 + m] = __uint_as_float(r[1]);
          }
          lb[2 * dt + h2] = cvt8(x);
        }
      }
    }
    if constexpr (PROJ) {
      // every wavefront has read S^T; stage W [o][c] (bf16, K layout) over the same buffers
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
      const float* Wg = p.proj_w + int64_t(h) * p.proj_sH;
      for (int e = t; e < D * Tl::kChunks; e += kThreads) {
        const int r = e / Tl::kChunks, c = e % Tl::kChunks;
        lds_store16(st_tile(r) + k_pos<D>(r % kBlock, c), In<float>::load8(Wg + r * D + 8 * c));
      }
      if (p.proj_b != nullptr) {
        // lane holds output features 32 dt + 8 q4 + 4 lg + {0..3} in oacc[dt][4 q4 .. 4 q4 + 3]
        const float* bias = p.proj_b + int64_t(h) * (p.proj_sH != 0 ? D : 0);
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 bb = *reinterpret_cast<const f32x4*>(bias + 32 * dt + 8 * q4 + 4 * lg);
#pragma unroll
            for (int m = 0; m < 4; ++m) oacc[dt][4 * q4 + m] += bb[m];
          }
      }
      SLA_WAIT_VMCNT(0);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const int row = 32 * dt + l32;               // output feature o
#pragma unroll
        for (int ks = 0; ks < kQs; ++ks)
          oacc[dt] = mfma32(lds_load16(st_tile(row) + k_pos<D>(row % kBlock, 2 * ks + lg)), lb[ks], oacc[dt]);
      }
    }
  }

  // ---- store: lane holds O[tq][32 dt + 8 (e / 4) + 4 lg + e % 4]; padded query rows are zero
  {
    if (!p.out_f32) {
      // bf16 output of a head: re-staged through the K buffer (the second head of a pair: the V
      // buffer; 64 rows of 2 D bytes, 16-byte chunk c of row r at c ^ (r % chunks)) so that every
      // store writes whole rows, 16 bytes a lane
      SLA_WAIT_LGKM0();
      SLA_BARRIER();                                 // every wavefront is done with the buffers
      lds_u8* ost = w / 2 ? Vb : Kb;
      const int r = 32 * (w % 2) + l32;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x4 o = {oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2], oacc[dt][4 * e4 + 3]};
          const int c = 4 * dt + e4;
          *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(
              ost + r * Tl::kRowB + 16 * (c ^ (r % Tl::kChunks)) + 8 * lg) = __builtin_convertvector(o, bf16x4);
        }
      SLA_WAIT_LGKM0();
      SLA_BARRIER();
      // each half of the workgroup (NW / 2 wavefronts) stores one head's tile
      constexpr int kHalfT = kThreads / (NW / 2);
      const int th = t % kHalfT;
      u16* ob = static_cast<u16*>(p.out) + ((int64_t(b) * p.Hq + h) * p.N + kBlock * i) * D;
#pragma unroll
      for (int n = 0; n < kBlock * Tl::kChunks / kHalfT; ++n) {
        const int e = th + kHalfT * n;
        const int rr = e / Tl::kChunks, c = e % Tl::kChunks;
        bf16x8 x = lds_load16(ost + rr * Tl::kRowB + 16 * (c ^ (rr % Tl::kChunks)));
        if (kBlock * i + rr >= p.n_valid) x = zero8();
        // streaming store: the output is not read again by this layer, and the next pass's reads
        // then find fewer dirty lines to evict
        __builtin_nontemporal_store(x, reinterpret_cast<bf16x8*>(ob + rr * D + 8 * c));
      }
      return;
    }
  }
  const int64_t obase = ((int64_t(b) * p.Hq + h) * p.N + tq) * D;
#pragma unroll
  for (int dt = 0; dt < kDt; ++dt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      f32x4 o = {oacc[dt][4 * e4], oacc[dt][4 * e4 + 1], oacc[dt][4 * e4 + 2], oacc[dt][4 * e4 + 3]};
      if (!qvalid) o = f32x4{0.f, 0.f, 0.f, 0.f};
      const int col = 32 * dt + 8 * e4 + 4 * lg;
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
    // maps shared by a GQA group of an even number of heads: two heads per workgroup share each
    // staged K/V tile (half the workgroups)
    if (p.group_map && (p.Hq / p.Hkv) % 2 == 0)
      attn_fwd_kernel<T, D, true, SLA_LIN_NONE, 4><<<dim3(grid.x / 2), 256, 0, st>>>(p);
    else
      attn_fwd_kernel<T, D, true, SLA_LIN_NONE, 2><<<grid, 128, 0, st>>>(p);
  } else if (lin == SLA_LIN_MARGINAL || lin == SLA_LIN_ROW_STATES) {
    if (p.proj_w != nullptr) attn_fwd_kernel<T, D, false, SLA_LIN_MARGINAL, 2, true><<<grid, 128, 0, st>>>(p);
    else attn_fwd_kernel<T, D, false, SLA_LIN_MARGINAL, 2><<<grid, 128, 0, st>>>(p);
  } else if (lin == SLA_LIN_GLOBAL_GATED) {
    attn_fwd_kernel<T, D, false, SLA_LIN_GLOBAL_GATED, 2><<<grid, 128, 0, st>>>(p);
  } else {
    attn_fwd_kernel<T, D, false, SLA_LIN_NONE, 2><<<grid, 128, 0, st>>>(p);
  }
}

// One causal pass of the selected-block kernel over explicit block lists (group map rows), fp32
// output: the building block of the three NSA branches.  k / v may be compressed tokens
// (cmp_stride > 0, n_keys of them); window > 0 adds the sliding-window rule for blocks without
// flag bit 0.
sla_status launch_causal_pass(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int n_valid,
                              int n_keys, float scale, int window, int cmp_block, int cmp_stride, const int* rowptr,
                              const int* idx, const uint8_t* flags, float* out, hipStream_t st) {
  const int nqb = q->N / kBlock;
  AttnParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr;
  p.qsB = q->sB; p.qsH = q->sH; p.qsN = q->sN;
  p.ksB = k->sB; p.ksH = k->sH; p.ksN = k->sN;
  p.vsB = v->sB; p.vsH = v->sH; p.vsN = v->sN;
  p.Hq = q->H; p.Hkv = k->H; p.Hs = k->H; p.N = q->N; p.nqb = nqb; p.n_valid = n_valid;
  p.nkb = k->N / kBlock; p.n_keys = n_keys; p.cmp_block = cmp_block; p.cmp_stride = cmp_stride;
  p.window = window; p.group_map = 1;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.crit_rowptr = rowptr; p.crit_idx = idx; p.crit_flags = flags;
  p.out = out; p.out_f32 = 1;
  const dim3 grid(nqb * q->H * q->B);
  const bool bf = q->dtype == SLA_BF16;
  if (q->d == 128) {
    if (bf) launch_attn<bf16raw, 128>(p, 1, SLA_LIN_NONE, grid, st);
    else launch_attn<float, 128>(p, 1, SLA_LIN_NONE, grid, st);
  } else {
    if (bf) launch_attn<bf16raw, 64>(p, 1, SLA_LIN_NONE, grid, st);
    else launch_attn<float, 64>(p, 1, SLA_LIN_NONE, grid, st);
  }
  return launch_status();
}

}  // namespace sla

extern "C" sla_status sla_attn_fwd(const sla_tensor* q, const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                                   float scale, int32_t causal, int32_t window_tokens, int32_t group_map,
                                   const int32_t* crit_rowptr, const int32_t* crit_idx, const uint8_t* crit_flags,
                                   const uint32_t* marg_bits, int32_t lin_mode,
                                   const void* H, const float* z, const float* H_all, const float* z_all,
                                   const float* w_gate, const float* proj_w, const float* proj_b,
                                   int32_t proj_heads, void* out, int32_t out_dtype, float* lse,
                                   void* workspace, size_t workspace_bytes, void* stream) {
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
  if (proj_w == nullptr && proj_b != nullptr) return SLA_ERR_NULL;
  if (proj_w != nullptr) {
    if (lin_mode != SLA_LIN_MARGINAL && lin_mode != SLA_LIN_ROW_STATES) return SLA_ERR_UNSUPPORTED;
    if (proj_heads != 1 && proj_heads != q->H) return SLA_ERR_SHAPE;
    if (!aligned16(proj_w) || (proj_b != nullptr && !aligned16(proj_b))) return SLA_ERR_ALIGN;
  }
  const int d = q->d, nqb = q->N / kBlock;
  const int Hs = group_map ? k->H : q->H;
  hipStream_t s = static_cast<hipStream_t>(stream);

  AttnParams p{};
  p.q = q->ptr; p.k = k->ptr; p.v = v->ptr;
  p.qsB = q->sB; p.qsH = q->sH; p.qsN = q->sN;
  p.ksB = k->sB; p.ksH = k->sH; p.ksN = k->sN;
  p.vsB = v->sB; p.vsH = v->sH; p.vsN = v->sN;
  p.Hq = q->H; p.Hkv = k->H; p.Hs = Hs; p.N = q->N; p.nqb = nqb; p.n_valid = n_valid;
  p.nkb = nqb; p.n_keys = n_valid; p.cmp_block = 0; p.cmp_stride = 0;
  p.window = window_tokens; p.group_map = group_map ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.crit_rowptr = crit_rowptr; p.crit_idx = crit_idx; p.crit_flags = crit_flags;
  p.out = out; p.out_f32 = out_dtype == SLA_F32;
  p.proj_w = proj_w; p.proj_b = proj_b;
  p.lse = lse;
  p.proj_sH = (proj_w != nullptr && proj_heads != 1) ? int64_t(q->d) * q->d : 0;

  if (lin_mode == SLA_LIN_MARGINAL) {
    if (H == nullptr || z == nullptr || marg_bits == nullptr) return SLA_ERR_NULL;
    const size_t need = sla_attn_workspace_bytes(q->B, Hs, nqb, d, lin_mode);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
    u16* S = static_cast<u16*>(workspace);
    float* u = reinterpret_cast<float*>(S + int64_t(q->B) * Hs * nqb * d * d);
    if (!aligned16(H) || !aligned16(z)) return SLA_ERR_ALIGN;
    if ((st = launch_marginal_states(static_cast<const u16*>(H), z, q->B, q->H, k->H, nqb, nqb, d, p.group_map, marg_bits, S, u, s)) !=
        SLA_OK)
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
  dim3 grid(nqb * q->H * q->B);
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
