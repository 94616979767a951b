// Linear-branch key states: H_j = phi(K_j)^T V_j (d x d) and z_j = sum phi(K_j) per
// 64-token key block, and optionally their sums over all keys.
//
// Method: marginal block pairs get linear attention with phi = elu + 1 at O(N d^2)
// cost (SLA analysis page for arXiv 2509.24006, comparison with LongCat-Video BSA);
// the per-key-block pre-reduction lets a query block read sum_j H_j instead of the
// keys.  SALAD's parallel linear branch covers all keys (SALAD page, method
// framework), which needs only the sum over every block.
//
// Layout: states are stored feature-transposed, H[c][r] = sum_s phi(K[s,r]) V[s,c], which is
// the operand layout the attention epilogue reads (16 contiguous bytes along r).  Per-block
// states are written in bf16 (rounded once from the fp32 sums): they are summed again in fp32
// by the marginal aggregation, whose matrix-core operands are bf16 anyway, and bf16 halves the
// pass's dominant cost, the state writes.  Sums over chunks of blocks stay fp32.
//
// Design (gfx950): one workgroup of 4 wavefronts per (KV head, run of cb key blocks).  Each
// thread loads its 16-byte pieces of K and V of the next block into registers while the current
// block is contracted (one block of prefetch), applies phi to K in fp32 and writes both tiles to
// LDS row-major in the layout of the transposing read; the 32x32x16 matrix-core operands
// phi(K)^T (A) and V (B) are both read with it.  Wavefront w owns H rows r = 32 w .. 32 w + 31
// (d = 128; at d = 64 a quarter of the 64 x 64 state) and gets z from one more product against
// a B operand of ones, so z sums exactly the rounded phi(K) values H uses.  A lane's accumulator
// holds 4 consecutive r for one c; bf16 states are re-staged through LDS and written with
// 1 KB-contiguous wavefront stores, fp32 run sums with 16-byte stores.  The pass is HBM-bound:
// K and V in, one state per block out.  Optionally it also writes the key block means of the
// prediction step from the same registers, so the pooling pass need not read K again.
#include "attn_tiles.h"
#include "sla_device.h"
#include "sla_host.h"

#include <algorithm>

namespace sla {

// Per-lane offset of a 32x32x16 operand read with two transposing reads (tr_operand) from a tile in
// the v_pos layout: the element each lane addresses is that of tr_operand_off in the plain layout.
template <int D>
__device__ __forceinline__ int kv_operand_off(int m0, int lane) {
  const int sg = (lane / 16) % 2, kk = lane % 16, lg = lane / 32;
  return v_pos<D>(8 * lg + kk / 4, m0 / 8 + 2 * sg + (kk % 4) / 2) + 8 * (kk % 2);
}

// The 16-byte pieces one thread moves per tile: element chunk e = t + 256 n of the 64 x D tile.
// load() only issues the global loads (raw input elements stay in registers, so the loads of
// the next block are in flight while the current one is contracted); store() converts, applies
// phi to K in fp32 and writes both tiles to LDS.
template <typename T, int D>
struct KvPiece {
  static constexpr int kChunks = D / 8;                  // 16-byte bf16 chunks per row
  static constexpr int kPer = kBlock * kChunks / 256;    // per thread: 4 (d 128) or 2 (d 64)
  static constexpr int kVec = sizeof(T) == 2 ? 1 : 2;    // 16-byte loads per 8 elements
  f32x4 k[kPer][kVec], v[kPer][kVec];                    // raw bits (bf16 inputs use [n][0] only)
  uint32_t valid;                                        // bit n: piece n is a valid token row

  __device__ __forceinline__ void load(const T* __restrict__ K, int64_t ksN, const T* __restrict__ V, int64_t vsN,
                                       int j, int n_valid) {
    valid = 0;
#pragma unroll
    for (int n = 0; n < kPer; ++n) {
      const int e = threadIdx.x + 256 * n;
      const int r = e / kChunks, c = e % kChunks;
      int s = kBlock * j + r;
      if (s < n_valid) valid |= 1u << n;
      else s = n_valid - 1;                              // in-bounds stand-in; zeroed in store()
      const f32x4* kp = reinterpret_cast<const f32x4*>(K + int64_t(s) * ksN + 8 * c);
      const f32x4* vp = reinterpret_cast<const f32x4*>(V + int64_t(s) * vsN + 8 * c);
#pragma unroll
      for (int h = 0; h < kVec; ++h) {
        k[n][h] = kp[h];
        v[n][h] = vp[h];
      }
    }
  }
  __device__ __forceinline__ void unpack(const f32x4* x, float* out) const {
    if constexpr (sizeof(T) == 2) {
      const uint32_t a[4] = {__float_as_uint(x[0][0]), __float_as_uint(x[0][1]), __float_as_uint(x[0][2]),
                             __float_as_uint(x[0][3])};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(a[i] << 16);
        out[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { out[i] = x[0][i]; out[4 + i] = x[1][i]; }
    }
  }
  // phi(K - shift) rounded to bf16 and V (zero for padded rows), into tiles in the V-tile layout of
  // the attention (v_pos: at d = 128 the chunk order that keeps a 32-lane transposing-read pass on
  // 64 distinct banks; at d = 64 the plain transposing layout, already conflict-free there).  A
  // thread's pieces all cover features 8 (t % kChunks) .. + 7, the 8 entries of `shift`.
  // POOL: ps = this thread's fp64 sums of its valid rows of raw K (before the shift), the
  // partial sums of the key block mean.
  template <bool POOL>
  __device__ __forceinline__ void store(lds_u8* kt, lds_u8* vt, const float* shift, double (&ps)[8]) const {
    if constexpr (POOL) {
#pragma unroll
      for (int m = 0; m < 8; ++m) ps[m] = 0.0;
    }
#pragma unroll
    for (int n = 0; n < kPer; ++n) {
      const int e = threadIdx.x + 256 * n;
      const int r = e / kChunks, c = e % kChunks;
      float kf[8];
      unpack(k[n], kf);
      if constexpr (POOL) {
        if ((valid >> n) & 1u) {
#pragma unroll
          for (int m = 0; m < 8; ++m) ps[m] += double(kf[m]);
        }
      }
      f32x8 f;
#pragma unroll
      for (int m = 0; m < 8; ++m) f[m] = phi(kf[m] - shift[m]);
      bf16x8 vb;
      if constexpr (sizeof(T) == 2) {
        vb = __builtin_bit_cast(bf16x8, v[n][0]);
      } else {
        const f32x8 vf = {v[n][0][0], v[n][0][1], v[n][0][2], v[n][0][3],
                          v[n][1][0], v[n][1][1], v[n][1][2], v[n][1][3]};
        vb = cvt8(vf);
      }
      const bool ok = (valid >> n) & 1u;
      lds_store16(kt + v_pos<D>(r, c), ok ? cvt8(f) : zero8());
      lds_store16(vt + v_pos<D>(r, c), ok ? vb : zero8());
    }
  }
};

// grid: x = run of cb key blocks, y = b * Hkv + g.  PER_BLOCK: every block's state goes to
// Hb (bf16) and z; otherwise the run's sum goes to Hf (fp32) and z at index y * gridDim.x + x.
// POOL: also kpool, each block's mean of the valid rows of K, [B, Hkv, nb, D] fp32, from fp64
// sums (each thread's rows, then the threads of a feature in a fixed order through LDS) and one
// rounding: the pooled keys of the prediction step, read here from the registers that already
// hold K, so K is read from memory once for both.
template <typename T, int D, bool PER_BLOCK, bool POOL>
__global__ __launch_bounds__(256) void kv_state_kernel(const T* __restrict__ k, int64_t ksB, int64_t ksH,
                                                       int64_t ksN, const T* __restrict__ v, int64_t vsB,
                                                       int64_t vsH, int64_t vsN, int Hkv, int nb, int n_valid,
                                                       int cb, const float* __restrict__ kshift,
                                                       u16* __restrict__ Hb, float* __restrict__ Hf,
                                                       float* __restrict__ zout, float* __restrict__ kpool) {
  constexpr int RB = 2 * D;
  constexpr int kCt = D == 128 ? 4 : 1;          // 32-column tiles of c per wavefront
  constexpr int kChunks = D / 8;                 // 16-byte chunks per 2D-byte row
  // phi(K) and V tiles; after a block's products the same 2 x 64 x 2D bytes stage its D x D bf16 state
  __shared__ __attribute__((aligned(1024))) unsigned char tsm[2 * kBlock * RB];
  constexpr int kRowGroups = 256 / kChunks;     // threads sharing one 8-feature chunk
  __shared__ double kred[POOL ? kRowGroups : 1][D];   // per-thread partial sums of the key block mean
  lds_u8* Kt = to_lds(tsm);
  lds_u8* Vt = Kt + kBlock * RB;
  const int x = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg % Hkv;
  const T* K = k + int64_t(b) * ksB + int64_t(g) * ksH;
  const T* V = v + int64_t(b) * vsB + int64_t(g) * vsH;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave;
  static_assert(256 % kChunks == 0, "a thread's K pieces share one 8-feature chunk");
  float shift[8];                                // smooth-K: this thread's 8 features of the key mean
#pragma unroll
  for (int m = 0; m < 8; ++m) shift[m] = kshift != nullptr ? kshift[int64_t(bg) * D + 8 * (t % kChunks) + m] : 0.f;
  const int rt = D == 128 ? w : w % 2;           // r rows 32 rt .. 32 rt + 31
  const int ct0 = D == 128 ? 0 : w / 2;          // first c tile
  const bool z_owner = D == 128 || w < 2;

  int aoff, boff[kCt];
  aoff = kv_operand_off<D>(32 * rt, lane);
#pragma unroll
  for (int ct = 0; ct < kCt; ++ct) boff[ct] = kv_operand_off<D>(32 * (ct0 + ct), lane);
  bf16x8 ones;
#pragma unroll
  for (int m = 0; m < 8; ++m) ones[m] = (__bf16)1.0f;

  f32x16 acc[kCt], zacc;
  auto clear = [&]() {
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct) acc[ct] = f32x16{};
    zacc = f32x16{};
  };
  // lane holds D[r = 32 rt + 8 q + 4 (lane / 32) + e % 4][c = 32 ct + lane % 32] in acc[ct][4 q + e % 4]
  // bf16 states go through LDS ([c][r], chunk c8 of row c at c8 ^ (c % kChunks)) so that every
  // wavefront store writes 1 KB of consecutive bytes; fp32 run sums are stored directly.
  auto store = [&](int64_t sidx) {
    const int c_l = lane % 32, r_l = 32 * rt + 4 * (lane / 32);
    if constexpr (PER_BLOCK) {
      __syncthreads();                  // every wavefront has read this block's operands
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        const int c = 32 * (ct0 + ct) + c_l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x4 = {acc[ct][4 * q], acc[ct][4 * q + 1], acc[ct][4 * q + 2], acc[ct][4 * q + 3]};
          const int ch = (r_l + 8 * q) / 8;
          lds_u8* pos = Kt + c * RB + 16 * (ch ^ (c % kChunks)) + 8 * (lane / 32);
          *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(pos) = __builtin_convertvector(x4, bf16x4);
        }
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < D * RB / (256 * 16); ++p) {
        const int e = t + 256 * p;
        const int row = e / kChunks, ch = e % kChunks;
        const bf16x8 x = lds_load16(Kt + row * RB + 16 * (ch ^ (row % kChunks)));
        *reinterpret_cast<bf16x8*>(Hb + sidx * D * D + row * D + 8 * ch) = x;
      }
    } else {
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        const int c = 32 * (ct0 + ct) + c_l;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x4 = {acc[ct][4 * q], acc[ct][4 * q + 1], acc[ct][4 * q + 2], acc[ct][4 * q + 3]};
          *reinterpret_cast<f32x4*>(Hf + sidx * D * D + int64_t(c) * D + r_l + 8 * q) = x4;
        }
      }
    }
    if (z_owner && c_l == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(zout + sidx * D + r_l + 8 * q) =
            f32x4{zacc[4 * q], zacc[4 * q + 1], zacc[4 * q + 2], zacc[4 * q + 3]};
    }
  };

  const int j0 = x * cb;
  const int j1 = min(min(nb, j0 + cb), (n_valid + kBlock - 1) / kBlock);   // blocks with valid rows
  clear();
  KvPiece<T, D> pc;
  if (j0 < j1) pc.load(K, ksN, V, vsN, j0, n_valid);
  for (int j = j0; j < j1; ++j) {
    __syncthreads();                    // the previous block's operands (and staged state) have been read
    double ps[8];
    pc.template store<POOL>(Kt, Vt, shift, ps);
    if constexpr (POOL) {
#pragma unroll
      for (int m = 0; m < 8; ++m) kred[t / kChunks][8 * (t % kChunks) + m] = ps[m];
    }
    __syncthreads();
    if (j + 1 < j1) pc.load(K, ksN, V, vsN, j + 1, n_valid);
    if (POOL && t < D) {                // after the next block's loads are issued; kred is rewritten
                                        // only after the next block's first barrier
      double tot = kred[0][t];
#pragma unroll
      for (int i = 1; i < kRowGroups; ++i) tot += kred[i][t];
      const int rows = min(kBlock, n_valid - kBlock * j);
      kpool[(int64_t(bg) * nb + j) * D + t] = float(rows == kBlock ? tot * (1.0 / kBlock) : tot / double(rows));
    }
#pragma unroll
    for (int ks = 0; ks < kBlock / 16; ++ks) {
      lds_u8* kk0 = Kt + 16 * ks * RB;
      lds_u8* vk0 = Vt + 16 * ks * RB;
      const bf16x8 a = tr_operand(kk0, aoff, 4 * RB);
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) acc[ct] = mfma32(a, tr_operand(vk0, boff[ct], 4 * RB), acc[ct]);
      if (z_owner) zacc = mfma32(a, ones, zacc);
    }
    if constexpr (PER_BLOCK) {
      store(int64_t(bg) * nb + j);
      clear();
    }
  }
  if constexpr (PER_BLOCK) {
    // blocks with no valid rows (only possible past n_valid): zero states
    for (int j = max(j0, j1); j < min(nb, j0 + cb); ++j) store(int64_t(bg) * nb + j);
  } else {
    store(int64_t(bg) * gridDim.x + x);
  }
}

// out[bg] = sum over p of in[bg * parts + p] (fixed order), for states of `len` floats, and the
// same for the z partials (zlen floats) in the workgroups from xh on: one launch for both.  The
// partials are read 16 at a time, all 16 loads in flight before the adds (one load at a time would
// expose a memory latency per partial).
__global__ __launch_bounds__(256) void sum_states_kernel(const float* __restrict__ in, const float* __restrict__ zin,
                                                         int parts, int64_t len, int64_t zlen, int xh,
                                                         float* __restrict__ out, float* __restrict__ zout) {
  constexpr int kU = 16;
  const bool is_z = int(blockIdx.x) >= xh;
  const float* src = is_z ? zin : in;
  float* dst = is_z ? zout : out;
  const int64_t n = is_z ? zlen : len;
  const int64_t bg = blockIdx.y;
  const int64_t e = (int64_t(is_z ? blockIdx.x - xh : blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < parts; p0 += kU) {
    f32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      x[u] = *reinterpret_cast<const f32x4*>(src + (bg * parts + min(p0 + u, parts - 1)) * n + e);
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u < parts) s += x[u];
  }
  *reinterpret_cast<f32x4*>(dst + bg * n + e) = s;
}

template <typename T>
static void launch_kv(const sla_tensor* k, const sla_tensor* v, int n_valid, int cb, int nch, const float* kshift,
                      u16* Hb, float* Hf, float* z, float* kpool, hipStream_t st) {
  const int nb = k->N / kBlock;
  dim3 grid(nch, k->B * k->H);
  const T* kp = static_cast<const T*>(k->ptr);
  const T* vp = static_cast<const T*>(v->ptr);
#define SLA_KV_LAUNCH(DD, PB, PL)                                                                                \
  kv_state_kernel<T, DD, PB, PL><<<grid, 256, 0, st>>>(kp, k->sB, k->sH, k->sN, vp, v->sB, v->sH, v->sN, k->H, \
                                                       nb, n_valid, cb, kshift, Hb, Hf, z, kpool)
  const bool pool = kpool != nullptr;
  if (k->d == 128) {
    if (Hb != nullptr) { if (pool) SLA_KV_LAUNCH(128, true, true); else SLA_KV_LAUNCH(128, true, false); }
    else { if (pool) SLA_KV_LAUNCH(128, false, true); else SLA_KV_LAUNCH(128, false, false); }
  } else {
    if (Hb != nullptr) { if (pool) SLA_KV_LAUNCH(64, true, true); else SLA_KV_LAUNCH(64, true, false); }
    else { if (pool) SLA_KV_LAUNCH(64, false, true); else SLA_KV_LAUNCH(64, false, false); }
  }
#undef SLA_KV_LAUNCH
}

static void launch_sum(const float* in, const float* zin, int parts, int d, int bgs, float* out, float* zout,
                       hipStream_t st) {
  const int64_t len = int64_t(d) * d;
  const int xh = int((len / 4 + 255) / 256), xz = (d / 4 + 255) / 256;
  sum_states_kernel<<<dim3(uint32_t(xh + xz), bgs), 256, 0, st>>>(in, zin, parts, len, d, xh, out, zout);
}

}  // namespace sla

extern "C" sla_status sla_linear_kv_reduce(const sla_tensor* k, const sla_tensor* v, int32_t n_valid,
                                           const float* k_shift, void* H, float* z, float* H_all, float* z_all,
                                           float* k_pool, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(k);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if (!same_geometry(k, v) || k->H != v->H || k->B != v->B) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, k->N)) != SLA_OK) return st;
  if (H == nullptr && H_all == nullptr) return SLA_ERR_NULL;
  if ((H == nullptr) != (z == nullptr) || (H_all == nullptr) != (z_all == nullptr)) return SLA_ERR_NULL;
  if ((H != nullptr && (!aligned16(H) || !aligned16(z))) || (H_all != nullptr && (!aligned16(H_all) || !aligned16(z_all))))
    return SLA_ERR_ALIGN;
  if ((k_shift != nullptr && !aligned16(k_shift)) || (k_pool != nullptr && !aligned16(k_pool))) return SLA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = k->N / kBlock;
  const int d = k->d;
  const int bgs = k->B * k->H;
  const bool bf = k->dtype == SLA_BF16;
  if (H_all != nullptr) {
    // fp32 sums over runs of key blocks into the workspace, then over the runs
    const size_t need = sla_kv_reduce_workspace_bytes(k->B, k->H, k->N, d, H != nullptr, 1);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
    const int cb = kv_sum_run(nb, bgs);
    const int nch = (nb + cb - 1) / cb;
    float* Hp = static_cast<float*>(workspace);
    float* zp = Hp + int64_t(bgs) * nch * d * d;
    float* kp = H == nullptr ? k_pool : nullptr;   // the key block means come from one of the two passes
    if (bf) launch_kv<bf16raw>(k, v, n_valid, cb, nch, k_shift, nullptr, Hp, zp, kp, s);
    else launch_kv<float>(k, v, n_valid, cb, nch, k_shift, nullptr, Hp, zp, kp, s);
    launch_sum(Hp, zp, nch, d, bgs, H_all, z_all, s);
  }
  if (H != nullptr) {
    // runs of a few blocks per workgroup (one block of prefetch), at least ~2048 workgroups
    const int cb = std::max(1, std::min(4, nb * bgs / 2048));
    const int nch = (nb + cb - 1) / cb;
    if (bf) launch_kv<bf16raw>(k, v, n_valid, cb, nch, k_shift, static_cast<u16*>(H), nullptr, z, k_pool, s);
    else launch_kv<float>(k, v, n_valid, cb, nch, k_shift, static_cast<u16*>(H), nullptr, z, k_pool, s);
  }
  return launch_status();
}
