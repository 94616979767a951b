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
// the operand layout the attention epilogue reads (16 contiguous bytes along r).
//
// Design (gfx950): one workgroup per (KV head, chunk of key blocks).  K and V blocks
// are loaded with 16-byte reads and written to LDS transposed ([feature][token]), with
// phi applied to K and rounded to bf16, so both matrix-core operands of the
// token contraction read 16 contiguous bytes per lane.  Each of the 4 wavefronts
// owns a quarter of the d x d output in fp32 accumulators; a chunk of several blocks
// accumulates in registers before one store.  The pass is HBM-bound and
// write-dominated (a fp32 state per block is twice the bytes of the block's K and V).
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

template <typename T, int D>
struct KvTile {
  static constexpr int kTpt = D / 32;            // tokens per thread in the transposing load
  static constexpr int kTg = kBlock / kTpt;      // token groups
  static constexpr int kStride = kBlock + 8;     // LDS row stride (bf16 elements)
};

// Loads key block j (rows >= n_valid as zero) into Kt = bf16(phi(K))^T and Vt = bf16(V)^T.
template <typename T, int D>
__device__ __forceinline__ void load_kv_transposed(const T* __restrict__ K, int64_t ksN, const T* __restrict__ V,
                                                   int64_t vsN, int j, int n_valid, u16* Kt, u16* Vt) {
  using Tile = KvTile<T, D>;
  const int t = threadIdx.x;
  const int tg = t % Tile::kTg, fg = t / Tile::kTg;    // tokens kTpt*tg.., features 8*fg..
  float kv[Tile::kTpt][8], vv[Tile::kTpt][8];
#pragma unroll
  for (int u = 0; u < Tile::kTpt; ++u) {
    const int tok = Tile::kTpt * tg + u;
    const int s = kBlock * j + tok;
    if (s < n_valid) {
      In<T>::load8_f32(K + int64_t(s) * ksN + 8 * fg, kv[u]);
      In<T>::load8_f32(V + int64_t(s) * vsN + 8 * fg, vv[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[u][e] = phi(kv[u][e]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kv[u][e] = vv[u][e] = 0.f;   // padding contributes nothing
    }
  }
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int row = 8 * fg + f;
    const int col = Tile::kTpt * tg;
    if constexpr (Tile::kTpt == 4) {
      typedef float f32x4_t __attribute__((ext_vector_type(4)));
      f32x4_t a = {kv[0][f], kv[1][f], kv[2][f], kv[3][f]};
      f32x4_t b = {vv[0][f], vv[1][f], vv[2][f], vv[3][f]};
      *reinterpret_cast<bf16x4*>(Kt + row * Tile::kStride + col) = __builtin_convertvector(a, bf16x4);
      *reinterpret_cast<bf16x4*>(Vt + row * Tile::kStride + col) = __builtin_convertvector(b, bf16x4);
    } else {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      typedef float f32x2_t __attribute__((ext_vector_type(2)));
      f32x2_t a = {kv[0][f], kv[1][f]};
      f32x2_t b = {vv[0][f], vv[1][f]};
      *reinterpret_cast<bf16x2*>(Kt + row * Tile::kStride + col) = __builtin_convertvector(a, bf16x2);
      *reinterpret_cast<bf16x2*>(Vt + row * Tile::kStride + col) = __builtin_convertvector(b, bf16x2);
    }
  }
}

// grid: x = chunk of `cb` key blocks, y = b * Hkv + g.  Output state index = y * nch + x,
// so with cb == 1 the output is laid out [B, Hkv, nb, d, d] / [B, Hkv, nb, d].
template <typename T, int D>
__global__ __launch_bounds__(256) void kv_state_kernel(const T* __restrict__ k, int64_t ksB, int64_t ksH,
                                                       int64_t ksN, const T* __restrict__ v, int64_t vsB,
                                                       int64_t vsH, int64_t vsN, int Hkv, int nb, int n_valid,
                                                       int cb, float* __restrict__ Hout,
                                                       float* __restrict__ zout) {
  using Tile = KvTile<T, D>;
  constexpr int kRt = D / 16 / 4;   // row tiles per wavefront
  constexpr int kCt = D / 16;       // column tiles
  __shared__ __attribute__((aligned(16))) u16 Kt[D * Tile::kStride];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * Tile::kStride];
  const int c = blockIdx.x, bg = blockIdx.y;
  const int nch = gridDim.x;
  const int b = bg / Hkv, g = bg % Hkv;
  const T* K = k + int64_t(b) * ksB + int64_t(g) * ksH;
  const T* V = v + int64_t(b) * vsB + int64_t(g) * vsH;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave, l16 = lane % 16, lg = lane / 16;

  f32x4 acc[kRt][kCt];
#pragma unroll
  for (int a = 0; a < kRt; ++a)
#pragma unroll
    for (int e = 0; e < kCt; ++e) acc[a][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;

  const int j0 = c * cb, j1 = min(nb, j0 + cb);
  for (int j = j0; j < j1; ++j) {
    if (kBlock * j >= n_valid) break;
    __syncthreads();
    load_kv_transposed<T, D>(K, ksN, V, vsN, j, n_valid, Kt, Vt);
    __syncthreads();
    if (t < D) {   // z: sum of the rounded phi(K) of this block, fixed order
      const u16* row = Kt + t * Tile::kStride;
#pragma unroll
      for (int s8 = 0; s8 < kBlock; s8 += 8) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(row + s8);
#pragma unroll
        for (int e = 0; e < 8; ++e) zacc += float(x[e]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < kBlock / 32; ++ks) {
      bf16x8 bv[kCt];
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct)
        bv[ct] = *reinterpret_cast<const bf16x8*>(Vt + (16 * ct + l16) * Tile::kStride + 32 * ks + 8 * lg);
#pragma unroll
      for (int a = 0; a < kRt; ++a) {
        const int rt = kRt * w + a;
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(Kt + (16 * rt + l16) * Tile::kStride + 32 * ks + 8 * lg);
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) acc[a][ct] = mfma16(av, bv[ct], acc[a][ct]);
      }
    }
  }
  // store transposed, [c][r]: lane holds r = 16 rt + 4 lg + e (e < 4) for c = 16 ct + l16
  const int64_t sidx = int64_t(bg) * nch + c;
  float* Hs = Hout + sidx * D * D;
#pragma unroll
  for (int a = 0; a < kRt; ++a) {
    const int rt = kRt * w + a;
#pragma unroll
    for (int ct = 0; ct < kCt; ++ct)
      *reinterpret_cast<f32x4*>(Hs + (16 * ct + l16) * D + 16 * rt + 4 * lg) = acc[a][ct];
  }
  if (t < D) zout[sidx * D + t] = zacc;
}

// out[bg] = sum over p of in[bg * parts + p] (fixed order), for states of `len` floats.
__global__ __launch_bounds__(256) void sum_states_kernel(const float* __restrict__ in, int parts, int64_t len,
                                                         float* __restrict__ out) {
  const int64_t bg = blockIdx.y;
  const int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (e >= len) return;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < parts; ++p) s += *reinterpret_cast<const f32x4*>(in + (bg * parts + p) * len + e);
  *reinterpret_cast<f32x4*>(out + bg * len + e) = s;
}

template <typename T>
static void launch_kv(const sla_tensor* k, const sla_tensor* v, int n_valid, int cb, int nch, float* H, float* z,
                      hipStream_t st) {
  const int nb = k->N / kBlock;
  dim3 grid(nch, k->B * k->H);
  const T* kp = static_cast<const T*>(k->ptr);
  const T* vp = static_cast<const T*>(v->ptr);
  if (k->d == 128)
    kv_state_kernel<T, 128><<<grid, 256, 0, st>>>(kp, k->sB, k->sH, k->sN, vp, v->sB, v->sH, v->sN, k->H, nb,
                                                  n_valid, cb, H, z);
  else
    kv_state_kernel<T, 64><<<grid, 256, 0, st>>>(kp, k->sB, k->sH, k->sN, vp, v->sB, v->sH, v->sN, k->H, nb,
                                                 n_valid, cb, H, z);
}

static void launch_sum(const float* in, int parts, int64_t len, int bgs, float* out, hipStream_t st) {
  dim3 grid(uint32_t((len / 4 + 255) / 256), bgs);
  sum_states_kernel<<<grid, 256, 0, st>>>(in, parts, len, out);
}

}  // namespace sla

extern "C" sla_status sla_linear_kv_reduce(const sla_tensor* k, const sla_tensor* v, int32_t n_valid, float* H,
                                           float* z, float* H_all, float* z_all, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  using namespace sla;
  sla_status st = check_tensor(k);
  if (st != SLA_OK) return st;
  if ((st = check_tensor(v)) != SLA_OK) return st;
  if (!same_geometry(k, v) || k->H != v->H || k->B != v->B) return SLA_ERR_SHAPE;
  if ((st = check_valid_len(n_valid, k->N)) != SLA_OK) return st;
  if (H == nullptr && H_all == nullptr) return SLA_ERR_NULL;
  if ((H == nullptr) != (z == nullptr) || (H_all == nullptr) != (z_all == nullptr)) return SLA_ERR_NULL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nb = k->N / kBlock;
  const int d = k->d;
  const int bgs = k->B * k->H;
  const bool bf = k->dtype == SLA_BF16;
  if (H != nullptr) {
    if (bf) launch_kv<bf16raw>(k, v, n_valid, 1, nb, H, z, s);
    else launch_kv<float>(k, v, n_valid, 1, nb, H, z, s);
    if (H_all != nullptr) {
      launch_sum(H, nb, int64_t(d) * d, bgs, H_all, s);
      launch_sum(z, nb, d, bgs, z_all, s);
    }
    return launch_status();
  }
  const size_t need = sla_kv_reduce_workspace_bytes(k->B, k->H, k->N, d, 0, 1);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return SLA_ERR_WORKSPACE;
  const int cb = 32;
  const int nch = (nb + cb - 1) / cb;
  float* Hp = static_cast<float*>(workspace);
  float* zp = Hp + int64_t(bgs) * nch * d * d;
  if (bf) launch_kv<bf16raw>(k, v, n_valid, cb, nch, Hp, zp, s);
  else launch_kv<float>(k, v, n_valid, cb, nch, Hp, zp, s);
  launch_sum(Hp, nch, int64_t(d) * d, bgs, H_all, s);
  launch_sum(zp, nch, d, bgs, z_all, s);
  return launch_status();
}
