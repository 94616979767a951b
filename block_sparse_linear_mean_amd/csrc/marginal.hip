// Marginal aggregation: per map row, the sums S = sum_j H_j and u = sum_j z_j over the
// row's marginal key blocks, which the linear branch of the attention epilogue reads as
// phi(q)^T S / (phi(q) . u).
//
// Method: marginal pairs get linear attention through per-key-block states (SLA analysis
// page for arXiv 2509.24006: critical pairs FlashAttention, marginal pairs linear attention
// at O(N d^2)).
//
// Design: gathering each row's states reads n_m whole d x d states per query block (about
// 20 GB of cache traffic for the 12-head 32K-token layer), so the sums are instead one
// product per head, S = M H, of the 0/1 marginal mask M [nqb x nkb] with the states
// H [nkb x d*d] (and z), on the bf16 matrix cores: H is read about once.  The mask comes in
// as one bit per (row, key block), as the classification writes it; each workgroup stages its
// rows' words in LDS and every lane expands its 8 mask bits into the 8 bf16 ones/zeros of its
// A operand.  B tiles
// (32 key blocks x 128 state columns) are converted to bf16 and staged row-major in LDS with
// 16-byte stores, and read back k-packed with the transposing LDS read (rows padded to 288 bytes,
// so every 16-lane group's four rows x 32 bytes hit all banks once); double buffered behind a
// register prefetch.  Each wavefront owns 64 rows x 128 columns,
// so one mask expansion feeds 8 matrix-core products.  Sums accumulate in fp32 in a fixed order
// (deterministic); S is written once in bf16, the precision the epilogue consumes.
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMgRows = 256;     // map rows per workgroup: 4 wavefronts x 64
constexpr int kMgCols = 128;     // state columns per workgroup
constexpr int kMgChunkW = 16;    // mask words per row held at once (512 key blocks)
constexpr int kMgBs = 128 + 16;  // LDS row stride of the row-major B tile (bf16): 288 bytes

// 8 mask bits -> 8 bf16 values 1.0 / 0.0 (bit m -> element m).
__device__ __forceinline__ bf16x8 expand_bits(uint32_t byte) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t two = (byte >> (2 * k)) & 3u;
    w[k] = ((two & 1u) | ((two & 2u) << 15)) * 0x3F80u;   // bf16(1.0) in the low / high half
  }
  return __builtin_bit_cast(bf16x8, w);
}

// grid: x = tile of 256 map rows, y = 128-column slice (state columns, then z columns),
// z = b * Hs + s.
template <int D>
__global__ __launch_bounds__(256) void marginal_gemm_kernel(const float* __restrict__ H, const float* __restrict__ z,
                                                            int Hq, int Hkv, int Hs, int nqb, int nkb, int group_map,
                                                            const uint32_t* __restrict__ bits,
                                                            u16* __restrict__ S, float* __restrict__ u) {
  __shared__ uint32_t mask[kMgRows][kMgChunkW + 1];
  __shared__ __attribute__((aligned(16))) u16 Bt[2][32 * kMgBs];

  const int it = blockIdx.x, slice = blockIdx.y, bs = blockIdx.z;
  const int b = bs / Hs, s = bs % Hs;
  const int g = group_map ? s : s / (Hq / Hkv);
  constexpr int kStateSlices = D * D / kMgCols;
  const bool is_z = slice >= kStateSlices;
  const int width = is_z ? D : D * D;
  const int c0 = is_z ? (slice - kStateSlices) * kMgCols : slice * kMgCols;
  const float* src = (is_z ? z + (int64_t(b) * Hkv + g) * nkb * D : H + (int64_t(b) * Hkv + g) * nkb * D * D) + c0;
  const int64_t row0 = int64_t(bs) * nqb + int64_t(it) * kMgRows;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave, l16 = lane % 16, lg = lane / 16;

  const int nw = (nkb + 31) / 32;
  const bool my_row = it * kMgRows + t < nqb;     // this thread stages the mask words of row0 + t
  const uint32_t* my_bits = bits + (row0 + t) * nw;

  constexpr int kCt = kMgCols / 16;
  f32x4 acc[4][kCt];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < kCt; ++c) acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B-tile load mapping: rows (key blocks) t / 16 and t / 16 + 16, columns cc .. cc + 7
  const int jr = t / 16, cc = 8 * (t % 16);
  const int nks_total = (nkb + 31) / 32;
  f32x4 pre[2][2];
  const bool col_ok = c0 + cc < width;   // z of d = 64 fills half a slice
  auto load_b = [&](int ksg) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = 32 * ksg + jr + 16 * q;
      const float* rp = src + int64_t(j) * width + cc;
      const bool ok = j < nkb && col_ok;
      pre[q][0] = ok ? *reinterpret_cast<const f32x4*>(rp) : f32x4{0.f, 0.f, 0.f, 0.f};
      pre[q][1] = ok ? *reinterpret_cast<const f32x4*>(rp + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // transposing-read address of this lane: row 8 (lane / 16) + (lane % 16) / 4, column 4 (lane % 4)
  const int tr_off = (8 * lg + (lane % 16) / 4) * kMgBs + 4 * (lane % 4);
  load_b(0);
  int buf = 0;
  for (int jc = 0; jc < nkb; jc += 32 * kMgChunkW) {
    __syncthreads();   // the previous chunk's masks are no longer read
#pragma unroll
    for (int q = 0; q < kMgChunkW; ++q) {
      const int wq = jc / 32 + q;
      mask[t][q] = (my_row && wq < nw) ? my_bits[wq] : 0u;
    }
    const int nks = min(kMgChunkW, (nkb - jc + 31) / 32);
    for (int ks = 0; ks < nks; ++ks) {
      const int ksg = jc / 32 + ks;
      u16* bt = Bt[buf];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const f32x8 x = {pre[q][0][0], pre[q][0][1], pre[q][0][2], pre[q][0][3],
                         pre[q][1][0], pre[q][1][1], pre[q][1][2], pre[q][1][3]};
        *reinterpret_cast<bf16x8*>(bt + (jr + 16 * q) * kMgBs + cc) = cvt8(x);
      }
      __syncthreads();
      if (ksg + 1 < nks_total) load_b(ksg + 1);
      // B[k = 8 lg + m][col 16 ct + l16]: rows 8 lg .. 8 lg + 3 and 8 lg + 4 .. 8 lg + 7
      lds_u8* bl = to_lds(bt);
      bf16x8 bop[kCt];
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        const bf16x4 lo = lds_read_tr4(bl + 2 * (tr_off + 16 * ct));
        const bf16x4 hi = lds_read_tr4(bl + 2 * (tr_off + 4 * kMgBs + 16 * ct));
        bop[ct] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const uint32_t word = mask[64 * w + 16 * rt + l16][ks];
        const bf16x8 aop = expand_bits((word >> (8 * lg)) & 0xffu);
#pragma unroll
        for (int ct = 0; ct < kCt; ++ct) acc[rt][ct] = mfma16(aop, bop[ct], acc[rt][ct]);
      }
      buf ^= 1;
    }
  }

  // lane holds rows 64 w + 16 rt + 4 lg + e, column c0 + 16 ct + l16
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = it * kMgRows + 64 * w + 16 * rt + 4 * lg + e;
      if (i >= nqb) continue;
      const int64_t r = int64_t(bs) * nqb + i;
#pragma unroll
      for (int ct = 0; ct < kCt; ++ct) {
        const int col = c0 + 16 * ct + l16;
        if (is_z) {
          if (col < D) u[r * D + col] = acc[rt][ct][e];
        } else {
          const __bf16 v = (__bf16)acc[rt][ct][e];
          S[r * D * D + col] = __builtin_bit_cast(u16, v);
        }
      }
    }
}

sla_status launch_marginal_states(const float* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const uint32_t* bits, u16* S, float* u, hipStream_t st) {
  const int Hs = group_map ? Hkv : Hq;
  dim3 grid((nqb + kMgRows - 1) / kMgRows, d * d / kMgCols + (d + kMgCols - 1) / kMgCols, B * Hs);
  if (d == 128)
    marginal_gemm_kernel<128><<<grid, 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, bits, S, u);
  else
    marginal_gemm_kernel<64><<<grid, 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, bits, S, u);
  return launch_status();
}

}  // namespace sla

extern "C" sla_status sla_marginal_states(const float* H, const float* z, int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t nqb, int32_t nkb, int32_t d, int32_t group_map,
                                          const uint32_t* marg_bits, void* S, float* u, void* stream) {
  using namespace sla;
  if (H == nullptr || z == nullptr || marg_bits == nullptr || S == nullptr || u == nullptr) return SLA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || nqb < 1 || nkb < 1) return SLA_ERR_SHAPE;
  if (nkb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SLA_ERR_UNSUPPORTED;
  if (!aligned16(H) || !aligned16(z) || !aligned16(S) || !aligned16(u)) return SLA_ERR_ALIGN;
  return launch_marginal_states(H, z, B, Hq, Hkv, nqb, nkb, d, group_map ? 1 : 0, marg_bits, static_cast<u16*>(S), u,
                                static_cast<hipStream_t>(stream));
}
