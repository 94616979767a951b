// Marginal aggregation: per map row, the sums S = sum_j H_j and u = sum_j z_j over the
// row's marginal key blocks, which the linear branch of the attention epilogue reads as
// phi(q)^T S / (phi(q) . u).
//
// Method: marginal pairs get linear attention through per-key-block states (SLA analysis
// page for arXiv 2509.24006: critical pairs FlashAttention, marginal pairs linear attention
// at O(N d^2)).
//
// Design: gathering each row's states reads n_m whole d x d states per query block (about
// 10 GB of cache traffic for the 12-head 32K-token layer), so the sums are instead one
// product per head, S = M H, of the 0/1 marginal mask M [nqb x nkb] with the bf16 states
// H [nkb x d*d] (and z), on the bf16 matrix cores, computed transposed (S^T = H^T M^T) so that a
// lane's accumulators hold 4 consecutive state columns of one row.
// A workgroup owns 256 map rows x 128 state columns; each of its 4 wavefronts takes 64 rows and
// all 128 columns, so each expanded mask operand feeds 4 products.  H tiles (32 key
// blocks x 128 columns, 8 KB) go straight from global memory to LDS in a 4-stage ring, in the
// bank-conflict-free layout of the transposing LDS read that feeds the A operand; the mask comes in as one bit per
// (row, key block), staged in LDS 512 key blocks at a time, and each lane expands 8 bits into
// its B operand.  A wavefront skips a step whose 64 x 32 mask block is all zero.  Sums
// accumulate in fp32 in a fixed order (deterministic); S is written once in bf16, the
// precision the epilogue consumes, re-staged through LDS for 1 KB-contiguous stores.  The z columns (u) take the same
// path from fp32 z converted to bf16 operands, in workgroups dispatched first.  State workgroups
// are numbered so that the row tiles of one column slice run on one XCD and share its L2.
#include "attn_tiles.h"
#include "sla_device.h"
#include "sla_host.h"

namespace sla {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMgRows = 256;    // map rows per workgroup
constexpr int kMgCols = 128;    // state columns per workgroup (256-byte tile rows)
constexpr int kMgK = 32;        // key blocks per step (one mask word)
constexpr int kMgStages = 4;    // H tiles in flight
constexpr int kMgWords = 16;    // mask words per row held in LDS (512 key blocks)
constexpr int kMgTileB = kMgK * kMgCols * 2;

// 8 mask bits -> 8 bf16 values 1.0 / 0.0 (bit m -> element m).  z = byte * 0x8001 holds the byte
// twice, at bits 0..7 and 15..22, so bit 16 + 2k of z is bit 2k + 1 of the byte: word k keeps bits
// 2k and 16 + 2k of z and scales them to bf16(1.0) = 0x3F80 in its low and high half with one
// 24-bit multiply by 0x3F80 >> 2k (exact: 0x3F80 is a multiple of 2^7).  Ten VALU operations with
// the byte extraction.
__device__ __forceinline__ bf16x8 expand_bits(uint32_t byte) {
  const uint32_t z = byte * 0x8001u;
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = (z & (0x00010001u << (2 * k))) * (0x3F80u >> (2 * k));
  return __builtin_bit_cast(bf16x8, w);
}

// 1-D grid: z workgroups (B * Hs * ceil(D / 128) * n_row_tiles, padded to a multiple of 8), then
// B * Hs * (D * D / 128) * n_row_tiles state workgroups.
template <int D>
__global__ __launch_bounds__(256) void marginal_gemm_kernel(const u16* __restrict__ H, const float* __restrict__ z,
                                                            int Hq, int Hkv, int Hs, int nqb, int nkb, int group_map,
                                                            const uint32_t* __restrict__ bits, u16* __restrict__ S,
                                                            float* __restrict__ u, int n_row_tiles, int n_z,
                                                            int n_zwg) {
  __shared__ __attribute__((aligned(1024))) unsigned char bsm[kMgStages][kMgTileB];
  __shared__ uint32_t mask[kMgRows][kMgWords + 1];

  // The first n_zwg workgroups (a multiple of 8) take the z columns, which go through registers
  // and take longer, so they start first; the state slices follow in XCD-contiguous order.
  constexpr int kStateSlices = D * D / kMgCols;
  constexpr int kZSlices = (D + kMgCols - 1) / kMgCols;
  const bool is_z = int(blockIdx.x) < n_zwg;
  int it, slice, bs;
  if (is_z) {
    const int zi = blockIdx.x;
    if (zi >= n_z) return;
    it = zi % n_row_tiles;
    slice = (zi / n_row_tiles) % kZSlices;
    bs = zi / n_row_tiles / kZSlices;
  } else {
    const int logical = xcd_logical(blockIdx.x - n_zwg, gridDim.x - n_zwg);
    it = logical % n_row_tiles;
    const int rest = logical / n_row_tiles;
    slice = rest % kStateSlices;
    bs = rest / kStateSlices;
  }
  const int b = bs / Hs, s = bs % Hs;
  const int g = group_map ? s : s / (Hq / Hkv);
  const int c0 = slice * kMgCols;
  const int64_t head = int64_t(b) * Hkv + g;
  const int t = threadIdx.x, lane = t % kWave;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);   // wave-uniform (feeds M0 and SGPR bases)
  const int row0 = it * kMgRows;
  const int nw = (nkb + 31) / 32;
  const int nsteps = nw;

  // ---- H tile staging: step ks holds key blocks 32 ks .. 32 ks + 31 (rows past nkb repeat row
  // nkb - 1; their mask bits are zero), columns c0 .. c0 + 127
  const u16* hsrc = H + head * nkb * D * D + c0;
  // H tiles have 256-byte rows, the rows of a d = 128 V tile: they take its layout (v_pos), whose
  // chunk order keeps a 32-lane transposing-read pass on 64 distinct banks (the plain transposing
  // layout puts two lanes on each bank at this row size).  Row 4 qi + lrow leaves lrow mod 4.
  const int lrow = lane / 16, lchunk = v_chunk_at<128>(lrow, lane % 16);
  auto issue = [&](int ks) {
    lds_u8* dst = to_lds(bsm[ks % kMgStages]);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int qi = 2 * w + n;                    // 1 KB step: rows 4 qi .. 4 qi + 3
      const int j = min(kMgK * ks + 4 * qi + lrow, nkb - 1);
      const uint32_t voff = uint32_t(j) * uint32_t(D * D * 2) + 16u * uint32_t(lchunk);
      load_lds16_sbase(hsrc, voff, dst + qi * 1024);
    }
  };
  // z slice: fp32 z rows converted to bf16 through registers (columns past D are zero)
  auto fill_z = [&](int ks) {
    lds_u8* dst = to_lds(bsm[ks % kMgStages]);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int e = t + 256 * n;                   // 512 chunks of 8 columns
      const int r = e / 16, c = e % 16;
      const int j = kMgK * ks + r, col = c0 + 8 * c;
      f32x8 x;
      if (j < nkb && col < D) {
        const float* zp = z + (head * nkb + j) * D + col;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(zp), hi = *reinterpret_cast<const f32x4*>(zp + 4);
        x = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) x[m] = 0.f;
      }
      lds_store16(dst + v_pos<128>(r, c), cvt8(x));
    }
  };

  // wavefront w: rows 64 w .. 64 w + 63 (two 32-row tiles) x all 128 columns (four 32-column tiles);
  // each expanded mask operand feeds 4 products
  f32x16 acc[2][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rr][ct][e] = 0.f;
  int aoff[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    // the operand lane l reads with the two transposing reads (as tr_operand_off, in the v_pos layout)
    const int sg = (lane / 16) % 2, kk = lane % 16, lg = lane / 32;
    aoff[ct] = v_pos<128>(8 * lg + kk / 4, 4 * ct + 2 * sg + (kk % 4) / 2) + 8 * (kk % 2);
  }
  const bool my_row = row0 + t < nqb;
  const uint32_t* my_bits = bits + (int64_t(bs) * nqb + min(row0 + t, nqb - 1)) * nw;

  auto load_mask = [&](int wc) {                   // words wc .. wc + 15 of this thread's row
    uint32_t wv[kMgWords];
#pragma unroll
    for (int q = 0; q < kMgWords; ++q) wv[q] = my_bits[min(wc + q, nw - 1)];   // all loads in flight at once
#pragma unroll
    for (int q = 0; q < kMgWords; ++q) mask[t][q] = (my_row && wc + q < nw) ? wv[q] : 0u;
  };

  if (!is_z) {
    for (int ks = 0; ks < min(kMgStages - 1, nsteps); ++ks) issue(ks);
    load_mask(0);                                  // overlaps the first copies' latency
  }
  for (int ks = 0; ks < nsteps; ++ks) {
    if (is_z) {
      __syncthreads();
      if (ks % kMgWords == 0) load_mask(ks);
      fill_z(ks);
      __syncthreads();
    } else {
      // this wavefront's copies of step ks are done once at most those of the later steps in flight are
      const int later = min(kMgStages - 2, nsteps - 1 - ks);
      if (later >= 2) SLA_WAIT_VMCNT(4);
      else if (later == 1) SLA_WAIT_VMCNT(2);
      else SLA_WAIT_VMCNT(0);
      SLA_WAIT_LGKM0();
      SLA_BARRIER();                               // step ks landed for every wavefront; step ks - 1 is consumed
      if (ks % kMgWords == 0 && ks > 0) {          // next 512 key blocks of mask words
        load_mask(ks);
        SLA_WAIT_LGKM0();
        SLA_BARRIER();
      }
      if (ks + kMgStages - 1 < nsteps) issue(ks + kMgStages - 1);
    }
    lds_u8* tile = to_lds(bsm[ks % kMgStages]);
    const int wq = ks % kMgWords;
    const uint32_t w0 = mask[64 * w + lane % 32][wq];
    const uint32_t w1 = mask[64 * w + 32 + lane % 32][wq];
    if (__ballot((w0 | w1) != 0u) == 0) continue;  // no marginal block of this wavefront's rows here
    // every A operand of the step (key blocks 16 h .. 16 h + 15, column tiles ct) is requested
    // first, the mask operands are expanded while they are in flight, then the 16 products
    bf16x8 a[2][4], bm[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) a[h][ct] = tr_operand(tile + 16 * h * 256, aoff[ct], 4 * 256);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sh = 8 * (2 * h + lane / 32);
      bm[h][0] = expand_bits((w0 >> sh) & 0xffu);
      bm[h][1] = expand_bits((w1 >> sh) & 0xffu);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        acc[0][ct] = mfma32(a[h][ct], bm[h][0], acc[0][ct]);
        acc[1][ct] = mfma32(a[h][ct], bm[h][1], acc[1][ct]);
      }
  }

  // lane holds S[row0 + 64 w + 32 rr + lane % 32][c0 + 32 ct + 8 q + 4 (lane / 32) + 0..3] in acc[rr][ct][4 q ..]
  if (is_z) {
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int i = row0 + 64 * w + 32 * rr + lane % 32;
      if (i >= nqb) continue;
      const int64_t r = int64_t(bs) * nqb + i;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = c0 + 32 * ct + 8 * q + 4 * (lane / 32);
          if (col < D)
            *reinterpret_cast<f32x4*>(u + r * D + col) =
                f32x4{acc[rr][ct][4 * q], acc[rr][ct][4 * q + 1], acc[rr][ct][4 * q + 2], acc[rr][ct][4 * q + 3]};
        }
    }
    return;
  }
  // S in bf16 through LDS (128 rows x 256 bytes at a time in the H ring, chunk c16 of row r at
  // c16 ^ (r % 16)), so that every wavefront store writes 1 KB of consecutive bytes
  lds_u8* stg = to_lds(bsm[0]);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
    if (w / 2 == half) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 64 * (w % 2) + 32 * rr + lane % 32;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 x4 = {acc[rr][ct][4 * q], acc[rr][ct][4 * q + 1], acc[rr][ct][4 * q + 2], acc[rr][ct][4 * q + 3]};
            lds_u8* pos = stg + row * 256 + 16 * ((4 * ct + q) ^ (row % 16)) + 8 * (lane / 32);
            *reinterpret_cast<__attribute__((address_space(3))) bf16x4*>(pos) = __builtin_convertvector(x4, bf16x4);
          }
      }
    }
    SLA_WAIT_LGKM0();
    SLA_BARRIER();
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int e = t + 256 * p;
      const int row = e / 16, ch = e % 16;
      const int i = row0 + 128 * half + row;
      if (i < nqb) {
        const bf16x8 x = lds_load16(stg + row * 256 + 16 * (ch ^ (row % 16)));
        *reinterpret_cast<bf16x8*>(S + (int64_t(bs) * nqb + i) * D * D + c0 + 8 * ch) = x;
      }
    }
  }
}

sla_status launch_marginal_states(const u16* H, const float* z, int B, int Hq, int Hkv, int nqb, int nkb, int d,
                                  int group_map, const uint32_t* bits, u16* S, float* u, hipStream_t st) {
  const int Hs = group_map ? Hkv : Hq;
  const int n_row_tiles = (nqb + kMgRows - 1) / kMgRows;
  const int64_t n_state = int64_t(B) * Hs * (d * d / kMgCols) * n_row_tiles;
  const int64_t n_z = int64_t(B) * Hs * ((d + kMgCols - 1) / kMgCols) * n_row_tiles;
  const int64_t n_zwg = (n_z + 7) / 8 * 8;
  const int64_t n = n_zwg + n_state;
  if (n > (int64_t(1) << 31) - 1) return SLA_ERR_UNSUPPORTED;
  if (d == 128)
    marginal_gemm_kernel<128><<<dim3(uint32_t(n)), 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, bits, S, u,
                                                                 n_row_tiles, int(n_z), int(n_zwg));
  else
    marginal_gemm_kernel<64><<<dim3(uint32_t(n)), 256, 0, st>>>(H, z, Hq, Hkv, Hs, nqb, nkb, group_map, bits, S, u,
                                                                n_row_tiles, int(n_z), int(n_zwg));
  return launch_status();
}

}  // namespace sla

extern "C" sla_status sla_marginal_states(const void* H, const float* z, int32_t B, int32_t Hq, int32_t Hkv,
                                          int32_t nqb, int32_t nkb, int32_t d, int32_t group_map,
                                          const uint32_t* marg_bits, void* S, float* u, void* stream) {
  using namespace sla;
  if (H == nullptr || z == nullptr || marg_bits == nullptr || S == nullptr || u == nullptr) return SLA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || nqb < 1 || nkb < 1) return SLA_ERR_SHAPE;
  if (nkb > SLA_MAX_KEY_BLOCKS) return SLA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SLA_ERR_UNSUPPORTED;
  if (!aligned16(H) || !aligned16(z) || !aligned16(S) || !aligned16(u)) return SLA_ERR_ALIGN;
  return launch_marginal_states(static_cast<const u16*>(H), z, B, Hq, Hkv, nqb, nkb, d, group_map ? 1 : 0, marg_bits,
                                static_cast<u16*>(S), u, static_cast<hipStream_t>(stream));
}
