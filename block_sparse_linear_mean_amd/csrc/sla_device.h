// Device-side helpers shared by the libsla kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

constexpr int kBlock = 64;   // tokens per pooled / attention block
constexpr int kWave = 64;    // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

// Raw bf16 storage type used for global tensors.
struct bf16raw { u16 bits; };

__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// 16x16x32 bf16 matrix-core product: D = A(16x32) * B(32x16) + C.
// Lane l holds A[l % 16][8 * (l / 16) .. +8], B[8 * (l / 16) .. +8][l % 16],
// and D[4 * (l / 16) + e][l % 16] for e = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cvt8(f32x8 x) { return __builtin_convertvector(x, bf16x8); }

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of 8 bf16 values in fp32: four two-element dot products against (1, 1)
__device__ __forceinline__ float sum8_bf16(bf16x8 x) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, s, false);
}

// 32x32x16 bf16 matrix-core product: D = A(32x16) * B(16x32) + C.
// Lane l holds A[l % 32][8 * (l / 32) .. +8], B[8 * (l / 32) .. +8][l % 32],
// and D[8 * (e / 4) + 4 * (l / 32) + e % 4][l % 32] for e = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ lds_u8* to_lds(void* p) { return (lds_u8*)p; }

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
__device__ __forceinline__ bf16x8 lds_load16(const lds_u8* p) { return *(const lds_bf16x8*)p; }
__device__ __forceinline__ void lds_store16(lds_u8* p, bf16x8 v) { *(lds_bf16x8*)p = v; }

// Transposing LDS read of 16-bit data (gfx950).  Within each group of 16 lanes, lane i
// receives element (i % 4) of the 8 bytes addressed by lane 4 * e + i / 4, for e = 0..3.
// So if lane k of a group addresses row r0 + k / 4, columns c0 + 4 (k % 4) .. +3 of a
// row-major 16-bit matrix, lane i receives rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ bf16x4 lds_read_tr4(lds_u8* addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
  return __builtin_bit_cast(bf16x4, v);
}

// Row-major LDS tile of 16-bit elements with RB-byte rows, laid out for the transposing read:
// 16-byte chunk c of row r sits at r * RB + 16 * (c ^ 2 (r % 4)).  A 16-lane group of the
// transposing read touches 4 consecutive rows in one 32-byte column window; the XOR moves the
// four rows' windows onto different banks.
template <int RB>
__device__ __forceinline__ int trs_pos(int r, int c) { return r * RB + 16 * (c ^ (2 * (r % 4))); }

// Per-lane byte offset of a 32x32x16 matrix-core operand read with two transposing reads from a
// trs-layout tile T[k][m]: lane l receives T[k0 + 8 (l / 32) + 0..7][m0 + l % 32], which is the A
// operand of A[m][k] = T[k][m] and the B operand of B[k][n] = T[k][n].  Read it as
// tr_operand(tile + k0 * RB, off, 4 * RB) for any k0 that is a multiple of 4.
template <int RB>
__device__ __forceinline__ int tr_operand_off(int m0, int lane) {
  const int sg = (lane / 16) % 2, kk = lane % 16, lg = lane / 32;
  return trs_pos<RB>(8 * lg + kk / 4, m0 / 8 + 2 * sg + (kk % 4) / 2) + 8 * (kk % 2);
}
__device__ __forceinline__ bf16x8 tr_operand(lds_u8* tile_k0, int off, int hi_step) {
  const bf16x4 lo = lds_read_tr4(tile_k0 + off);
  const bf16x4 hi = lds_read_tr4(tile_k0 + off + hi_step);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at lds + 16 l
// (lds must be the same for the whole wavefront).  Issued from a self-contained asm block
// (M0 set inside it, no output registers), so the copy's completion is tracked only by the
// caller's explicit SLA_WAIT_VMCNT: the compiler would otherwise drain every copy in flight
// before any LDS read, which serialises the K/V pipeline.
__device__ __forceinline__ void load_lds16(const void* gsrc, lds_u8* lds) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gsrc), "s"(lds_addr)
      : "memory");
}

// The same copy with a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte offset, which
// keeps the per-lane address state to one 32-bit register per distinct offset.  (The kernels using
// this issue nothing else that reads or writes M0.)
__device__ __forceinline__ void load_lds16_sbase(const void* sbase, uint32_t voff_bytes, lds_u8* lds) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff_bytes), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// The 4-byte form: lane l's dword lands at lds + 4 l.
__device__ __forceinline__ void load_lds4_sbase(const void* sbase, uint32_t voff_bytes, lds_u8* lds) {
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff_bytes), "s"(sbase), "s"(lds_addr)
      : "memory");
}

// max / sum with the partner lane l ^ 32 (v_permlane32_swap, no LDS round trip).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dealt round-robin to the 8 XCDs of the chip, each with its own L2.  This maps a
// hardware workgroup index of a 1-D grid of n to a logical index such that the workgroups one XCD
// receives form one contiguous range of the logical order (in dispatch order within the range).
__device__ __forceinline__ int xcd_logical(int bid, int n) {
  const int xcd = bid % 8, slot = bid / 8;
  const int q = n / 8, r = n % 8;
  return xcd * q + min(xcd, r) + slot;
}

// s_waitcnt encodings (gfx9 family): wait until at most N vector-memory operations of this
// wavefront are outstanding; the other counters are left unconstrained.
#define SLA_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8))
// wait until this wavefront's LDS operations have completed (lgkmcnt(0)), nothing else
#define SLA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))
// Workgroup barrier without a memory fence: the compiler may not move memory operations across
// it, and the caller states with SLA_WAIT_* which of its own operations must have completed.
// (A fenced barrier would also wait for every direct-to-LDS load still in flight.)
#define SLA_BARRIER()                 \
  do {                                \
    asm volatile("" ::: "memory");    \
    __builtin_amdgcn_s_barrier();     \
    asm volatile("" ::: "memory");    \
  } while (0)

// Eight consecutive input elements as bf16 (bf16 inputs: one 16-byte load; fp32: two).
template <typename T> struct In;
template <> struct In<bf16raw> {
  static constexpr int kVec = 8;  // elements per 16-byte load
  __device__ __forceinline__ static bf16x8 load8(const bf16raw* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static void load8_f32(const bf16raw* p, float* out) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(a[i] << 16);
      out[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
  }
};
template <> struct In<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static bf16x8 load8(const float* p) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    f32x8 x = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return cvt8(x);
  }
  __device__ __forceinline__ static void load8_f32(const float* p, float* out) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
  }
};

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// phi = elu + 1 (alpha = 1).
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

}  // namespace sla
