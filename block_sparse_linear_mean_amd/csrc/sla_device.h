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
