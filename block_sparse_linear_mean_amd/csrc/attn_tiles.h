// LDS tiles of 64 rows of a [*, d] bf16 tensor and their global -> LDS copies, shared by the
// attention forward and backward kernels.
#pragma once

#include "sla_device.h"

namespace sla {

// Tile geometry of one 64-key block of K or V in LDS: row-major bf16, 16-byte chunks
// permuted within each row so that both readers are free of bank conflicts:
//  * K is read as the A operand of S^T = K Q^T (16 contiguous bytes per lane, 32 rows at a
//    time): chunk c of row r sits at position c ^ (r % chunks);
//  * V is read with the transposing LDS read (8 bytes per lane, 4 rows x 32 bytes per
//    16-lane group): chunk c of row r sits at position c ^ 2 (r % 4).
// The epilogue's S^T tile ([c][r], 128 x 128 bf16) reuses the K layout over both buffers.
template <int D>
struct AttnTile {
  static constexpr int kRowB = 2 * D;             // bytes per row
  static constexpr int kChunks = D / 8;           // 16-byte chunks per row
  static constexpr int kTileB = kBlock * kRowB;   // one 64-row tile
  static constexpr int kInst = kTileB / 1024;     // 1 KB direct-load steps per tile
};

template <int D>
__device__ __forceinline__ int k_pos(int r, int c) {
  return r * AttnTile<D>::kRowB + 16 * (c ^ (r % AttnTile<D>::kChunks));
}
// V layout: the transposing-read swizzle c ^ 2 (r % 4); at d = 128 also the chunks whose bit 1
// is set move to the other half of the row (c ^ 8): the two 16-lane groups of a 32-lane read
// pass then touch disjoint banks (chunks 4 dt + {0, 1} and 4 dt + {2, 3} of the same 4 rows).
template <int D>
__device__ __forceinline__ int v_pos(int r, int c) {
  if constexpr (D == 128) return r * AttnTile<D>::kRowB + 16 * (c ^ (2 * (r % 4)) ^ (8 * ((c >> 1) & 1)));
  return trs_pos<AttnTile<D>::kRowB>(r, c);
}
// The chunk that v_pos places at position pos of row r (its inverse within a row).
template <int D>
__device__ __forceinline__ int v_chunk_at(int r, int pos) {
  if constexpr (D == 128) return pos ^ (2 * (r % 4)) ^ (8 * (((pos >> 1) & 1) ^ (r & 1)));
  return pos ^ (2 * (r % 4));
}

// Stage rows 64 j .. 64 j + 63 of X (row stride sN elements) into an LDS tile.  bf16 inputs go
// straight from global memory to LDS: a 1 KB step q covers R = 1024 / rowbytes rows, and lane l
// fetches the global chunk that belongs at LDS offset q * 1024 + 16 l.  With the swizzles above
// that chunk's byte offset from the step's first row is a per-lane constant, except for the K
// layout at d = 128 where it takes 4 values (q % 4); so each wavefront keeps at most four 32-bit
// offsets and all other address arithmetic is wave-uniform.  fp32 inputs are converted through
// registers.  The NW wavefronts of a workgroup split the tile's steps.
template <int D, int NW>
struct StageOff {
  static constexpr int kSteps = AttnTile<D>::kInst / NW;   // steps per wavefront
  static constexpr int kLanes = kSteps < 4 ? kSteps : 4;
  uint32_t lane[kLanes];          // per-lane part of this wavefront's step n, index n % kLanes
  uint32_t step[kSteps];          // this wavefront's steps: byte offset of the step's first row
};

template <int D, bool KLAYOUT, int NW>
__device__ __forceinline__ StageOff<D, NW> stage_offsets(int64_t sN) {
  using Tl = AttnTile<D>;
  using SO = StageOff<D, NW>;
  constexpr int R = 1024 / Tl::kRowB;             // rows per 1 KB step: 4 (d 128) or 8 (d 64)
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = (16 * lane) / Tl::kRowB;          // row within the step
  const int pc = lane % Tl::kChunks;              // physical chunk
  SO o;
#pragma unroll
  for (int m = 0; m < SO::kLanes; ++m) {
    const int q = w * SO::kSteps + m;             // q % 4 repeats with period 4 in m
    const int c = KLAYOUT ? pc ^ ((q * R + r) % Tl::kChunks) : v_chunk_at<D>(r, pc);
    o.lane[m] = uint32_t(2 * (r * sN + 8 * c));
  }
#pragma unroll
  for (int n = 0; n < SO::kSteps; ++n)
    o.step[n] = uint32_t(int64_t(w * SO::kSteps + n) * R * sN * 2);
  return o;
}

template <typename T, int D, bool KLAYOUT, int NW>
__device__ __forceinline__ void stage_tile(const T* __restrict__ X, int64_t sN, int j, lds_u8* tile,
                                           const StageOff<D, NW>& off) {
  using Tl = AttnTile<D>;
  using SO = StageOff<D, NW>;
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);   // wave-uniform: the LDS base goes to M0
  if constexpr (sizeof(T) == 2) {
    // one 64-bit tile base per tile; each copy adds a wave-uniform step offset to a per-lane offset
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(X) + int64_t(kBlock * j) * sN * 2;
#pragma unroll
    for (int n = 0; n < SO::kSteps; ++n) {
      const int q = w * SO::kSteps + n;
      const uint32_t vo = off.lane[KLAYOUT ? n % SO::kLanes : 0] + off.step[n];
      load_lds16_sbase(tb, vo, tile + q * 1024);
    }
  } else {
#pragma unroll
    for (int n = 0; n < Tl::kChunks * kBlock / (kWave * NW); ++n) {
      const int e = t + kWave * NW * n;
      const int r = e / Tl::kChunks, c = e % Tl::kChunks;
      const bf16x8 x = In<T>::load8(X + int64_t(kBlock * j + r) * sN + 8 * c);
      lds_store16(tile + (KLAYOUT ? k_pos<D>(r, c) : v_pos<D>(r, c)), x);
    }
  }
}

// Half tiles: rows 32 h .. 32 h + 31 of a tile are 1 KB steps h * kInst / 2 ... of it, shared by
// the NW wavefronts (kInst / 2 / NW steps each).  The per-lane part of a step's offset is that of
// the full-tile copy (it depends on the step only through step % 4, which both orders share);
// the wave-uniform part is the step's first row relative to the half's first row.
template <int D, int NW>
struct HalfSteps {
  static constexpr int kSteps = AttnTile<D>::kInst / 2 / NW;
  uint32_t step[kSteps];
  uint32_t klane[kSteps];   // the K layout's per-lane part of step n (used at d = 128 with 2 steps)
};

template <int D, int NW>
__device__ __forceinline__ HalfSteps<D, NW> half_steps(int64_t sN) {
  using Tl = AttnTile<D>;
  constexpr int R = 1024 / Tl::kRowB;
  constexpr int kS = HalfSteps<D, NW>::kSteps;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r = (16 * lane) / Tl::kRowB, pc = lane % Tl::kChunks;
  HalfSteps<D, NW> o;
#pragma unroll
  for (int n = 0; n < kS; ++n) {
    o.step[n] = uint32_t(int64_t(kS * w + n) * R * sN * 2);
    // a half's step q = h kInst / 2 + kS w + n leaves the remainder (kS w + n) % 4 (kInst / 2 is
    // a multiple of 4 at d = 128), which is all the K layout's chunk order depends on
    const int c = pc ^ (((kS * w + n) * R + r) % Tl::kChunks);
    o.klane[n] = uint32_t(2 * (r * sN + 8 * c));
  }
  return o;
}

// Stage rows 32 h .. 32 h + 31 of key block j of X into the same rows of an LDS tile (the
// layout of stage_tile).
template <typename T, int D, bool KLAYOUT, int NW>
__device__ __forceinline__ void stage_half(const T* __restrict__ X, int64_t sN, int j, int h, lds_u8* tile,
                                           const StageOff<D, NW>& off, const HalfSteps<D, NW>& hs) {
  using Tl = AttnTile<D>;
  constexpr int kHS = HalfSteps<D, NW>::kSteps;
  // the K layout's per-lane offset depends on the step only at d = 128, through step % 4: the
  // half's step q = h kInst/2 + kHS w + n has the remainder of this wavefront's full-tile step
  // m = (q - kSteps w) % 4 = (n + (kHS - kSteps) w) % 4, which is n (kHS = 4) or n + 2 w (kHS = 2)
  static_assert(kHS >= 1 && (D == 64 || kHS == 4 || kHS == 2), "half tiles: unsupported wavefront count");
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);
  if constexpr (sizeof(T) == 2) {
    const unsigned char* tb = reinterpret_cast<const unsigned char*>(X) + int64_t(kBlock * j + 32 * h) * sN * 2;
#pragma unroll
    for (int n = 0; n < kHS; ++n) {
      const int q = h * (Tl::kInst / 2) + kHS * w + n;
      uint32_t lo = off.lane[0];
      if constexpr (KLAYOUT && D == 128) {
        if constexpr (kHS == 4) lo = off.lane[n];
        else lo = hs.klane[n];   // computed per step: a select between two entries of off.lane
                                 // becomes an indexed read that the compiler moves to LDS
      }
      const uint32_t vo = lo + hs.step[n];
      load_lds16_sbase(tb, vo, tile + q * 1024);
    }
  } else {
#pragma unroll
    for (int n = 0; n < Tl::kChunks * 32 / (kWave * NW); ++n) {
      const int e = t + kWave * NW * n;
      const int r = 32 * h + e / Tl::kChunks, c = e % Tl::kChunks;
      const bf16x8 x = In<T>::load8(X + int64_t(kBlock * j + r) * sN + 8 * c);
      lds_store16(tile + (KLAYOUT ? k_pos<D>(r, c) : v_pos<D>(r, c)), x);
    }
  }
}

}  // namespace sla
