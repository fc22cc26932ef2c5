// Device building blocks shared by the WAITS kernels (gfx950 / CDNA4).
//
// Both QK^T passes are built from one MFMA shape, v_mfma_f32_32x32x16_bf16
// (bf16 inputs) or v_mfma_f32_32x32x2_f32 (fp32 inputs), on 32 x 32 output
// tiles held by one 64-lane wavefront:
//   A operand (32 x Dk): lane l supplies row (l % 32);
//   B operand (Dk x 32): lane l supplies column (l % 32);
//   both with the same contraction slots, so loading the same head-dim
//   elements into the same (lane half, register) positions of A and B makes
//   the instruction sequence compute full dot products.  Lane half hf = l / 32
//   carries head-dim elements [hf * D/2, (hf + 1) * D/2).
//   Output: lane l holds column (l % 32) and the 16 rows
//   8 * (v / 4) + 4 * hf + (v % 4), v = 0..15.
// Every lane therefore owns one output column with 16 of its rows, so a
// reduction along rows (over keys in pass 1, over queries in pass 2) is
// in-lane work plus one exchange between the two lane halves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace waits {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tag for bf16 inputs (the kernels only move and multiply their bits).
struct bf16_t {
  uint16_t bits;
};

constexpr int WAVE = 64;
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * WAVE;
constexpr int TILE = 32;  // rows of an MFMA operand tile
constexpr int MAXB = 32;  // sequences per launch (tables travel as kernel arguments)

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Geometry of one 32-row operand tile of head_dim D and element type T.
template <typename T, int D>
struct TileGeom {
  static constexpr int ELT = sizeof(T);
  static constexpr int ROW_BYTES = D * ELT;
  static constexpr int NV = ROW_BYTES / 32;          // 16-B vectors per lane (half a row)
  static constexpr int LDS_STRIDE = ROW_BYTES + 16;  // padded row pitch in LDS
  static constexpr int STAGE_V = ROW_BYTES / 128;    // 16-B vectors per thread per tile
  static constexpr int LDS_BYTES = TILE * LDS_STRIDE;
  static_assert(ROW_BYTES % 128 == 0, "row must split into 8 x 16-byte parts");
};

// acc += A * B over the whole head dimension.  a and b are the lane's
// NV vectors of its half row.
template <typename T, int D>
__device__ __forceinline__ void mma_tile(f32x16& acc, const u32x4* a,
                                         const u32x4* b) {
  constexpr int NV = TileGeom<T, D>::NV;
  if constexpr (std::is_same<T, bf16_t>::value) {
#pragma unroll
    for (int v = 0; v < NV; ++v)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, a[v]), __builtin_bit_cast(bf16x8, b[v]),
          acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const f32x4 av = __builtin_bit_cast(f32x4, a[v]);
      const f32x4 bv = __builtin_bit_cast(f32x4, b[v]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], acc, 0, 0, 0);
    }
  }
}

// Row index (within the 32-row A tile) of output register v for lane half hf.
__device__ __forceinline__ constexpr int out_row(int v, int hf) {
  return 8 * (v >> 2) + 4 * hf + (v & 3);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, WAVE);
}

// Which sequence a flat work-item index belongs to: first[i] is the first item
// of sequence i, first[nb] the total.  nb <= MAXB, so a scan is cheap.
__device__ __forceinline__ int find_seq(const int32_t* first, int nb, int item) {
  int p = 0;
  while (p + 1 < nb && item >= first[p + 1]) ++p;
  return p;
}

}  // namespace waits
