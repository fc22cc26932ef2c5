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

// Word 3 of a raw (untyped, stride 0) buffer resource on gfx9-family parts:
// 32-bit data format, so untyped loads return data and reads at or past
// num_records bytes return zeros.
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

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

// Two independent tiles sharing one operand, MFMAs interleaved so neither
// chain waits on its own previous result.  shared_is_a: the shared operand is
// the A side (acc_t += S * X_t), else the B side (acc_t += X_t * S).
template <typename T, int D, bool shared_is_a>
__device__ __forceinline__ void mma_tile2(f32x16& acc0, f32x16& acc1, const u32x4* x0,
                                          const u32x4* x1, const u32x4* sh) {
  constexpr int NV = TileGeom<T, D>::NV;
  if constexpr (std::is_same<T, bf16_t>::value) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const bf16x8 s = __builtin_bit_cast(bf16x8, sh[v]);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, x0[v]);
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, x1[v]);
      if constexpr (shared_is_a) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s, a0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s, a1, acc1, 0, 0, 0);
      } else {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, s, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, s, acc1, 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const f32x4 s = __builtin_bit_cast(f32x4, sh[v]);
      const f32x4 a0 = __builtin_bit_cast(f32x4, x0[v]);
      const f32x4 a1 = __builtin_bit_cast(f32x4, x1[v]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (shared_is_a) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(s[e], a0[e], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(s[e], a1[e], acc1, 0, 0, 0);
        } else {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[e], s[e], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[e], s[e], acc1, 0, 0, 0);
        }
      }
    }
  }
}

// Sum of 16 values as a balanced tree (short dependency chains).
__device__ __forceinline__ float sum16(const float* p) {
  const float a = (p[0] + p[1]) + (p[2] + p[3]);
  const float b = (p[4] + p[5]) + (p[6] + p[7]);
  const float c = (p[8] + p[9]) + (p[10] + p[11]);
  const float d = (p[12] + p[13]) + (p[14] + p[15]);
  return (a + b) + (c + d);
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

// Wait until every vector-memory load this wave issued has completed
// (s_waitcnt vmcnt(0), expcnt and lgkmcnt left open), and keep the scheduler
// from moving instructions across the wait.
__device__ __forceinline__ void vm_wait_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Inclusive prefix sum over the 64 lanes in lane order, on the VALU through
// DPP (row shifts within each 16-lane row, then the row broadcasts of lanes
// 15 and 31), with no LDS round trip.  Lanes without a source read 0.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// src[0] + src[stride] + ... + src[(n - 1) stride], added in that order from
// +0 (bit for bit the plain loop's result), with eight loads in flight per
// round instead of one memory round trip per term.
__device__ __forceinline__ float ordered_strided_sum(const float* src, int64_t stride, int n) {
  float s = 0.f;
  for (int i0 = 0; i0 < n; i0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i0 + i < n ? src[(int64_t)(i0 + i) * stride] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i0 + i < n) s += v[i];
  }
  return s;
}

// Sum over each group of 4 consecutive lanes (DPP quad permutes).
__device__ __forceinline__ int quad_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  return x;
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, WAVE);
}

// x plus its value in lane l ^ 16 (add_xor16) or l ^ 32 (add_xor32), in
// every lane, without LDS: v_permlane16_swap / v_permlane32_swap exchange
// 16-lane (32-lane) halves between two registers; both hold x, so each lane
// ends with its own value and its partner's, whose sum (commutative) equals
// x + __shfl_xor(x, 16 / 32) bit for bit.
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Which sequence a flat work-item index belongs to: first[i] is the first item
// of sequence i, first[nb] the total.  nb <= MAXB, so a scan is cheap.
__device__ __forceinline__ int find_seq(const int32_t* first, int nb, int item) {
  int p = 0;
  while (p + 1 < nb && item >= first[p + 1]) ++p;
  return p;
}

}  // namespace waits
