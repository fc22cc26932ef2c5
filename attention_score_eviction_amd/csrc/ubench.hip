// Microbenchmarks of the QK^T passes' instruction mix on gfx950: what one
// 16x16x32 bf16 MFMA, one exponential epilogue element-instruction triple
// (v_fma_f32, v_exp_f32, v_add_f32, as in p = exp2(s * c - off); sum += p)
// and their combinations cost per SIMD.  Measurement only: built into its
// own library (libwaits_ubench.so), never part of the WAITS path.
//
// Every wave runs ITERS iterations of one mode's loop body (8 independent
// MFMA chains and/or 8 independent VALU chains, so issue rate and not
// latency bounds it) and records its shader-clock cycles (s_memtime) and
// 100 MHz real-time ticks (s_memrealtime).  Waves w and w + 4 of a workgroup
// share a SIMD (hardware wave -> SIMD map, also reported), so 256 threads
// put one wave on each SIMD of a CU, 512 threads two.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

// The WAITS select kernel with its phase marks recorded: thread 0 of each
// workgroup stamps the shader clock (s_memtime) at the end of each phase.
__device__ long long g_select_marks[256 * 9];
#define WAITS_SELECT_MARK(k)                                                                 \
  do {                                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < 256) g_select_marks[blockIdx.x * 9 + (k)] = __builtin_amdgcn_s_memtime(); \
  } while (0)
#include "select_compact.hpp"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

enum Mode {
  M_MFMA = 0,        // 8 MFMAs
  M_TRIPLE = 1,      // 8 (fma, exp, add) triples
  M_EXP = 2,         // 8 exps
  M_FMA = 3,         // 8 fmas
  M_ADD = 4,         // 8 adds
  M_MIXED = 5,       // 8 MFMAs and 8 triples, interleaved by the compiler
  M_CLUSTERS = 6,    // 8 MFMAs, then 8 triples (scheduling barrier between)
  M_PRIO = 7,        // as M_CLUSTERS, MFMAs at raised wave priority
  M_SPLIT_TRIPLE = 8,  // waves < W/2: 8 MFMAs; the others: 8 triples
  M_SPLIT_FMA = 9,     // waves < W/2: 8 MFMAs; the others: 8 fmas
  M_SPLIT_EXP = 10,    // waves < W/2: 8 MFMAs; the others: 8 exps
  N_MODES = 11
};

template <int MODE>
__global__ void __launch_bounds__(512) mix_kernel(float* out, long long* stamps, int iters, float c) {
  constexpr int NM = 8, NV = 8;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (tid + i));
    b[i] = (__bf16)(0.002f * (tid - i));
  }
  f32x4 acc[NM];
  for (int m = 0; m < NM; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  float x[NV], sum[NV];
  for (int v = 0; v < NV; ++v) {
    x[v] = 0.01f * (tid + v);
    sum[v] = 0.f;
  }
  const bool split = MODE >= M_SPLIT_TRIPLE;
  const bool do_m = MODE == M_MFMA || MODE == M_MIXED || MODE == M_CLUSTERS || MODE == M_PRIO ||
                    (split && wave < nw / 2);
  const bool do_v = (MODE >= M_TRIPLE && MODE <= M_PRIO) || (split && wave >= nw / 2);
  constexpr bool triple = MODE == M_TRIPLE || MODE == M_MIXED || MODE == M_CLUSTERS || MODE == M_PRIO ||
                          MODE == M_SPLIT_TRIPLE;
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if (do_m) {
      if constexpr (MODE == M_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m], 0, 0, 0);
      if constexpr (MODE == M_PRIO) __builtin_amdgcn_s_setprio(0);
    }
    if constexpr (MODE == M_CLUSTERS) __builtin_amdgcn_sched_barrier(0);
    if (do_v) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (triple) {
          sum[v] += __builtin_amdgcn_exp2f(fmaf(x[v], c, -sum[v]));
        } else if constexpr (MODE == M_EXP || MODE == M_SPLIT_EXP) {
          x[v] = __builtin_amdgcn_exp2f(x[v]);
        } else if constexpr (MODE == M_FMA || MODE == M_SPLIT_FMA) {
          x[v] = fmaf(x[v], c, -x[v]);
        } else {
          x[v] = x[v] + c;
        }
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
  for (int m = 0; m < NM; ++m) r += acc[m][0] + acc[m][3];
  for (int v = 0; v < NV; ++v) r += sum[v] + x[v];
  out[blockIdx.x * blockDim.x + tid] = r;
  if ((tid & 63) == 0) {
    const int w = blockIdx.x * nw + wave;
    stamps[2 * w] = t1 - t0;
    stamps[2 * w + 1] = r1 - r0;
  }
}

// HW_ID (hwreg 4): bits 5:4 = SIMD of the wave
__global__ void simd_map_kernel(int* out) {
  const unsigned hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
  if ((threadIdx.x & 63) == 0) out[threadIdx.x >> 6] = (int)((hw >> 4) & 3);
}

template <int MODE>
int run_mode(int threads, int blocks, int iters, float* out, long long* stamps, double* res) {
  hipLaunchKernelGGL(mix_kernel<MODE>, dim3(blocks), dim3(threads), 0, 0, out, stamps, 16, 1.0001f);
  hipLaunchKernelGGL(mix_kernel<MODE>, dim3(blocks), dim3(threads), 0, 0, out, stamps, iters, 1.0001f);
  if (hipDeviceSynchronize() != hipSuccess) return 4;
  const int nw = threads / 64, waves = blocks * nw;
  std::vector<long long> h((size_t)waves * 2);
  if (hipMemcpy(h.data(), stamps, sizeof(long long) * h.size(), hipMemcpyDeviceToHost) != hipSuccess) return 4;
  long long mx[2] = {0, 0}, rt = 0;
  for (int w = 0; w < waves; ++w) {
    const int half = (w % nw) >= nw / 2;
    mx[half] = std::max(mx[half], h[2 * w]);
    rt = std::max(rt, h[2 * w + 1]);
  }
  res[0] = (double)mx[0] / iters;   // cycles per iteration, slowest wave of the first half
  res[1] = (double)mx[1] / iters;   // ... of the second half
  res[2] = (double)std::max(mx[0], mx[1]) / ((double)rt / 100e6) / 1e9;   // shader clock, GHz
  return 0;
}

// The passes' own shape at NT = 4 row tiles (head_dim 128): per iteration a
// wave issues 32 MFMAs (8 accumulators x 4 head-dim steps) into acc[par]
// and the epilogue of acc[par ^ 1] (32 elements per lane: fma, exp2, add
// into four row sums), the two pinned into groups of G MFMAs followed by
// 3 G VALU instructions (G = 32: one cluster, as the kernels issue them).
// TM_MFMA and TM_EPI run only one of the two streams.
enum TileMode { TM_MFMA = 0, TM_EPI = 1, TM_MIX = 2 };

template <int TM, int G, int PRIO, int NT = 4, int LB = 512>
__global__ void __launch_bounds__(LB) tile_kernel(float* out, long long* stamps, int iters, float c) {
  static_assert(G >= 1 && G <= 32 && 32 % G == 0, "G divides 32");
  static_assert(NT >= 1 && NT <= 4 && (NT == 4 || (TM == TM_MIX && G == 32)), "fewer tiles: one cluster only");
  const int tid = threadIdx.x;
  bf16x8 a[4], b[2][4];
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)(0.001f * (tid + i + s));
      b[0][s][i] = (__bf16)(0.002f * (tid - i + s));
      b[1][s][i] = (__bf16)(0.003f * (tid - i - s));
    }
  f32x4 acc[2][2 * NT];
  for (int p = 0; p < 2; ++p)
    for (int m = 0; m < 2 * NT; ++m) acc[p][m] = f32x4{0.01f * m, 0.f, 0.f, 0.f};
  float m4[4] = {0.1f, 0.2f, 0.3f, 0.4f}, sum[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      if constexpr (TM != TM_EPI) {
        // opaque operands: the two parities' MFMAs are not merged or hoisted
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          asm volatile("" : "+v"(b[0][s]));
          asm volatile("" : "+v"(b[1][s]));
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              const int m = t * 2 + kt;
              acc[par][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  b[kt][s], a[t], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[par][m], 0, 0, 0);
            }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
      } else {
#pragma unroll
        for (int m = 0; m < 2 * NT; ++m) asm volatile("" : "+v"(acc[par ^ 1][m]));
      }
      if constexpr (TM != TM_MFMA) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float sv = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pv[i] = __builtin_amdgcn_exp2f(fmaf(acc[par ^ 1][t * 2 + kt][i], c, -m4[t]));
            sv += (pv[0] + pv[1]) + (pv[2] + pv[3]);
          }
          sum[t] += sv;
        }
      }
      if constexpr (TM == TM_MIX) {
        if constexpr (G < 32) {
#pragma unroll
          for (int g = 0; g < 32 / G; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, G, 0);      // G MFMAs
            __builtin_amdgcn_sched_group_barrier(0x002, 3 * G, 0);  // then 3 G VALU
          }
        } else {
          __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 96, 0);
        }
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
  for (int p = 0; p < 2; ++p)
    for (int m = 0; m < 2 * NT; ++m) r += acc[p][m][0] + acc[p][m][3];
  for (int t = 0; t < 4; ++t) r += sum[t];
  out[blockIdx.x * blockDim.x + tid] = r;
  if ((tid & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + (tid >> 6);
    stamps[2 * w] = t1 - t0;
    stamps[2 * w + 1] = r1 - r0;
  }
}

// res[0] = cycles per iteration (32 MFMAs and/or 32 epilogue elements per
// wave) of the slowest wave, res[1] = shader clock in GHz.
template <int TM, int G, int PRIO, int NT = 4, int LB = 512>
int run_tile(int threads, int blocks, int iters, float* out, long long* stamps, double* res) {
  if (threads > LB) return 1;
  hipLaunchKernelGGL((tile_kernel<TM, G, PRIO, NT, LB>), dim3(blocks), dim3(threads), 0, 0, out, stamps, 16, 1.0001f);
  hipLaunchKernelGGL((tile_kernel<TM, G, PRIO, NT, LB>), dim3(blocks), dim3(threads), 0, 0, out, stamps, iters,
                     1.0001f);
  if (hipDeviceSynchronize() != hipSuccess) return 4;
  const int waves = blocks * (threads / 64);
  std::vector<long long> h((size_t)waves * 2);
  if (hipMemcpy(h.data(), stamps, sizeof(long long) * h.size(), hipMemcpyDeviceToHost) != hipSuccess) return 4;
  long long mx = 0, rt = 0;
  for (int w = 0; w < waves; ++w) {
    mx = std::max(mx, h[2 * w]);
    rt = std::max(rt, h[2 * w + 1]);
  }
  res[0] = (double)mx / iters;
  res[1] = (double)mx / ((double)rt / 100e6) / 1e9;
  return 0;
}


// Operand placement in the passes' shape (one cluster at raised priority,
// four row tiles, the epilogue of the other accumulator set): OP_VGPR lets
// the compiler keep everything in arch VGPRs; OP_AGPR_AB issues the MFMAs
// from inline asm with both multiplicands in AGPRs and the accumulators in
// VGPRs (so only the epilogue's operands go through the VGPR file's read
// ports); OP_AGPR_ACC holds the accumulators in AGPRs (the epilogue reads
// them back with v_accvgpr_read).  Timing only: the asm form leaves the
// compiler no view of the MFMA hazards, so its values are not meaningful.
enum OperandPlace { OP_VGPR = 0, OP_AGPR_AB = 1, OP_AGPR_ACC = 2 };

template <int TM, int OP>
__global__ void __launch_bounds__(512) operand_kernel(float* out, long long* stamps, int iters, float c) {
  constexpr int NT = 4;
  const int tid = threadIdx.x;
  bf16x8 a[4], b[2][4];
  for (int s = 0; s < 4; ++s)
    for (int i = 0; i < 8; ++i) {
      a[s][i] = (__bf16)(0.001f * (tid + i + s));
      b[0][s][i] = (__bf16)(0.002f * (tid - i + s));
      b[1][s][i] = (__bf16)(0.003f * (tid - i - s));
    }
  if constexpr (OP == OP_AGPR_AB) {
    for (int s = 0; s < 4; ++s) asm volatile("" : "+a"(a[s]));
  }
  f32x4 acc[2][2 * NT];
  for (int p = 0; p < 2; ++p)
    for (int m = 0; m < 2 * NT; ++m) acc[p][m] = f32x4{0.01f * m, 0.f, 0.f, 0.f};
  float m4[4] = {0.1f, 0.2f, 0.3f, 0.4f}, sum[4] = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      if constexpr (TM != TM_EPI) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (OP == OP_AGPR_AB) {
            asm volatile("" : "+a"(b[0][s]));
            asm volatile("" : "+a"(b[1][s]));
          } else {
            asm volatile("" : "+v"(b[0][s]));
            asm volatile("" : "+v"(b[1][s]));
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              const int m = t * 2 + kt;
              if constexpr (OP == OP_AGPR_AB) {
                if (s == 0)
                  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                               : "=v"(acc[par][m]) : "a"(b[kt][s]), "a"(a[t]));
                else
                  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                               : "+v"(acc[par][m]) : "a"(b[kt][s]), "a"(a[t]));
              } else {
                acc[par][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    b[kt][s], a[t], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[par][m], 0, 0, 0);
              }
            }
        __builtin_amdgcn_s_setprio(0);
        if constexpr (OP == OP_AGPR_ACC) {
#pragma unroll
          for (int m = 0; m < 2 * NT; ++m) asm volatile("" : "+a"(acc[par][m]));
        }
      } else {
#pragma unroll
        for (int m = 0; m < 2 * NT; ++m) {
          if constexpr (OP == OP_AGPR_ACC) asm volatile("" : "+a"(acc[par ^ 1][m]));
          else asm volatile("" : "+v"(acc[par ^ 1][m]));
        }
      }
      if constexpr (TM != TM_MFMA) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float sv = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pv[i] = __builtin_amdgcn_exp2f(fmaf(acc[par ^ 1][t * 2 + kt][i], c, -m4[t]));
            sv += (pv[0] + pv[1]) + (pv[2] + pv[3]);
          }
          sum[t] += sv;
        }
      }
      if constexpr (TM == TM_MIX) {
        __builtin_amdgcn_sched_group_barrier(0x008, 32, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 96, 0);
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = 0.f;
  for (int p = 0; p < 2; ++p)
    for (int m = 0; m < 2 * NT; ++m) r += acc[p][m][0] + acc[p][m][3];
  for (int t = 0; t < 4; ++t) r += sum[t];
  out[blockIdx.x * blockDim.x + tid] = r;
  if ((tid & 63) == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + (tid >> 6);
    stamps[2 * w] = t1 - t0;
    stamps[2 * w + 1] = r1 - r0;
  }
}

template <int TM, int OP>
int run_operands(int blocks, int iters, float* out, long long* stamps, double* res) {
  hipLaunchKernelGGL((operand_kernel<TM, OP>), dim3(blocks), dim3(512), 0, 0, out, stamps, 16, 1.0001f);
  hipLaunchKernelGGL((operand_kernel<TM, OP>), dim3(blocks), dim3(512), 0, 0, out, stamps, iters, 1.0001f);
  if (hipDeviceSynchronize() != hipSuccess) return 4;
  const int waves = blocks * 8;
  std::vector<long long> h((size_t)waves * 2);
  if (hipMemcpy(h.data(), stamps, sizeof(long long) * h.size(), hipMemcpyDeviceToHost) != hipSuccess) return 4;
  long long mx = 0, rt = 0;
  for (int w = 0; w < waves; ++w) {
    mx = std::max(mx, h[2 * w]);
    rt = std::max(rt, h[2 * w + 1]);
  }
  res[0] = (double)mx / iters;
  res[1] = (double)mx / ((double)rt / 100e6) / 1e9;
  return 0;
}
}  // namespace

extern "C" {

// Runs every mode on `blocks` workgroups of `threads` (256 or 512) threads
// for `iters` iterations; res[3 * mode + {0, 1, 2}] = cycles per iteration
// of the slowest wave of the first and of the second half of each
// workgroup's waves, and the shader clock in GHz.  simd[w] (w < threads/64)
// = the SIMD wave w of a workgroup ran on.  Returns 0, or 4 on a HIP error.
int waits_ubench_mix(int threads, int blocks, int iters, double* res, int* simd) {
  if (threads != 256 && threads != 512) return 1;
  float* out = nullptr;
  long long* stamps = nullptr;
  int* map = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * threads) != hipSuccess) return 4;
  if (hipMalloc(&stamps, sizeof(long long) * 2 * blocks * (threads / 64)) != hipSuccess) return 4;
  if (hipMalloc(&map, sizeof(int) * 16) != hipSuccess) return 4;
  int rc = 0;
  rc = rc ? rc : run_mode<M_MFMA>(threads, blocks, iters, out, stamps, res + 3 * M_MFMA);
  rc = rc ? rc : run_mode<M_TRIPLE>(threads, blocks, iters, out, stamps, res + 3 * M_TRIPLE);
  rc = rc ? rc : run_mode<M_EXP>(threads, blocks, iters, out, stamps, res + 3 * M_EXP);
  rc = rc ? rc : run_mode<M_FMA>(threads, blocks, iters, out, stamps, res + 3 * M_FMA);
  rc = rc ? rc : run_mode<M_ADD>(threads, blocks, iters, out, stamps, res + 3 * M_ADD);
  rc = rc ? rc : run_mode<M_MIXED>(threads, blocks, iters, out, stamps, res + 3 * M_MIXED);
  rc = rc ? rc : run_mode<M_CLUSTERS>(threads, blocks, iters, out, stamps, res + 3 * M_CLUSTERS);
  rc = rc ? rc : run_mode<M_PRIO>(threads, blocks, iters, out, stamps, res + 3 * M_PRIO);
  rc = rc ? rc : run_mode<M_SPLIT_TRIPLE>(threads, blocks, iters, out, stamps, res + 3 * M_SPLIT_TRIPLE);
  rc = rc ? rc : run_mode<M_SPLIT_FMA>(threads, blocks, iters, out, stamps, res + 3 * M_SPLIT_FMA);
  rc = rc ? rc : run_mode<M_SPLIT_EXP>(threads, blocks, iters, out, stamps, res + 3 * M_SPLIT_EXP);
  if (rc == 0) {
    hipLaunchKernelGGL(simd_map_kernel, dim3(1), dim3(threads), 0, 0, map);
    if (hipMemcpy(simd, map, sizeof(int) * (threads / 64), hipMemcpyDeviceToHost) != hipSuccess) rc = 4;
  }
  (void)hipFree(out);
  (void)hipFree(stamps);
  (void)hipFree(map);
  return rc;
}

int waits_ubench_modes(void) { return N_MODES; }

// The fused select+compact (select_kernel<16, true>) on `layers` sequences of
// n keys, 8 KV heads, head_dim 128 (bf16), budget kept keys per head: the
// headline's shape at layers = 32, n = 16384, budget = 128.  Scores: a fixed
// hash of the position, most in [0, 1e-3) and one key in a hundred near 1 (a
// heavy-hitter-like tail).  res[0..7] = median cycles per workgroup of the
// phases between marks k and k + 1 (0 start, 1 first barrier, 2..5 the four
// radix passes, 6 totals, 7 output placed, 8 gather done), res[8] = median
// total cycles, res[9] = microseconds per launch (HIP events over 20).
int waits_ubench_select(int layers, int n, int budget, double* res) {
  const int hkv = 8, d = 128, heads = layers * hkv;
  if (layers < 1 || layers > waits::MAXB || heads > 256 || n < 1 || n > 16 * waits::SEL_THREADS) return 1;
  if (budget < 1 || budget > waits::SEL_FUSE_MAX) return 1;
  const int64_t T = (int64_t)layers * n;
  std::vector<float> hs((size_t)hkv * T);
  for (size_t i = 0; i < hs.size(); ++i) {
    uint32_t x = (uint32_t)i * 2654435761u;
    x ^= x >> 15;
    x *= 2246822519u;
    x ^= x >> 13;
    const float f = (float)(x >> 8) * (1.0f / 16777216.0f);
    hs[i] = (x % 100u == 0u) ? 0.5f + 0.5f * f : 1e-3f * f * f;
  }
  float* sc = nullptr;
  unsigned char *k = nullptr, *v = nullptr, *ko = nullptr, *vo = nullptr;
  int32_t* idx = nullptr;
  const size_t kv_bytes = (size_t)T * hkv * d * 2, out_bytes = (size_t)heads * budget * d * 2;
  int rc = 0;
  if (hipMalloc(&sc, hs.size() * 4) != hipSuccess || hipMalloc(&k, kv_bytes) != hipSuccess ||
      hipMalloc(&v, kv_bytes) != hipSuccess || hipMalloc(&ko, out_bytes) != hipSuccess ||
      hipMalloc(&vo, out_bytes) != hipSuccess || hipMalloc(&idx, (size_t)heads * budget * 4) != hipSuccess)
    rc = 4;
  if (!rc && hipMemcpy(sc, hs.data(), hs.size() * 4, hipMemcpyHostToDevice) != hipSuccess) rc = 4;
  if (!rc && (hipMemset(k, 0x3c, kv_bytes) != hipSuccess || hipMemset(v, 0x3d, kv_bytes) != hipSuccess)) rc = 4;
  std::vector<long long> marks(256 * 9);
  if (!rc) {
    waits::SelectArgs a;
    std::memset(&a, 0, sizeof(a));
    a.scores = sc;
    a.idx = idx;
    a.T = T;
    a.hkv = hkv;
    a.budget = budget;
    a.k = k;
    a.v = v;
    a.k_out = ko;
    a.v_out = vo;
    a.st.kv_tok = (int64_t)hkv * d;
    a.st.kv_head = d;
    a.elt = 2;
    a.row_shift = 4;  // 256-byte rows: 16 vectors of 16 bytes
    a.tab.nb = layers;
    for (int i = 0; i < layers; ++i) {
      a.tab.n[i] = n;
      a.tab.tok0[i] = (int64_t)i * n;
    }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) rc = 4;
    for (int w = 0; w < 5 && !rc; ++w)
      hipLaunchKernelGGL((waits::select_kernel<16, true>), dim3(heads), dim3(waits::SEL_THREADS), 0, 0, a);
    if (!rc && hipDeviceSynchronize() != hipSuccess) rc = 4;
    if (!rc && hipMemcpyFromSymbol(marks.data(), HIP_SYMBOL(g_select_marks), sizeof(long long) * marks.size()) !=
                   hipSuccess)
      rc = 4;
    if (!rc) {
      (void)hipEventRecord(e0, 0);
      for (int w = 0; w < 20; ++w)
        hipLaunchKernelGGL((waits::select_kernel<16, true>), dim3(heads), dim3(waits::SEL_THREADS), 0, 0, a);
      (void)hipEventRecord(e1, 0);
      float ms = 0.f;
      if (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) rc = 4;
      res[9] = ms * 1e3 / 20.0;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
  }
  if (!rc) {
    std::vector<long long> ph((size_t)heads);
    for (int k2 = 0; k2 <= 8; ++k2) {
      for (int h = 0; h < heads; ++h)
        ph[h] = k2 < 8 ? marks[h * 9 + k2 + 1] - marks[h * 9 + k2] : marks[h * 9 + 8] - marks[h * 9];
      std::nth_element(ph.begin(), ph.begin() + heads / 2, ph.end());
      res[k2] = (double)ph[heads / 2];
    }
  }
  (void)hipFree(sc);
  (void)hipFree(k);
  (void)hipFree(v);
  (void)hipFree(ko);
  (void)hipFree(vo);
  (void)hipFree(idx);
  return rc;
}

// The passes' shape (tile_kernel) on `blocks` workgroups of `threads` (256
// or 512) threads; configurations in order: MFMAs only, epilogue only, one
// cluster at raised priority, then groups of G = 32, 16, 8, 4, 2, 1 MFMAs.
// res[2 * i + {0, 1}] = cycles per iteration of the slowest wave, clock GHz.
int waits_ubench_tile(int threads, int blocks, int iters, double* res) {
  if (threads != 256 && threads != 512) return 1;
  if (iters < 2 || iters % 2) return 1;
  float* out = nullptr;
  long long* stamps = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * threads) != hipSuccess) return 4;
  if (hipMalloc(&stamps, sizeof(long long) * 2 * blocks * (threads / 64)) != hipSuccess) return 4;
  int rc = 0;
  rc = rc ? rc : run_tile<TM_MFMA, 32, 0>(threads, blocks, iters, out, stamps, res + 0);
  rc = rc ? rc : run_tile<TM_EPI, 32, 0>(threads, blocks, iters, out, stamps, res + 2);
  rc = rc ? rc : run_tile<TM_MIX, 32, 1>(threads, blocks, iters, out, stamps, res + 4);
  rc = rc ? rc : run_tile<TM_MIX, 32, 0>(threads, blocks, iters, out, stamps, res + 6);
  rc = rc ? rc : run_tile<TM_MIX, 16, 0>(threads, blocks, iters, out, stamps, res + 8);
  rc = rc ? rc : run_tile<TM_MIX, 8, 0>(threads, blocks, iters, out, stamps, res + 10);
  rc = rc ? rc : run_tile<TM_MIX, 4, 0>(threads, blocks, iters, out, stamps, res + 12);
  rc = rc ? rc : run_tile<TM_MIX, 2, 0>(threads, blocks, iters, out, stamps, res + 14);
  rc = rc ? rc : run_tile<TM_MIX, 1, 0>(threads, blocks, iters, out, stamps, res + 16);
  (void)hipFree(out);
  (void)hipFree(stamps);
  return rc;
}

// The kernels' one-cluster order at more waves per SIMD: configurations
// (threads, row tiles per wave) = (512, 4), (768, 4), (768, 3), (1024, 3),
// (1024, 2) on `blocks` workgroups; res[2 * i + {0, 1}] = cycles per
// iteration of the slowest wave and the clock in GHz.
int waits_ubench_tile_waves(int blocks, int iters, double* res) {
  if (iters < 2 || iters % 2) return 1;
  float* out = nullptr;
  long long* stamps = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * 1024) != hipSuccess) return 4;
  if (hipMalloc(&stamps, sizeof(long long) * 2 * blocks * 16) != hipSuccess) return 4;
  int rc = 0;
  rc = rc ? rc : run_tile<TM_MIX, 32, 1, 4, 512>(512, blocks, iters, out, stamps, res + 0);
  rc = rc ? rc : run_tile<TM_MIX, 32, 1, 4, 768>(768, blocks, iters, out, stamps, res + 2);
  rc = rc ? rc : run_tile<TM_MIX, 32, 1, 3, 768>(768, blocks, iters, out, stamps, res + 4);
  rc = rc ? rc : run_tile<TM_MIX, 32, 1, 3, 1024>(1024, blocks, iters, out, stamps, res + 6);
  rc = rc ? rc : run_tile<TM_MIX, 32, 1, 2, 1024>(1024, blocks, iters, out, stamps, res + 8);
  (void)hipFree(out);
  (void)hipFree(stamps);
  return rc;
}

// Operand placement at two waves per SIMD (512 threads), configurations in
// order: MFMAs only / MFMAs + epilogue with everything in VGPRs; the same
// with both multiplicands in AGPRs (inline-asm MFMAs, accumulators in
// VGPRs); epilogue only / MFMAs + epilogue with the accumulators in AGPRs.
// res[2 * i + {0, 1}] = cycles per iteration of the slowest wave, clock GHz.
int waits_ubench_operands(int blocks, int iters, double* res) {
  if (iters < 2 || iters % 2) return 1;
  float* out = nullptr;
  long long* stamps = nullptr;
  if (hipMalloc(&out, sizeof(float) * blocks * 512) != hipSuccess) return 4;
  if (hipMalloc(&stamps, sizeof(long long) * 2 * blocks * 8) != hipSuccess) return 4;
  int rc = 0;
  rc = rc ? rc : run_operands<TM_MFMA, OP_VGPR>(blocks, iters, out, stamps, res + 0);
  rc = rc ? rc : run_operands<TM_MIX, OP_VGPR>(blocks, iters, out, stamps, res + 2);
  rc = rc ? rc : run_operands<TM_MFMA, OP_AGPR_AB>(blocks, iters, out, stamps, res + 4);
  rc = rc ? rc : run_operands<TM_MIX, OP_AGPR_AB>(blocks, iters, out, stamps, res + 6);
  rc = rc ? rc : run_operands<TM_EPI, OP_AGPR_ACC>(blocks, iters, out, stamps, res + 8);
  rc = rc ? rc : run_operands<TM_MIX, OP_AGPR_ACC>(blocks, iters, out, stamps, res + 10);
  (void)hipFree(out);
  (void)hipFree(stamps);
  return rc;
}

}  // extern "C"
