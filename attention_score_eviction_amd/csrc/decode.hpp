// Decode attention over a compacted KV cache: one new query per query head
// attends over the kept rows of its KV head (WAITS README "Quickstart":
// generation after init_cache runs on the kept key-value pairs).
//
//   out[i, g, :] = sum_{j < len[i]} softmax_j(scale <q[i, g], K[i, h, j]>) V[i, h, j]
//   lse[i, g]    = ln sum_{j < len[i]} exp(scale <q[i, g], K[i, h, j]>),  h = g / G
//
// Work item = (sequence, KV head, key split, chunk of GC query heads of the
// group); the group's query heads share every K/V row the item reads, so a
// row leaves HBM once per item.  Four waves:
//   A. scores: 16-key tiles on 16x16 MFMAs (A = K rows read straight from
//      HBM, B = the GC query vectors, held in registers), into an LDS table
//      sc[key][query] in log2 units;
//   B. per query head: max over the split's keys, p = exp2(s - max) in
//      place, and their sum (fp32);
//   C. o[g] += p[g][j] * V[j] on the VALU in fp32 (p never leaves fp32):
//      lanes cover a row in 16-byte chunks, so each load instruction reads
//      whole rows; DEC_VU rows in flight per lane; then a sum over the lanes
//      of one chunk and over the waves.
// Phases A and C keep several tiles / rows of loads in flight per wave so
// that HBM latency is covered within each work item.
// One split writes out / lse directly; several write (max, sum, o) partials
// that decode_combine_kernel merges.  Work is HBM-bound: K and V rows are
// read once, everything else is small.
#pragma once

#include "device_common.hpp"

namespace waits {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / WAVE;
constexpr int DEC_MAX_KS = 1024;     // keys per work item (LDS score table)
constexpr int DEC_MAX_SPLITS = 1024; // splits per (sequence, query head)
constexpr int DEC_TU = 4;            // score tiles per wave with loads in flight together
constexpr int DEC_VU = 8;            // V rows per lane with loads in flight together

struct DecodeArgs {
  const void* q;         // [B, Hq, D]
  const void* kc;        // [B, Hkv, cap, D]
  const void* vc;        // [B, Hkv, cap, D]
  const int32_t* lens;   // [B], clamped to [0, cap]
  float* out;            // [B, Hq, D]
  float* lse;            // [B, Hq] or null
  float2* part_ml;       // [B, Hq, nsplit] (max in log2 units, sum) when nsplit > 1
  float* part_o;         // [B, Hq, nsplit, D]
  int B, hq, hkv, G, D, cap, ks, nsplit, ngc;
  float scale_log2;      // scale * log2(e)
};

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, WAVE));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}

template <typename T, int D, int GC>
__global__ void __launch_bounds__(DEC_THREADS) decode_kernel(const DecodeArgs a) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int ELT = BF ? 2 : 4;
  constexpr int ROWB = D * ELT;            // bytes per cache row
  constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  constexpr int KPW = WAVE / CPR;          // rows per wave step in phase C
  constexpr int EPC = 16 / ELT;            // elements per chunk
  constexpr int NCH = CPR / 4;             // chunks per lane group in phase A
  static_assert(CPR <= WAVE && CPR % 4 == 0, "row chunks");
  static_assert(GC >= 1 && GC <= 8, "query heads per item");
  __shared__ __attribute__((aligned(16))) float sc[DEC_MAX_KS][GC];
  __shared__ float ored[DEC_WAVES][GC][D];
  __shared__ float st_m[GC], st_l[GC];

  int item = blockIdx.x;
  const int gc = item % a.ngc;
  item /= a.ngc;
  const int split = item % a.nsplit;
  item /= a.nsplit;
  const int h = item % a.hkv;
  const int b = item / a.hkv;
  const int len = min(max(a.lens[b], 0), a.cap);
  const int kbeg = split * a.ks;
  const int nk = max(0, min(kbeg + a.ks, len) - kbeg);  // keys of this item
  const int g0 = h * a.G + gc * GC;                     // its first query head
  const int gn = min(GC, a.G - gc * GC);                // query heads it owns
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t head_row = (int64_t)(b * a.hkv + h) * a.cap;
  const unsigned char* kbase = static_cast<const unsigned char*>(a.kc) + head_row * ROWB;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.vc) + head_row * ROWB;
  const unsigned char* qbase = static_cast<const unsigned char*>(a.q) + ((int64_t)b * a.hq + g0) * ROWB;

  // A. scores.  MFMA 16x16: lane l supplies key row l % 16 and query l % 16;
  // lane group l / 16 takes the 16-byte chunks 4 s + l / 16 of both (the same
  // contraction indices in A and B); the output lane holds keys 4 (l/16) + i
  // of query l % 16.
  if (nk > 0) {
    const int c16 = lane & 15, g4 = lane >> 4;
    u32x4 qf[NCH];
#pragma unroll
    for (int s = 0; s < NCH; ++s) {
      const u32x4 x = ld16(qbase + (int64_t)min(c16, gn - 1) * ROWB + (4 * s + g4) * 16);
      qf[s] = c16 < gn ? x : u32x4{0u, 0u, 0u, 0u};
    }
    // DEC_TU tiles per wave and step: their loads are all in flight before
    // the first MFMA (one tile at a time leaves HBM latency exposed)
    for (int t0 = wave; t0 * 16 < nk; t0 += DEC_WAVES * DEC_TU) {
      u32x4 kf[DEC_TU][NCH];
#pragma unroll
      for (int r = 0; r < DEC_TU; ++r) {
        const int row = min(kbeg + (t0 + r * DEC_WAVES) * 16 + c16, len - 1);  // past the item: loaded, unused
        const unsigned char* kr = kbase + (int64_t)row * ROWB;
#pragma unroll
        for (int s = 0; s < NCH; ++s) kf[r][s] = ld16(kr + (4 * s + g4) * 16);
      }
#pragma unroll
      for (int r = 0; r < DEC_TU; ++r) {
        const int t = t0 + r * DEC_WAVES;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NCH; ++s) {
          if constexpr (BF) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[r][s]),
                                                          __builtin_bit_cast(bf16x8, qf[s]), acc, 0, 0, 0);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[r][s][u]), __uint_as_float(qf[s][u]),
                                                         acc, 0, 0, 0);
          }
        }
        if (c16 < GC) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = t * 16 + 4 * g4 + i;
            if (j < nk) sc[j][c16] = acc[i] * a.scale_log2;
          }
        }
      }
    }
  }
  __syncthreads();

  // B. per query head: max, exp2 in place, sum.
  for (int g = wave; g < GC; g += DEC_WAVES) {
    float m = -INFINITY;
    for (int j = lane; j < nk; j += WAVE) m = fmaxf(m, sc[j][g]);
    m = wave_max_f(m);
    float l = 0.f;
    for (int j = lane; j < nk; j += WAVE) {
      const float p = fast_exp2(sc[j][g] - m);
      sc[j][g] = p;
      l += p;
    }
    l = wave_sum_f(l);
    if (lane == 0) {
      st_m[g] = m;
      st_l[g] = l;
    }
  }
  __syncthreads();

  // C. o[g] = sum_j p[g][j] V[j] for this lane's chunk; KPW rows per wave step.
  const int slot = lane / CPR, ch = lane % CPR;
  float o[GC][EPC];
#pragma unroll
  for (int g = 0; g < GC; ++g)
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[g][e] = 0.f;
  constexpr int STEP = DEC_WAVES * KPW;
  for (int j0 = wave * KPW + slot; j0 < nk; j0 += DEC_VU * STEP) {
    u32x4 vv[DEC_VU];
#pragma unroll
    for (int r = 0; r < DEC_VU; ++r) {
      const int j = min(j0 + r * STEP, nk - 1);  // past the item: a valid row, weight 0
      vv[r] = ld16(vbase + (int64_t)(kbeg + j) * ROWB + ch * 16);
    }
#pragma unroll
    for (int r = 0; r < DEC_VU; ++r) {
      const int j = j0 + r * STEP;
      float p[GC];
#pragma unroll
      for (int g = 0; g < GC; ++g) p[g] = j < nk ? sc[j][g] : 0.f;
      float ve[EPC];
      if constexpr (BF) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          ve[2 * w] = __uint_as_float(vv[r][w] << 16);
          ve[2 * w + 1] = __uint_as_float(vv[r][w] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) ve[w] = __uint_as_float(vv[r][w]);
      }
#pragma unroll
      for (int g = 0; g < GC; ++g)
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[g][e] = fmaf(p[g], ve[e], o[g][e]);
    }
  }
  // sum over the lanes holding the same chunk, then over the waves
#pragma unroll
  for (int off = CPR; off < WAVE; off <<= 1)
#pragma unroll
    for (int g = 0; g < GC; ++g)
#pragma unroll
      for (int e = 0; e < EPC; ++e) o[g][e] += __shfl_xor(o[g][e], off, WAVE);
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GC; ++g)
#pragma unroll
      for (int e = 0; e < EPC; ++e) ored[wave][g][ch * EPC + e] = o[g][e];
  }
  __syncthreads();

  for (int x = tid; x < GC * D; x += DEC_THREADS) {
    const int g = x / D, e = x - g * D;
    if (g >= gn) continue;
    float os = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) os += ored[w][g][e];
    const float m = st_m[g], l = st_l[g];
    const int64_t bg = (int64_t)b * a.hq + g0 + g;
    if (a.nsplit == 1) {
      a.out[bg * D + e] = l > 0.f ? os / l : 0.f;
      if (e == 0 && a.lse) a.lse[bg] = l > 0.f ? (m + log2f(l)) * LN2 : -INFINITY;
    } else {
      a.part_o[(bg * a.nsplit + split) * D + e] = os;
      if (e == 0) a.part_ml[bg * a.nsplit + split] = make_float2(m, l);
    }
  }
}

// Merge the splits of each (sequence, query head): one wave each.
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s o_s 2^(m_s - M) / L
__global__ void __launch_bounds__(DEC_THREADS) decode_combine_kernel(const DecodeArgs a) {
  __shared__ float wts[DEC_WAVES][DEC_MAX_SPLITS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t bg = (int64_t)blockIdx.x * DEC_WAVES + wave;
  if (bg >= (int64_t)a.B * a.hq) return;
  const float2* ml = a.part_ml + bg * a.nsplit;
  float M = -INFINITY;
  for (int s = lane; s < a.nsplit; s += WAVE)
    if (ml[s].y > 0.f) M = fmaxf(M, ml[s].x);
  M = wave_max_f(M);
  float L = 0.f;
  for (int s = lane; s < a.nsplit; s += WAVE) {
    const float w = ml[s].y > 0.f ? fast_exp2(ml[s].x - M) : 0.f;
    wts[wave][s] = w;
    L += ml[s].y * w;
  }
  L = wave_sum_f(L);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's LDS writes done (lgkmcnt(0))
  __builtin_amdgcn_wave_barrier();
  const float* po = a.part_o + bg * a.nsplit * a.D;
  for (int e = lane; e < a.D; e += WAVE) {
    float os = 0.f;
    for (int s = 0; s < a.nsplit; ++s) os = fmaf(po[(int64_t)s * a.D + e], wts[wave][s], os);
    a.out[bg * a.D + e] = L > 0.f ? os / L : 0.f;
  }
  if (lane == 0 && a.lse) a.lse[bg] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
}

}  // namespace waits
