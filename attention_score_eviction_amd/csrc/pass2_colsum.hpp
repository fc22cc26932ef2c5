// Pass 2: the WAITS key scores, a weighted column sum of causal softmax
// attention (WAITS README, introduction):
//   s[h, k] = sum_{g in group h} sum_{q >= k} w[q] exp(scale <Q[g,q], K[h,k]> - lse[g,q])
//   w[q]    = 1 / (1 + exp(-a (q - (N - b - 0.5))))
// with the per-row factor folded into one exponent offset,
//   off[q] = lse[g,q] * log2 e + log2(1 + exp(-a (q - c))),
// so each element costs one fma and one v_exp_f32: p = exp2(dot * scale*log2 e - off).
// A row whose fp32 weight is 0 has off = +inf and adds exactly 0.
//
// Work item = (sequence, KV head h, block of 4 * SW * 32 keys).  The
// workgroup owns its keys for its whole life: each wave keeps SW 32-key
// tiles of K in registers as the MFMA B operand, so each lane owns one key
// column and accumulates its score in-lane; 32-row tiles of packed query rows
// (the G query heads of h interleaved) stream through double-buffered LDS as
// the A operand, from the last row down to the first row that can see the
// block.  Every key is owned by exactly one workgroup, so the scores need no
// atomics and are bitwise reproducible.  Row tiles are visited last-first so
// that workgroups of one head running side by side read the same Q rows at
// the same time (L2 reuse); consecutive work items cycle through the KV
// heads, so with 8 KV heads each head's rows stay in one XCD's L2.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

template <typename T, int D, int SW>
__global__ void __launch_bounds__(NTHREADS)
colsum_kernel(const ColsumArgs args) {
  using Geo = TileGeom<T, D>;
  constexpr int WGKEYS = NWAVES * SW * TILE;
  constexpr int HALF = Geo::ROW_BYTES / 2;
  constexpr int FLUSH = 32;  // row tiles per partial sum (two-level accumulation)
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][Geo::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float offs[2][TILE];
  __shared__ __attribute__((aligned(16))) int qrows[2][TILE];

  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int hkv = args.hkv, G = args.G;
  const int h = local % hkv;
  const int kblk = local / hkv;
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const int64_t tok0 = tab.tok0[p];
  const float a = tab.a[p], c = tab.c[p];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const unsigned char* qb = static_cast<const unsigned char*>(args.q);
  const unsigned char* kb = static_cast<const unsigned char*>(args.k);

  const int key_wg0 = kblk * WGKEYS;
  const int key_w0 = key_wg0 + wave * SW * TILE;

  // Stationary operand: this lane's key of each of the wave's key tiles.
  u32x4 kf[SW][Geo::NV];
  int key[SW];
#pragma unroll
  for (int t = 0; t < SW; ++t) {
    key[t] = key_w0 + t * TILE + col;
    const bool ok = key[t] < N;
    const unsigned char* src =
        kb + ((tok0 + (ok ? key[t] : 0)) * args.st.kv_tok + (int64_t)h * args.st.kv_head) * Geo::ELT +
        hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v)
      kf[t][v] = ok ? ld16(src + 16 * v) : u32x4{0u, 0u, 0u, 0u};
  }

  const int r_first = max(0, key_wg0 - q0) * G;  // first packed row that sees the block
  const int rt_first = r_first / TILE;
  const int RT = (PR + TILE - 1) / TILE;
  const int ntiles = RT - rt_first;
  const float cl2 = args.scale_log2;

  // Staging role: 8 threads per Q row, ROW_BYTES / 8 bytes each; threads
  // 0..31 also stage the row's exponent offset and position.
  const int srow = tid >> 3, spart = tid & 7;
  u32x4 sv[Geo::STAGE_V];
  float s_off = INFINITY;
  int s_q = -1;
  auto load_tile = [&](int rt) {
    const int r = rt * TILE + srow;
    const bool ok = r < PR;
    const int j = r / G;
    const int g = h * G + (r - j * G);
    const int q = q0 + j;
    const unsigned char* src =
        qb + ((tok0 + (ok ? q : 0)) * args.st.q_tok + (int64_t)g * args.st.q_head) * Geo::ELT +
        spart * (Geo::ROW_BYTES / 8);
#pragma unroll
    for (int i = 0; i < Geo::STAGE_V; ++i)
      sv[i] = ok ? ld16(src + 16 * i) : u32x4{0u, 0u, 0u, 0u};
    if (tid < TILE) {
      const int r2 = rt * TILE + tid;
      s_off = INFINITY;
      s_q = -1;
      if (r2 < PR) {
        const int j2 = r2 / G;
        const int g2 = h * G + (r2 - j2 * G);
        const int q2 = q0 + j2;
        const float lse = args.lse[(int64_t)g2 * args.T + tok0 + q2];
        const float e = expf(-a * ((float)q2 - c));  // w = 1 / (1 + e)
        s_off = fmaf(lse, LOG2E, log2f(1.f + e));
        s_q = q2;
      }
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* dst = lds[buf] + srow * Geo::LDS_STRIDE + spart * (Geo::ROW_BYTES / 8);
#pragma unroll
    for (int i = 0; i < Geo::STAGE_V; ++i) st16(dst + 16 * i, sv[i]);
    if (tid < TILE) {
      offs[buf][tid] = s_off;
      qrows[buf][tid] = s_q;
    }
  };

  float part[SW], total[SW];
#pragma unroll
  for (int t = 0; t < SW; ++t) {
    part[t] = 0.f;
    total[t] = 0.f;
  }

  load_tile(RT - 1);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int rt = RT - 1 - it;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(rt - 1);
    const int buf = it & 1;
    const int rq_lo = q0 + (rt * TILE) / G;
    const int rq_hi = q0 + (min(rt * TILE + TILE, PR) - 1) / G;

    const unsigned char* arow = lds[buf] + col * Geo::LDS_STRIDE + hf * HALF;
    u32x4 af[Geo::NV];
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) af[v] = ld16(arow + 16 * v);
    float o[16];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&offs[buf][8 * jj + 4 * hf]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * jj + e] = ov[e];
    }

#pragma unroll
    for (int t = 0; t < SW; ++t) {
      const int kt_lo = key_w0 + t * TILE;
      if (kt_lo >= N || kt_lo > rq_hi) continue;  // wave-uniform: no key visible
      f32x16 acc = {};
      mma_tile<T, D>(acc, af, kf[t]);
      float s = 0.f;
      if (kt_lo + TILE - 1 > rq_lo) {  // tile crosses the causal diagonal
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int4 qv = *reinterpret_cast<const int4*>(&qrows[buf][8 * jj + 4 * hf]);
          const int qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * jj + e;
            const float pv = fast_exp2(fmaf(acc[v], cl2, -o[v]));
            s += (key[t] <= qq[e]) ? pv : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) s += fast_exp2(fmaf(acc[v], cl2, -o[v]));
      }
      part[t] += s;
    }
    if ((it % FLUSH) == FLUSH - 1) {
#pragma unroll
      for (int t = 0; t < SW; ++t) {
        total[t] += part[t];
        part[t] = 0.f;
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < SW; ++t) {
    float sc = total[t] + part[t];
    sc += wave_xor32(sc);
    if (hf == 0 && key[t] < N) args.scores[(int64_t)h * args.T + tok0 + key[t]] = sc;
  }
}

}  // namespace waits
