// Pass 1: the softmax normaliser (log-sum-exp) of every processed query row.
//
// WAITS weights the causal softmax attention of each query row (WAITS README,
// introduction); the normaliser of row q of query head g is
//   lse[g, q] = ln sum_{k <= q} exp(scale * <Q[g, q], K[g / G, k]>).
//
// Work item = (sequence, KV head h, row group, key chunk).  The G query heads
// of h are packed into one row space, packed row r = G * (q - q0) + (g - hG),
// so every MFMA tile shares the K operand across the group.  A workgroup
// (4 waves) keeps SW tiles of 32 packed query rows per wave in registers as
// the MFMA B operand, streams 32-key tiles of K through double-buffered LDS
// as the A operand, and keeps a running max / sum per (lane, row) -- each
// lane owns one query row and 16 keys of every tile, so the running state is
// in-lane; the two lane halves merge once at the end.  Exponentials are
// exp2 of (dot * scale*log2 e - running max * scale*log2 e), one fma + one
// v_exp_f32 per element.
//
// When a batch has few live rows (large a), rows alone cannot fill 256
// compute units, so the key range is split into chunks; each chunk writes a
// partial (max, sum) pair per row and lse_combine_kernel merges them.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

template <typename T, int D, int SW>
__global__ void __launch_bounds__(NTHREADS)
lse_kernel(const LseArgs args) {
  using Geo = TileGeom<T, D>;
  constexpr int WGROWS = NWAVES * SW * TILE;
  constexpr int HALF = Geo::ROW_BYTES / 2;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][Geo::LDS_BYTES];

  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int hkv = args.hkv, G = args.G;
  const int h = local % hkv;
  const int rest = local / hkv;
  const int nc = tab.nc[p];
  const int rg = tab.rg[p] - 1 - rest / nc;  // larger row groups first
  const int chunk = rest - (rest / nc) * nc;
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const int64_t tok0 = tab.tok0[p];

  const int row_wg0 = rg * WGROWS;
  const int qmax_wg = q0 + (min(row_wg0 + WGROWS, PR) - 1) / G;
  const int kbeg = chunk * tab.kc[p];
  const int kend = min(kbeg + tab.kc[p], qmax_wg + 1);
  if (kbeg >= kend) return;  // no row of this group reaches this chunk

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const unsigned char* qb = static_cast<const unsigned char*>(args.q);
  const unsigned char* kb = static_cast<const unsigned char*>(args.k);
  const int row_w0 = row_wg0 + wave * SW * TILE;

  // Stationary operand: this lane's query row of each of the wave's tiles.
  u32x4 qf[SW][Geo::NV];
  int qrow[SW];
  int tq_lo[SW], tq_hi[SW];
  bool tvalid[SW];
#pragma unroll
  for (int t = 0; t < SW; ++t) {
    const int r0 = row_w0 + t * TILE;
    tvalid[t] = r0 < PR;
    tq_lo[t] = q0 + r0 / G;
    tq_hi[t] = q0 + (min(r0 + TILE, PR) - 1) / G;
    const int r = r0 + col;
    const bool ok = r < PR;
    const int j = r / G;
    const int g = h * G + (r - j * G);
    const int q = q0 + j;
    qrow[t] = ok ? q : -1;
    const unsigned char* src =
        qb + ((tok0 + (ok ? q : 0)) * args.st.q_tok + (int64_t)g * args.st.q_head) * Geo::ELT + hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v)
      qf[t][v] = ok ? ld16(src + 16 * v) : u32x4{0u, 0u, 0u, 0u};
  }

  float m[SW], l[SW];
#pragma unroll
  for (int t = 0; t < SW; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
  }
  const float cl2 = args.scale_log2;
  const int ntiles = (kend - kbeg + TILE - 1) / TILE;

  // Staging role: 8 threads per K row, ROW_BYTES / 8 bytes each.
  const int srow = tid >> 3, spart = tid & 7;
  u32x4 sv[Geo::STAGE_V];
  auto load_tile = [&](int kt0) {
    const int key = kt0 + srow;
    const bool ok = key < kend;
    const unsigned char* src =
        kb + ((tok0 + (ok ? key : 0)) * args.st.kv_tok + (int64_t)h * args.st.kv_head) * Geo::ELT +
        spart * (Geo::ROW_BYTES / 8);
#pragma unroll
    for (int i = 0; i < Geo::STAGE_V; ++i)
      sv[i] = ok ? ld16(src + 16 * i) : u32x4{0u, 0u, 0u, 0u};
  };
  auto store_tile = [&](int buf) {
    unsigned char* dst = lds[buf] + srow * Geo::LDS_STRIDE + spart * (Geo::ROW_BYTES / 8);
#pragma unroll
    for (int i = 0; i < Geo::STAGE_V; ++i) st16(dst + 16 * i, sv[i]);
  };

  load_tile(kbeg);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int kt0 = kbeg + it * TILE;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(kt0 + TILE);

    const unsigned char* arow = lds[it & 1] + col * Geo::LDS_STRIDE + hf * HALF;
    u32x4 af[Geo::NV];
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) af[v] = ld16(arow + 16 * v);

#pragma unroll
    for (int t = 0; t < SW; ++t) {
      if (!tvalid[t] || kt0 > tq_hi[t]) continue;  // wave-uniform
      f32x16 acc = {};
      mma_tile<T, D>(acc, af, qf[t]);
      float x[16];
      float mt = -INFINITY;
      if (kt0 + TILE - 1 > tq_lo[t]) {  // tile crosses the causal diagonal
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kt0 + out_row(v, hf);
          x[v] = key <= qrow[t] ? acc[v] : -INFINITY;
          mt = fmaxf(mt, x[v]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          x[v] = acc[v];
          mt = fmaxf(mt, x[v]);
        }
      }
      const float mn = fmaxf(m[t], mt);
      const float alpha = (mn == m[t]) ? 1.f : fast_exp2((m[t] - mn) * cl2);
      const float off = (mn == -INFINITY) ? 0.f : mn * cl2;
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) s += fast_exp2(fmaf(x[v], cl2, -off));
      l[t] = l[t] * alpha + s;
      m[t] = mn;
    }

    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }

  const int rgrows = tab.prow[p];  // = row groups * WGROWS
#pragma unroll
  for (int t = 0; t < SW; ++t) {
    const float mo = wave_xor32(m[t]);
    const float lo = wave_xor32(l[t]);
    const float mx = fmaxf(m[t], mo);
    float lt = 0.f;
    if (mx != -INFINITY)
      lt = l[t] * fast_exp2((m[t] - mx) * cl2) + lo * fast_exp2((mo - mx) * cl2);
    if (hf == 0 && qrow[t] >= 0) {
      const int r = row_w0 + t * TILE + col;
      const int j = r / G;
      const int g = h * G + (r - j * G);
      if (nc == 1) {
        args.lse[(int64_t)g * args.T + tok0 + qrow[t]] = fmaf(mx, args.scale, logf(lt));
      } else {
        args.part[tab.ws0[p] + ((int64_t)h * rgrows + r) * nc + chunk] =
            make_float2(mx * cl2, lt);
      }
    }
  }
}

// Merge the per-chunk (max * scale*log2 e, sum) pairs of each row into lse.
// A team of lanes per (KV head, packed row); a row reads the chunks that
// start at or before its own position (later chunks hold no key of its
// causal range).
__global__ void __launch_bounds__(256)
lse_combine_kernel(const CombineArgs args) {
  // Sequence p's rows take args.team[p] lanes each (a power of two dividing
  // 64, sized to its chunk count): each lane takes every team-th chunk, then
  // the team reduces.  Every sequence's threads start on a wave boundary, so
  // the team size is uniform within a wave.
  const SeqTable& tab = args.tab;
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const bool in_range = gid < tab.first[tab.nb];
  const int p = find_seq(tab.first, tab.nb, in_range ? gid : 0);
  const int team = args.team[p];
  const int loc = gid - tab.first[p];
  const int local = loc / team;  // (KV head, packed row) of the sequence
  const int tl = loc - local * team;
  const int G = args.G;
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const bool live = in_range && local < args.hkv * PR;  // the wave padding holds no row
  const int h = live ? local / PR : 0;
  const int r = live ? local - h * PR : 0;
  const int j = r / G;
  const int g = h * G + (r - j * G);
  const int q = q0 + j;
  const int nc = tab.nc[p];
  const int last = tab.kc[p] > 0 ? q / tab.kc[p] : nc - 1;  // kc 0: every chunk wrote every row
  const float2* pp = args.part + tab.ws0[p] + ((int64_t)h * tab.prow[p] + r) * nc;
  float mx = -INFINITY;
  if (live)
    for (int c = tl; c <= last; c += team) mx = fmaxf(mx, pp[c].x);
  for (int o = team / 2; o > 0; o /= 2) mx = fmaxf(mx, __shfl_xor(mx, o, WAVE));
  float lt = 0.f;
  if (live && mx != -INFINITY)
    for (int c = tl; c <= last; c += team) lt += pp[c].y * exp2f(pp[c].x - mx);
  for (int o = team / 2; o > 0; o /= 2) lt += __shfl_xor(lt, o, WAVE);
  if (live && tl == 0) args.lse[(int64_t)g * args.T + tab.tok0[p] + q] = (mx + log2f(lt)) * LN2;
}

}  // namespace waits
