// Both QK^T passes for bf16 heads of 257..448 packed rows, on 16x16x32 MFMA
// tiles (v_mfma_f32_16x16x32_bf16).  Same work, same data movement and same
// results as few_rows_kernel, but rows go to waves in 16-row tiles, so a head
// pads to a multiple of 16 rows rather than to 512: at 420 rows the workgroup
// runs 27 tiles, 7/7/7/6 per SIMD, where 32-row tiles run 8 per SIMD.  A
// 16-row tile reads twice the MFMA operand registers per flop, so per row it
// costs more than a 32-row tile; past 448 rows (8 tiles on some SIMD) the
// 32-row kernel is the faster one.
//
// MFMA layout (16x16x32): lane l supplies row/column l % 16 of A/B and, in
// step s of the head-dim loop, the 8 elements of 16-byte chunk KS*(l/16) + s
// of that row (the same chunk in A and B, so the steps add up to the full
// dot product); the output lane l holds column l % 16 and rows 4 (l/16) + i.
//
// Work item, staging and stage loop follow few_rows_kernel: 8 waves, wave w
// owns the 16-row tiles w + 8 t (t < NT); K moves HBM -> registers (a ring of
// FR_RING stages of buffer loads) -> LDS (double buffer, one barrier per
// 128-key stage) -> every wave; the MFMAs of 32-key sub-tile g issue as one
// cluster at raised wave priority, followed in the same basic block by the
// epilogue of sub-tile g - 1, with no branch between them on sub-tiles below
// every row's diagonal.  A wave holds NT or NT - 1 live tiles: two copies of
// the stage loop, chosen once per wave.
//
// Pass 1: MFMA(A = K tile, B = Q rows): a lane owns one query row and 8 keys
// of a 32-key sub-tile; lazy exponent reference as in few_rows_kernel; the
// four lane groups of a row merge their (reference, sum) at the end.
// Pass 2: MFMA(A = Q rows, B = K tile): a lane owns one key and 4 rows of each
// tile; p = exp2(dot * scale*log2 e - off[row]) summed in-lane, then over the
// four lane groups, then over the waves in a fixed order (no atomics).
#pragma once

#include "device_common.hpp"
#include "few_rows.hpp"
#include "kernel_args.hpp"

namespace waits {

template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr int FR16_SUB = 4;  // 32-key sub-tiles per stage of the 16-row-tile kernel

// LDS of the 16-row-tile workgroup (8 waves, NT tiles each).
template <int D, int NT>
struct Fr16Lds {
  static constexpr int ROWS = 8 * NT * 16;
  alignas(16) unsigned char lds[2][FR16_SUB][TileGeom<bf16_t, D>::LDS_BYTES];  // K double buffer
  alignas(16) float row_off[ROWS];
  alignas(16) int row_q[ROWS];
  alignas(16) float red[2 * FR16_SUB][8][2 * TILE];  // key k: [2k], [2k + 1]
};

// One work item (index `item` among the items of `first`) on the whole
// 512-thread workgroup, L its LDS.
template <int D, bool PASS2, int NT>
__device__ __forceinline__ void few_rows16_body(const FrArgs& args, const int32_t* first, int item,
                                                Fr16Lds<D, NT>& L) {
  using T = bf16_t;
  using Geo = TileGeom<T, D>;
  constexpr int FR_WAVES = 8;
  constexpr int FR_THREADS = FR_WAVES * WAVE;
  constexpr int T16 = 16;
  constexpr int ROWS = FR_WAVES * NT * T16;
  static_assert(ROWS <= FR_ROWS, "at most FR_ROWS rows per workgroup");
  constexpr int KS = D / 32;                                 // MFMA steps per 16x16 tile
  constexpr int CPR = Geo::ROW_BYTES / 16;                   // 16-byte chunks per K row
  constexpr int FR_SUB = FR16_SUB;
  constexpr int FR_STAGE = FR_SUB * TILE;
  constexpr int CHUNKS = FR_STAGE * CPR;
  constexpr int SV = (CHUNKS + FR_THREADS - 1) / FR_THREADS;
  static_assert(FR_RING % 2 == 0, "LDS buffer parity follows the unrolled stage index");
  auto& lds = L.lds;
  auto& row_off = L.row_off;
  auto& row_q = L.row_q;
  auto& red = L.red;

  const SeqTable& tab = args.tab;
  const int p = find_seq(first, tab.nb, item);
  const int local = item - first[p];
  const int hkv = args.hkv, G = args.G;
  const int h = local % hkv;
  const int chunk = local / hkv;  // one row block: the whole head
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const int64_t tok0 = tab.tok0[p];
  const int nc = tab.nc[p];
  const int kbeg = chunk * tab.kc[p];
  const int kend = min(kbeg + tab.kc[p], N);
  const int nsub = (kend - kbeg + TILE - 1) / TILE;
  const int nst = (nsub + FR_SUB - 1) / FR_SUB;

  const int tid = threadIdx.x;
  if (kbeg >= kend) {  // no keys (the host plans none such): empty pass-1 partials
    if constexpr (!PASS2) {
      for (int r = tid; r < PR && nc > 1; r += FR_THREADS)
        args.part[tab.ws0[p] + ((int64_t)h * tab.prow[p] + r) * nc + chunk] = make_float2(-INFINITY, 0.f);
    }
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, g4 = lane >> 4;
  const unsigned char* qb = static_cast<const unsigned char*>(args.q);
  const unsigned char* kb = static_cast<const unsigned char*>(args.k);
  const float cl2 = args.scale_log2;

  for (int r = tid; r < ROWS; r += FR_THREADS) {
    int q = -1;
    float off = INFINITY;
    if (r < PR) {
      const int j = r / G;
      q = q0 + j;
      if constexpr (PASS2) {
        const int g = h * G + (r - j * G);
        const float lse = args.lse[(int64_t)g * args.T + tok0 + q];
        const float e = expf(-tab.a[p] * ((float)q - tab.c[p]));  // w = 1 / (1 + e)
        off = fmaf(lse, LOG2E, log2f(1.f + e));
      }
    }
    row_q[r] = q;
    if constexpr (PASS2) row_off[r] = off;
  }

  // live tiles of this wave (NT or NT - 1: the host picks NT so)
  const int ntv = min(NT, max(0, (PR / T16 + (PR % T16 != 0) - wave + FR_WAVES - 1) / FR_WAVES));

  // Stationary Q fragments: this lane's row of tile t, chunks KS*g4 .. + KS.
  u32x4 qf[NT][KS];
  int tlo[NT], thi[NT], qrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int r0 = (wave + t * FR_WAVES) * T16;
    tlo[t] = q0 + min(r0, PR - 1) / G;
    thi[t] = q0 + (min(r0 + T16, PR) - 1) / G;
    const int r = r0 + c16;
    const bool ok = r < PR;
    const int rc = ok ? r : PR - 1;
    const int j = rc / G;
    const int g = h * G + (rc - j * G);
    const int q = q0 + j;
    qrow[t] = ok ? q : -1;
    const unsigned char* src =
        qb + ((tok0 + q) * args.st.q_tok + (int64_t)g * args.st.q_head) * Geo::ELT + g4 * KS * 16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 x = ld16(src + 16 * s);
      qf[t][s] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // K staging: as few_rows_kernel (buffer loads from the chunk's first key).
  const int row_bytes = (int)(args.st.kv_tok * Geo::ELT);
  const unsigned char* kseq =
      kb + ((tok0 + kbeg) * args.st.kv_tok + (int64_t)h * args.st.kv_head) * Geo::ELT;
  const int krange = (int)min((int64_t)(N - kbeg) * row_bytes, (int64_t)0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kseq), 0, krange, BUFFER_RSRC_WORD3);
  int voff[SV];
#pragma unroll
  for (int i = 0; i < SV; ++i) {
    const int cid = min(tid + i * FR_THREADS, CHUNKS - 1);
    voff[i] = (cid / CPR) * row_bytes + (cid % CPR) * 16;
  }
  u32x4 ring[FR_RING][SV];
  auto issue = [&](int stage, u32x4* dst) __attribute__((always_inline)) {
    const int sbase = min(stage, nst - 1) * FR_STAGE * row_bytes;
#pragma unroll
    for (int i = 0; i < SV; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff[i] + sbase, 0, 0));
  };
  auto commit = [&](int buf, const u32x4* src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int cid = tid + i * FR_THREADS;
      if (cid < CHUNKS) {
        const int row = cid / CPR;
        st16(lds[buf][row / TILE] + (row % TILE) * Geo::LDS_STRIDE + (cid % CPR) * 16, src[i]);
      }
    }
  };

  float mref[NT], lsum[NT];
  float off[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    mref[t] = -INFINITY;
    lsum[t] = 0.f;
  }

  // acc[parity][tile][key tile]: the 16x16 outputs of one 32-key sub-tile
  f32x4 acc[2][NT][2];
  u32x4 kf[2][KS];  // [key tile][step]

  auto read_k = [&](int buf, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const unsigned char* krow = lds[buf][u] + (kt * T16 + c16) * Geo::LDS_STRIDE + g4 * KS * 16;
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[kt][s] = ld16(krow + 16 * s);
    }
  };

  // MFMAs of the NTV live tiles into acc[par]
  auto mma = [&](int par, auto ntv_c) __attribute__((always_inline)) {
    constexpr int NTV = decltype(ntv_c)::value;
#pragma unroll
    for (int t = 0; t < NTV; ++t) {
      acc[par][t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[par][t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < NTV; ++t)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kv = __builtin_bit_cast(bf16x8, kf[kt][s]);
          const bf16x8 qv = __builtin_bit_cast(bf16x8, qf[t][s]);
          if constexpr (PASS2)
            acc[par][t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qv, kv, acc[par][t][kt], 0, 0, 0);
          else
            acc[par][t][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv, acc[par][t][kt], 0, 0, 0);
        }
  };

  // pass-1 helpers over the 8 logits of tile t (key tile kt, key 4 g4 + i)
  auto p1_logits = [&](int par, int t, bool diag, int ktj, float* x) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = acc[par][t][kt][i];
        x[4 * kt + i] = (diag && ktj + kt * T16 + 4 * g4 + i > qrow[t]) ? -INFINITY : a;
      }
  };
  auto p1_rescale = [&](int t, const float* x) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 8; ++v) mx = fmaxf(mx, x[v]);
    if (mx != -INFINITY) {
      const float mnew = fmaxf(mref[t], mx * cl2);
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) s += fast_exp2(fmaf(x[v], cl2, -mnew));
      const float alpha = (mref[t] == -INFINITY) ? 0.f : fast_exp2(mref[t] - mnew);
      lsum[t] = lsum[t] * alpha + s;
      mref[t] = mnew;
    }
  };

  // Pass-1 sums: tiles with ln[t] < 2^64 take them, the others (the sum would
  // pass 2^64, is NaN, or the lane has no reference yet) move their reference.
  // Checked once per sub-tile after every tile's exponentials, so those share
  // one basic block with the next sub-tile's MFMAs.
  auto p1_commit = [&](int par, const float* ln, const bool* live, bool diag, int ktj,
                       auto ntv_c) __attribute__((always_inline)) {
    constexpr int NTV = decltype(ntv_c)::value;
    bool ok = true;
#pragma unroll
    for (int t = 0; t < NTV; ++t) ok = ok && (!live[t] || ln[t] < 0x1p64f);
    // wave-uniform: the compiler keeps the rare path's set-up out of the hot block
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) == 0, 1)) {
#pragma unroll
      for (int t = 0; t < NTV; ++t)
        if (live[t]) lsum[t] = ln[t];
    } else {
#pragma unroll
      for (int t = 0; t < NTV; ++t) {
        if (!live[t]) continue;
        if (ln[t] < 0x1p64f) {
          lsum[t] = ln[t];
        } else {
          float x[8];
          p1_logits(par, t, diag, ktj, x);
          p1_rescale(t, x);
        }
      }
    }
  };

  // Epilogue of a sub-tile below the causal diagonal of every row (no masks,
  // no branches before the sums); csum[kt]: pass-2 key sums of this lane.
  auto epi_clean = [&](int par, auto ntv_c, float* csum) __attribute__((always_inline)) {
    constexpr int NTV = decltype(ntv_c)::value;
    float ln[NTV];
    bool live[NTV];
#pragma unroll
    for (int t = 0; t < NTV; ++t) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (PASS2) pv[i] = fast_exp2(fmaf(acc[par][t][kt][i], cl2, -off[t][i]));
          else pv[i] = fast_exp2(fmaf(acc[par][t][kt][i], cl2, -mref[t]));
        }
        const float sv = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if constexpr (PASS2) {
          csum[kt] += sv;
        } else {
          ln[t] = (kt == 0 ? lsum[t] : ln[t]) + sv;
        }
      }
      live[t] = true;
    }
    if constexpr (!PASS2) p1_commit(par, ln, live, false, 0, ntv_c);
  };

  // Epilogue of any other sub-tile j: chunk padding (skipped), sub-tiles no
  // row of a tile can see (skipped), sub-tiles crossing the diagonal (masked).
  auto epi_general = [&](int par, int j, auto ntv_c, float* csum) __attribute__((always_inline)) {
    constexpr int NTV = decltype(ntv_c)::value;
    if (j < 0 || j >= nsub) return;
    const int ktj = kbeg + j * TILE;
    float ln[NTV];
    bool live[NTV];
    bool diag_any = false;
#pragma unroll
    for (int t = 0; t < NTV; ++t) {
      live[t] = ktj <= thi[t];
      ln[t] = lsum[t];
      if (!live[t]) continue;
      const bool diag = ktj + TILE - 1 > tlo[t];
      diag_any = diag_any || diag;
      if constexpr (PASS2) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(fmaf(acc[par][t][kt][i], cl2, -off[t][i]));
          if (diag) {
            const int4 qv = *reinterpret_cast<const int4*>(&row_q[(wave + t * FR_WAVES) * T16 + 4 * g4]);
            const int qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (ktj + kt * T16 + c16 > qq[i]) pv[i] = 0.f;
          }
          csum[kt] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
        }
      } else {
        float x[8];
        p1_logits(par, t, diag, ktj, x);
        float sv = 0.f;
#pragma unroll
        for (int v = 0; v < 8; ++v) sv += fast_exp2(fmaf(x[v], cl2, -mref[t]));
        ln[t] = lsum[t] + sv;
      }
    }
    // masking a tile that does not cross the diagonal changes nothing, so
    // the rare path may mask every tile when any one crosses it
    if constexpr (!PASS2) p1_commit(par, ln, live, diag_any, ktj, ntv_c);
  };

  // pass 2: key sums of sub-tile j -> LDS slot (fixed-order cross-wave sum in flush).
  // One v_permlane16_swap of the two key tiles' sums (odd 16-lane rows of the
  // first with even rows of the second) leaves lane group g4 with key tile
  // g4 & 1's sum over lane groups 2 (g4 >> 1) and 2 (g4 >> 1) + 1; every lane
  // stores it as half g4 >> 1 of its key, and the flush adds the two halves.
  auto red_store = [&](int j, const float* csum) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(csum[0]), __float_as_uint(csum[1]), false,
                                                    false);
    const float hs = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    red[j & (2 * FR_SUB - 1)][wave][2 * ((g4 & 1) * T16 + c16) + (g4 >> 1)] = hs;
  };
  // Run by the last wave: waves with higher indices hold no more tiles than
  // lower ones, so the last SIMD (waves 3 and 7) carries the fewest tiles.
  auto flush = [&](int j) __attribute__((always_inline)) {
    const int ft = tid - (FR_THREADS - WAVE);  // lane of the last wave
    if (j >= 0 && j < nsub && ft >= 0 && ft < TILE) {
      const int key = kbeg + j * TILE + ft;
      float sc = 0.f;
#pragma unroll
      for (int w = 0; w < FR_WAVES; ++w) {
        const float2 hv = *reinterpret_cast<const float2*>(&red[j & (2 * FR_SUB - 1)][w][2 * ft]);
        sc += hv.x + hv.y;
      }
      if (key < kend) args.scores[(int64_t)h * args.T + tok0 + key] = sc;
    }
  };

  // Sub-tile g of LDS stage buffer buf, slot u (parity par = u & 1, a
  // constant): the MFMAs into acc[par] issue as one cluster at raised wave
  // priority, then the epilogue of sub-tile g - 1 from acc[par ^ 1] at normal
  // priority (s_setprio also keeps the compiler from interleaving the two:
  // the matrix core and the exponential epilogue overlap only partly inside a
  // wave, and this order measured 3-4% faster than the interleaved one).
  // csum starts at -0, so the first add of a key's sum folds away (x + -0 is
  // x for every x; the flush's sums start at +0).
  auto subtile = [&](int buf, int u, int g, auto par_c, auto ntv_c) __attribute__((always_inline)) {
    constexpr int par = decltype(par_c)::value;
    const int j = g - 1;
    const bool clean = j >= 0 && j < nsub && kbeg + j * TILE + TILE - 1 <= q0;
    float csum[2] = {-0.f, -0.f};
    if (clean) {
      read_k(buf, u);
      __builtin_amdgcn_s_setprio(1);
      mma(par, ntv_c);
      __builtin_amdgcn_s_setprio(0);
      epi_clean(par ^ 1, ntv_c, csum);
    } else {
      read_k(buf, u);
      __builtin_amdgcn_s_setprio(1);
      mma(par, ntv_c);
      __builtin_amdgcn_s_setprio(0);
      epi_general(par ^ 1, j, ntv_c, csum);
    }
    if constexpr (PASS2) {
      if (j >= 0) red_store(j, csum);
    }
  };

  vm_wait_all();
#pragma unroll
  for (int s = 0; s < FR_RING; ++s) issue(s, ring[s]);
  __syncthreads();  // row table visible
  if constexpr (PASS2) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&row_off[(wave + t * FR_WAVES) * T16 + 4 * g4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) off[t][i] = ov[i];
    }
  }

  // The stage loop, for this wave's live tile count (a wave-uniform branch
  // taken once; both paths meet the same barriers).
  const int nst_pad = (nst + FR_RING - 1) / FR_RING * FR_RING;
  auto stages = [&](auto ntv_c) __attribute__((always_inline)) {
    commit(0, ring[0]);
    issue(FR_RING, ring[0]);
    __syncthreads();
#pragma unroll
    for (int u2 = 0; u2 < FR_SUB; u2 += 2) {  // stage 0
      subtile(0, u2, u2, IntC<0>{}, ntv_c);
      subtile(0, u2 + 1, u2 + 1, IntC<1>{}, ntv_c);
    }
    commit(1, ring[1]);
    issue(FR_RING + 1, ring[1]);
    __syncthreads();
    for (int st0 = 1; st0 < 1 + nst_pad; st0 += FR_RING) {
#pragma unroll
      for (int s = 0; s < FR_RING; ++s) {
        const int st = st0 + s;
        const int buf = (1 + s) & 1;  // == st & 1
        if constexpr (PASS2) {
#pragma unroll
          for (int u = 0; u < FR_SUB; ++u) flush(st * FR_SUB + u - FR_SUB - 1);
        }
#pragma unroll
        for (int u2 = 0; u2 < FR_SUB; u2 += 2) {
          subtile(buf, u2, st * FR_SUB + u2, IntC<0>{}, ntv_c);
          subtile(buf, u2 + 1, st * FR_SUB + u2 + 1, IntC<1>{}, ntv_c);
        }
        {
          const int nxt = (2 + s) % FR_RING;  // == (st + 1) % FR_RING
          commit(buf ^ 1, ring[nxt]);
          issue(st + 1 + FR_RING, ring[nxt]);
        }
        __syncthreads();
      }
    }
  };
  if (ntv == NT) stages(IntC<NT>{});
  else stages(IntC<NT - 1>{});

  if constexpr (PASS2) {
    const int st = nst_pad;
#pragma unroll
    for (int u = 0; u < FR_SUB; ++u) flush(st * FR_SUB + u - 1);
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // merge the four lane groups holding this row: offsets 16, 32
      float m = mref[t], l = lsum[t];
#pragma unroll
      for (int o = 16; o <= 32; o *= 2) {
        const float mo = __shfl_xor(m, o, WAVE);
        const float lo = __shfl_xor(l, o, WAVE);
        const float mx = fmaxf(m, mo);
        float lt = 0.f;
        if (mx != -INFINITY)
          lt = (m == -INFINITY ? 0.f : l * fast_exp2(m - mx)) + (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mx));
        m = mx;
        l = lt;
      }
      if (g4 == 0 && t < ntv && qrow[t] >= 0) {
        const int r = (wave + t * FR_WAVES) * T16 + c16;
        const int j = r / G;
        const int g = h * G + (r - j * G);
        if (nc == 1) {
          args.lse[(int64_t)g * args.T + tok0 + qrow[t]] = (m + log2f(l)) * LN2;
        } else {
          args.part[tab.ws0[p] + ((int64_t)h * tab.prow[p] + r) * nc + chunk] = make_float2(m, l);
        }
      }
    }
  }
}

template <int D, bool PASS2, int NT>
__global__ void __launch_bounds__(512)
few_rows16_kernel(const FrArgs args) {
  __shared__ Fr16Lds<D, NT> L;
  few_rows16_body<D, PASS2, NT>(args, args.tab.first, blockIdx.x, L);
}

}  // namespace waits
