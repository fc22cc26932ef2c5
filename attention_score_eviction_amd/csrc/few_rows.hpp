// Both QK^T passes for sequences whose processed rows are few: when the G
// query heads of a KV head have at most FR_ROWS packed rows in total (large
// a: only the last rows carry weight), one workgroup holds every row of the
// head in registers and streams K past them exactly once.  Heads with more
// rows run here too, one block of FR_ROWS packed rows per workgroup (the
// block's keys end at its last query): pass 1 always, pass 2 while the
// blocks' partial column sums fit the workspace limits of the host plan.
//
// Work item = (sequence, KV head h, row block, key chunk).  8 waves; wave w owns packed
// row tiles w and w + 8 (32 rows each, MFMA operand fragments in
// registers).  K moves in stages of FR_SUB 32-key sub-tiles: HBM -> registers
// (FR_RING stages of loads in flight) -> LDS (double buffer, one barrier per
// stage) -> every wave.  Each wave issues the MFMAs of sub-tile g in the same
// basic block as the exponential epilogue of sub-tile g - 1, so the matrix
// and vector pipes work side by side.
//
// Pass 1 (log-sum-exp, WAITS README introduction: the softmax normaliser of
// every weighted row).  MFMA(A = K tile, B = Q rows): each lane owns one
// query row and 16 keys per tile, so the row's running (reference, sum) pair
// is in-lane.  The exponent reference is lazy: elements cost one fma, one
// v_exp_f32 and one add against a fixed per-lane reference, and the
// reference moves (with a rescale of the sum) only when a tile overflows the
// sum past 2^64 or the lane has no reference yet -- a per-tile check instead
// of a per-element max.  Exponent arithmetic is in log2 units
// (scale * log2 e folded into the fma).
//
// Pass 2 (weighted column sums).  MFMA(A = Q rows, B = K tile): each lane
// owns one key and 16 rows per tile; p = exp2(dot * scale*log2 e - off[row])
// with off = lse * log2 e + log2(1 + exp(-a (q - c))) (w folded in, off =
// +inf for rows whose fp32 weight is 0).  In-lane sums, then each lane half
// stores its rows' sum to LDS and one wave per sub-tile (8-wave shapes: one
// per SIMD) adds the two halves of every wave in a fixed order.  A head in one block has every row here, so that
// sum is the score, written straight to the score array; a head in several
// blocks writes it as the block's partial (cpart), and rowblock_reduce_kernel
// adds the blocks in order -- no atomics, bitwise reproducible.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int FR_ROWS = 512;                          // packed rows of the largest workgroup
constexpr int FR_RING = 2;                            // stages of loads in flight

struct FrArgs {
  const void* q;
  const void* k;
  float* lse;                 // pass 1 out (single chunk) / pass 2 in: [Hq, T]
  float2* part;               // pass 1 partials when a head's keys are split
  float* scores;              // pass 2 out: [Hkv, T]
  float* cpart;               // pass 2 of heads in several row blocks: each block's column
                              // sums, [ws0 + (row block * hkv + h) * N + key] (keys the block sees)
  Strides st;
  int64_t T;
  int32_t G;
  int32_t hkv;
  float scale;
  float scale_log2;
  SeqTable tab;               // nc / kc: key chunks; first[]: items
};

// LDS of a workgroup of FR_WAVES waves, each owning FR_TW row tiles: ROWS =
// FR_WAVES * FR_TW * 32 packed rows (a head with fewer rows takes the
// smallest workgroup that holds them, so short windows do not pad to
// FR_ROWS).  Stages are SUB 32-key sub-tiles (one barrier each); smaller
// workgroups take shorter stages to keep each thread's share of the load
// ring small.
template <typename T, int D, int FR_WAVES, int FR_TW>
struct FrLds {
  static constexpr int ROWS = FR_WAVES * FR_TW * TILE;
  static constexpr int SUB = FR_WAVES >= 8 ? 4 : 2;
  alignas(16) unsigned char lds[2][SUB][TileGeom<T, D>::LDS_BYTES];  // K double buffer
  alignas(16) float row_off[ROWS];   // pass 2: exponent offsets
  alignas(16) int row_q[ROWS];       // row position (-1: padding)
  // pass 2: per-wave key sums of a sub-tile; 2 SUB slots, so one stage's
  // stores never meet the previous stage's flushes; key k: [2k], [2k + 1]
  alignas(16) float red[2 * SUB][FR_WAVES][2 * TILE];
};

// One work item on threads [0, FR_WAVES * 64) of the workgroup: `item` is
// its index among the items of `first` (first work item of each sequence),
// L the workgroup's LDS.
template <typename T, int D, bool PASS2, int FR_WAVES, int FR_TW>
__device__ __forceinline__ void few_rows_body(const FrArgs& args, const int32_t* first, int item,
                                              FrLds<T, D, FR_WAVES, FR_TW>& L) {
  constexpr int FR_THREADS = FR_WAVES * WAVE;
  constexpr int ROWS = FR_WAVES * FR_TW * TILE;
  static_assert(ROWS <= FR_ROWS, "at most FR_ROWS rows per workgroup");
  constexpr int FR_SUB = FrLds<T, D, FR_WAVES, FR_TW>::SUB;
  constexpr int FR_STAGE = FR_SUB * TILE;
  using Geo = TileGeom<T, D>;
  constexpr int HALF = Geo::ROW_BYTES / 2;
  constexpr int CPR = Geo::ROW_BYTES / 16;                    // 16-byte chunks per K row
  constexpr int CHUNKS = FR_STAGE * CPR;                       // per stage
  constexpr int SV = (CHUNKS + FR_THREADS - 1) / FR_THREADS;   // chunks per thread per stage
  static_assert(FR_SUB % 2 == 0, "accumulator parity follows the sub-tile index");
  auto& lds = L.lds;
  auto& row_off = L.row_off;
  auto& row_q = L.row_q;
  auto& red = L.red;

  const SeqTable& tab = args.tab;
  const int p = find_seq(first, tab.nb, item);
  const int local = item - first[p];
  const int hkv = args.hkv, G = args.G;
  const int h = local % hkv;
  const int rest = local / hkv;
  const int nc = tab.nc[p];
  const int rb = tab.nrb[p] - 1 - rest / nc;  // row block (larger key ranges first)
  const int chunk = rest - (rest / nc) * nc;
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const int64_t tok0 = tab.tok0[p];
  const int rbase = rb * ROWS;                // first packed row of the block
  const int qb0 = q0 + rbase / G;             // its first query
  // Keys: pass 2 of a head in one row block, the sequence's keys in chunks of
  // kc; otherwise (pass 1, and pass 2 of a head in several row blocks) the
  // keys up to the block's last query, cut into nc chunks.
  const bool blocks = tab.nrb[p] > 1;
  int kbeg, kend;
  if (PASS2 && !blocks) {
    kbeg = chunk * tab.kc[p];
    kend = min(kbeg + tab.kc[p], N);
  } else {
    const int nkeys = min(N, q0 + (min(rbase + ROWS, PR) - 1) / G + 1);
    const int kc = ((nkeys + nc - 1) / nc + TILE - 1) / TILE * TILE;
    kbeg = chunk * kc;
    kend = min(kbeg + kc, nkeys);
  }
  const int nsub = (kend - kbeg + TILE - 1) / TILE;     // 32-key sub-tiles
  const int nst = (nsub + FR_SUB - 1) / FR_SUB;          // stages

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: uniform branches
  const int lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const unsigned char* qb = static_cast<const unsigned char*>(args.q);
  const unsigned char* kb = static_cast<const unsigned char*>(args.k);
  const float cl2 = args.scale_log2;

  if (kbeg >= kend) {  // a chunk past the block's keys
    if constexpr (!PASS2) {  // its pass-1 partials are empty
      for (int r = tid; r < ROWS && rbase + r < PR; r += FR_THREADS)
        args.part[tab.ws0[p] + ((int64_t)h * tab.prow[p] + rbase + r) * nc + chunk] =
            make_float2(-INFINITY, 0.f);
    }
    return;  // pass 2: the reduce reads no key of this range for this block
  }

  // Row table (and pass-2 exponent offsets): one thread per packed row.
  for (int r = tid; r < ROWS; r += FR_THREADS) {
    int q = -1;
    float off = INFINITY;
    if (rbase + r < PR) {
      const int j = (rbase + r) / G;
      q = q0 + j;
      if constexpr (PASS2) {
        const int g = h * G + (rbase + r - j * G);
        const float lse = args.lse[(int64_t)g * args.T + tok0 + q];
        const float e = expf(-tab.a[p] * ((float)q - tab.c[p]));  // w = 1 / (1 + e)
        off = fmaf(lse, LOG2E, log2f(1.f + e));
      }
    }
    row_q[r] = q;
    if constexpr (PASS2) row_off[r] = off;
  }

  // Stationary Q fragments: row tiles wave and wave + FR_WAVES.
  u32x4 qf[FR_TW][Geo::NV];
  int tlo[FR_TW], thi[FR_TW];
  bool tval[FR_TW];
  int qrow[FR_TW];
#pragma unroll
  for (int t = 0; t < FR_TW; ++t) {
    const int r0 = rbase + (wave + t * FR_WAVES) * TILE;
    tval[t] = r0 < PR;
    tlo[t] = q0 + r0 / G;
    thi[t] = q0 + (min(r0 + TILE, PR) - 1) / G;
    const int r = r0 + col;
    const bool ok = r < PR;
    const int rc = ok ? r : PR - 1;  // loads stay unconditional (in-bounds address)
    const int j = rc / G;
    const int g = h * G + (rc - j * G);
    const int q = q0 + j;
    qrow[t] = ok ? q : -1;
    const unsigned char* src =
        qb + ((tok0 + q) * args.st.q_tok + (int64_t)g * args.st.q_head) * Geo::ELT + hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) {
      const u32x4 x = ld16(src + 16 * v);
      qf[t][v] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // K staging: ring of FR_RING stages in registers, fetched with buffer loads
  // over head h's rows from the chunk's first key to the sequence end: one
  // 32-bit offset add per load, and the hardware range check returns zeros
  // past the sequence (the host keeps a chunk's K span below 2^31 bytes).
  // Stages past the chunk re-read its last stage, so every thread issues the
  // same number of loads per stage and the compiler waits for exactly the
  // oldest stage.  Rows past the chunk but inside the sequence carry real
  // keys; they are never used: sub-tiles are 32-key aligned with the chunk
  // end, sub-tiles past it skip their epilogue, and keys past the sequence
  // are causal-masked (pass 1) or not written (pass 2).
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
  auto issue = [&](int stage, u32x4* dst) {
    const int sbase = min(stage, nst - 1) * FR_STAGE * row_bytes;
#pragma unroll
    for (int i = 0; i < SV; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, voff[i] + sbase, 0, 0));
  };
  auto commit = [&](int buf, int stage, const u32x4* src) {
    (void)stage;
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int cid = tid + i * FR_THREADS;
      if (cid < CHUNKS) {
        const int row = cid / CPR;
        st16(lds[buf][row / TILE] + (row % TILE) * Geo::LDS_STRIDE + (cid % CPR) * 16, src[i]);
      }
    }
  };

  // pass-1 state (per lane, per row tile): log2-unit reference and sum
  float mref[FR_TW], lsum[FR_TW];
  // pass-2 state: this lane's rows' offsets
  float off[FR_TW][16];
#pragma unroll
  for (int t = 0; t < FR_TW; ++t) {
    mref[t] = -INFINITY;
    lsum[t] = 0.f;
  }

  // Pass-1 logits of row tile t in sub-tile ktj (acc holds dot products):
  // on a sub-tile crossing the diagonal, keys past the lane's row are -inf.
  auto p1_logits = [&](const f32x16& a, int t, bool diag, int ktj, float* x) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      x[v] = (diag && ktj + out_row(v, hf) > qrow[t]) ? -INFINITY : a[v];
  };
  // Pass-1 reference move for row tile t: taken when the tile would carry
  // the lane's sum past 2^64, makes it NaN, or the lane has no reference yet
  // (its exponentials are then +inf or NaN); the sum is rescaled to the new
  // reference.  Rare, so it is checked once per sub-tile, after every tile's
  // exponentials: all of them then share one basic block with the next
  // sub-tile's MFMAs.
  auto p1_rescale = [&](int t, const float* x) {
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, x[v]);
    if (mx != -INFINITY) {
      const float mnew = fmaxf(mref[t], mx * cl2);
      float p2[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) p2[v] = fast_exp2(fmaf(x[v], cl2, -mnew));
      const float alpha = (mref[t] == -INFINITY) ? 0.f : fast_exp2(mref[t] - mnew);
      lsum[t] = lsum[t] * alpha + sum16(p2);
      mref[t] = mnew;
    }
  };
  // ln[t]: candidate sums; tiles with ln[t] < 2^64 take them, others move
  // their reference.  diag/ktj as for p1_logits; live[t] false: tile skipped.
  auto p1_commit = [&](const f32x16* acc, const float* ln, const bool* live, bool diag, int ktj) {
    bool ok = true;
#pragma unroll
    for (int t = 0; t < FR_TW; ++t) ok = ok && (!live[t] || ln[t] < 0x1p64f);
    // wave-uniform: the compiler keeps the rare path's set-up out of the hot block
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) == 0, 1)) {
#pragma unroll
      for (int t = 0; t < FR_TW; ++t)
        if (live[t]) lsum[t] = ln[t];
    } else {
#pragma unroll
      for (int t = 0; t < FR_TW; ++t) {
        if (!live[t]) continue;
        if (ln[t] < 0x1p64f) {
          lsum[t] = ln[t];
        } else {
          float x[16];
          p1_logits(acc[t], t, diag, ktj, x);
          p1_rescale(t, x);
        }
      }
    }
  };

  // Epilogue of a sub-tile strictly below the causal diagonal of every row of
  // this workgroup (no masks, no branches before the sums).
  auto epi_clean = [&](f32x16* acc, float& csum) {
    float ln[FR_TW];
    bool live[FR_TW];
#pragma unroll
    for (int t = 0; t < FR_TW; ++t) {
      float pv[16];
      if constexpr (PASS2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(acc[t][v], cl2, -off[t][v]));
        csum += sum16(pv);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(acc[t][v], cl2, -mref[t]));
        ln[t] = lsum[t] + sum16(pv);
        live[t] = true;
      }
    }
    if constexpr (!PASS2) p1_commit(acc, ln, live, false, 0);
  };

  // Epilogue of any other sub-tile: chunk padding (skipped), sub-tiles no row
  // of a row tile can see (skipped), sub-tiles crossing the diagonal (masked).
  auto epi_general = [&](f32x16* acc, int j, float& csum) {
    if (j < 0 || j >= nsub) return;
    const int ktj = kbeg + j * TILE;
    float ln[FR_TW];
    bool live[FR_TW];
    bool diag_any = false;
#pragma unroll
    for (int t = 0; t < FR_TW; ++t) {
      live[t] = tval[t] && ktj <= thi[t];
      ln[t] = lsum[t];
      if (!live[t]) continue;
      const bool diag = ktj + TILE - 1 > tlo[t];
      diag_any = diag_any || diag;
      float pv[16];
      if constexpr (PASS2) {
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(acc[t][v], cl2, -off[t][v]));
        if (diag) {
          const int lrow = (wave + t * FR_WAVES) * TILE;  // tile's first row in the LDS tables
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int4 qv = *reinterpret_cast<const int4*>(&row_q[lrow + 8 * jj + 4 * hf]);
            const int qq[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ktj + col > qq[e]) pv[4 * jj + e] = 0.f;
          }
        }
        csum += sum16(pv);
      } else {
        float x[16];
        p1_logits(acc[t], t, diag, ktj, x);
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(x[v], cl2, -mref[t]));
        ln[t] = lsum[t] + sum16(pv);
      }
    }
    // masking a tile that does not cross the diagonal changes nothing, so
    // the rare path may mask every tile when any one crosses it
    if constexpr (!PASS2) p1_commit(acc, ln, live, diag_any, ktj);
  };

  auto read_k = [&](int buf, int u, u32x4* kf) {
    const unsigned char* krow = lds[buf][u] + col * Geo::LDS_STRIDE + hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) kf[v] = ld16(krow + 16 * v);
  };
  auto mma_both = [&](f32x16* acc, const u32x4* kf) {
    if constexpr (FR_TW == 1) {
      acc[0] = f32x16{};
      if constexpr (PASS2) mma_tile<T, D>(acc[0], qf[0], kf);
      else mma_tile<T, D>(acc[0], kf, qf[0]);
    } else {
      static_assert(FR_TW % 2 == 0, "row tiles go in pairs");
#pragma unroll
      for (int t = 0; t < FR_TW; t += 2) {
        acc[t] = f32x16{};
        acc[t + 1] = f32x16{};
        mma_tile2<T, D, !PASS2>(acc[t], acc[t + 1], qf[t], qf[t + 1], kf);
      }
    }
  };
  // pass 2: sub-tile j's per-wave key sums -> its key scores (fixed order)
  // each lane half stores its own rows' sum; the flush adds the two halves
  auto red_store = [&](int j, float csum) { red[j & (2 * FR_SUB - 1)][wave][2 * col + hf] = csum; };
  // Flush slot u of a stage (one sub-tile).  Every wave holds the same row
  // tiles, so whichever SIMD runs a flush carries it on top of a full share:
  // with 8 waves, slots 0..3 go to waves 4..7, one per SIMD (waves w and
  // w + 4 share one), instead of all four to the last wave.  Smaller shapes
  // flush on their last wave.  Each key's sum keeps the same order.
  auto flush = [&](int j, int u) {
    constexpr bool SPREAD = FR_WAVES >= 2 * FR_SUB;
    const int fw = SPREAD ? FR_WAVES - FR_SUB + u : FR_WAVES - 1;
    const int ft = tid - fw * WAVE;  // lane of the flushing wave
    if (j >= 0 && j < nsub && ft >= 0 && ft < TILE) {
      const int key = kbeg + j * TILE + ft;
      float sc = 0.f;
#pragma unroll
      for (int w = 0; w < FR_WAVES; ++w) {
        const float2 hv = *reinterpret_cast<const float2*>(&red[j & (2 * FR_SUB - 1)][w][2 * ft]);
        sc += hv.x + hv.y;
      }
      if (key < kend) {
        if (blocks) args.cpart[tab.ws0[p] + ((int64_t)rb * hkv + h) * N + key] = sc;
        else args.scores[(int64_t)h * args.T + tok0 + key] = sc;
      }
    }
  };

  // Sub-tile g: MFMAs into acc[g & 1] in the same block as the epilogue of
  // sub-tile g - 1 from acc[(g - 1) & 1].  Pass 1 issues the MFMAs as one
  // cluster at raised wave priority before the epilogue (3% faster on long
  // prompts' row blocks; pass 2 measured no gain from it and keeps the
  // compiler's interleave).  csum starts at -0: its first add folds away.
  f32x16 acc[2][FR_TW];
  u32x4 kf[Geo::NV];
  auto mma_prio = [&](f32x16* a, const u32x4* k) {
    if constexpr (!PASS2) __builtin_amdgcn_s_setprio(1);
    mma_both(a, k);
    if constexpr (!PASS2) __builtin_amdgcn_s_setprio(0);
  };
  auto subtile = [&](int buf, int u, int g) {
    const int j = g - 1;
    const bool clean = j >= 0 && j < nsub && kbeg + j * TILE + TILE - 1 <= qb0;
    float csum = -0.f;
    if (clean) {
      read_k(buf, u, kf);
      mma_prio(acc[u & 1], kf);
      epi_clean(acc[(u & 1) ^ 1], csum);
    } else {
      read_k(buf, u, kf);
      mma_prio(acc[u & 1], kf);
      epi_general(acc[(u & 1) ^ 1], j, csum);
    }
    if constexpr (PASS2) {
      if (j >= 0) red_store(j, csum);
    }
  };

  // Q (and the row table's loads) complete before the K ring starts, so the
  // loads in flight at the loop head are exactly the ring, oldest first --
  // the same order every later iteration sees.
  vm_wait_all();
#pragma unroll
  for (int s = 0; s < FR_RING; ++s) issue(s, ring[s]);
  __syncthreads();  // row table visible
  if constexpr (PASS2) {
#pragma unroll
    for (int t = 0; t < FR_TW; ++t) {
      const int lrow = (wave + t * FR_WAVES) * TILE;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 ov = *reinterpret_cast<const f32x4*>(&row_off[lrow + 8 * jj + 4 * hf]);
#pragma unroll
        for (int e = 0; e < 4; ++e) off[t][4 * jj + e] = ov[e];
      }
    }
  }
  commit(0, 0, ring[0]);
  issue(FR_RING, ring[0]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < FR_SUB; ++u) subtile(0, u, u);  // stage 0
  commit(1, 1, ring[1]);
  issue(FR_RING + 1, ring[1]);
  __syncthreads();

  // Stage st: sub-tiles st*FR_SUB + u, then stage st + 1 goes to LDS.  The
  // loop runs a multiple of FR_RING stages with no early exit (stages past
  // the chunk do no arithmetic that is kept), so every unrolled step sees the
  // same loads in flight and waits only for the oldest stage.
  const int nst_pad = (nst + FR_RING - 1) / FR_RING * FR_RING;
  for (int st0 = 1; st0 < 1 + nst_pad; st0 += FR_RING) {
#pragma unroll
    for (int s = 0; s < FR_RING; ++s) {
      const int st = st0 + s;
      const int buf = (1 + s) & 1;  // == st & 1
      if constexpr (PASS2) {
#pragma unroll
        for (int u = 0; u < FR_SUB; ++u) flush(st * FR_SUB + u - FR_SUB - 1, u);  // previous stage's epilogues
      }
#pragma unroll
      for (int u = 0; u < FR_SUB; ++u) subtile(buf, u, st * FR_SUB + u);
      {
        const int nxt = (2 + s) % FR_RING;  // == (st + 1) % FR_RING
        commit(buf ^ 1, st + 1, ring[nxt]);
        issue(st + 1 + FR_RING, ring[nxt]);
      }
      __syncthreads();
    }
  }

  if constexpr (PASS2) {
    const int st = nst_pad;  // epilogues of the last stage
#pragma unroll
    for (int u = 0; u < FR_SUB; ++u) flush(st * FR_SUB + u - 1, u);
  } else {
#pragma unroll
    for (int t = 0; t < FR_TW; ++t) {
      const float mo = wave_xor32(mref[t]);
      const float lo = wave_xor32(lsum[t]);
      const float mx = fmaxf(mref[t], mo);
      float lt = 0.f;
      if (mx != -INFINITY) {
        lt = (mref[t] == -INFINITY ? 0.f : lsum[t] * fast_exp2(mref[t] - mx)) +
             (mo == -INFINITY ? 0.f : lo * fast_exp2(mo - mx));
      }
      if (hf == 0 && qrow[t] >= 0) {
        const int r = rbase + (wave + t * FR_WAVES) * TILE + col;
        const int j = r / G;
        const int g = h * G + (r - j * G);
        if (nc == 1) {
          args.lse[(int64_t)g * args.T + tok0 + qrow[t]] = (mx + log2f(lt)) * LN2;
        } else {
          args.part[tab.ws0[p] + ((int64_t)h * tab.prow[p] + r) * nc + chunk] = make_float2(mx, lt);
        }
      }
    }
  }
}

template <typename T, int D, bool PASS2, int FR_WAVES, int FR_TW>
__global__ void __launch_bounds__(FR_WAVES * WAVE)
few_rows_kernel(const FrArgs args) {
  __shared__ FrLds<T, D, FR_WAVES, FR_TW> L;
  few_rows_body<T, D, PASS2, FR_WAVES, FR_TW>(args, args.tab.first, blockIdx.x, L);
}

// Pass 2 of heads in several row blocks: a key's score is the sum, in
// row-block order, of the column sums of the blocks whose rows can see it.
// Block rb sees key k when G (k - q0) is at most its last packed row, i.e.
// from block floor(G max(0, k - q0) / rows) on (the last block sees every key).
struct RowBlockReduceArgs {
  const float* cpart;
  float* scores;
  int64_t T;
  int32_t hkv;
  int32_t G;
  int32_t rows;               // packed rows per block
  SeqTable tab;               // first[]: items (hkv * N per sequence); nrb, n, q0, ws0, tok0
};

__global__ void __launch_bounds__(256)
rowblock_reduce_kernel(const RowBlockReduceArgs args) {
  const SeqTable& tab = args.tab;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= tab.first[tab.nb]) return;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int N = tab.n[p];
  const int h = local / N;
  const int key = local - h * N;
  const int nrb = tab.nrb[p];
  const int64_t R = (int64_t)args.G * max(0, key - tab.q0[p]);
  const int rb0 = (int)min<int64_t>(R / args.rows, nrb - 1);
  const int64_t stride = (int64_t)args.hkv * N;
  const float* src = args.cpart + tab.ws0[p] + (int64_t)h * N + key + rb0 * stride;
  args.scores[(int64_t)h * args.T + tab.tok0[p] + key] = ordered_strided_sum(src, stride, nrb - rb0);
}

}  // namespace waits
