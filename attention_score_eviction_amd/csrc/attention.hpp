// Prefill attention forward with the per-row log-sum-exp: the model's causal
// attention call that the WAITS plugin sits in (README "Quickstart").  Its
// row normaliser is exactly what WAITS pass 1 computes, so a caller that
// runs this kernel hands `lse` straight to the pass-2 column sums and pass
// 1's QK^T costs nothing extra.
//
//   out[t0 + q, g, :] = sum_{k <= q} softmax_k(scale <Q[q, g], K[k, h]>) V[k, h, :]
//   lse[g, t0 + q]    = ln sum_{k <= q} exp(scale <Q[q, g], K[k, h]>),   h = g / G
//
// Work item = (sequence, KV head, block of AT_ROWS packed rows); packed row r
// of KV head h is query position r / G of query head h G + r % G, so the G
// query heads that share K/V rows share the workgroup.  Four waves (one per
// SIMD, so a wave may hold 512 registers: the O accumulators and the Q
// fragments sit in AGPRs), each with two 32-row tiles that share every K and
// V fragment it reads.
// Keys 0 .. the block's last query stream through LDS in 64-key stages: K
// row-major (padded rows), V transposed (V^T[d][key]) so that it can be the
// A operand of O^T += V^T P^T; a one-stage register ring keeps the next
// stage's loads in flight (the K/V rows are re-read by every row block of the
// head, so most come from L2).  Per 32-key sub-tile and row tile:
//   S^T = K Q^T           32x32x16 MFMAs; a lane owns one row and 16 keys
//   softmax epilogue      lazy exponent reference shared by the two lanes of
//                         a row; P rounded to bf16 for the MFMA, sums in fp32
//   O^T += V^T P^T        32x32x16 MFMAs into fp32 accumulators
// Per sub-tile g a wave issues its S^T MFMAs, then P V^T of sub-tile g - 1,
// and in the same basic block the softmax of sub-tile g, which overlaps those
// P V^T MFMAs and writes the next P operands.  V^T keeps its keys in the order the P^T operand lanes hold
// them (bits 2 and 3 of a key's index within its 32-key tile swapped), so a
// lane reads its 8 keys of one head-dim row as one 16-byte load.  V has three
// LDS buffers: P V^T of a stage's last sub-tile runs in the next stage, while
// other waves may already write the stage after that.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int AT_WAVES = 4;
constexpr int AT_TW = 2;                     // 32-row tiles per wave
constexpr int AT_THREADS = AT_WAVES * WAVE;
constexpr int AT_ROWS = AT_WAVES * AT_TW * TILE;  // packed rows per workgroup
constexpr int AT_SUB = 2;                    // 32-key sub-tiles per stage
constexpr int AT_STAGE = AT_SUB * TILE;      // keys per stage
constexpr int AT_RING = 1;                   // stages of loads in flight

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  bf16_t* out;                // [T, Hq, D], dense
  float* lse;                 // [Hq, T] or null
  Strides st;                 // Q and K/V element strides
  int64_t ntok;               // T
  int32_t G;
  int32_t hkv;
  int32_t hq;
  float scale_log2;           // scale * log2(e)
  SeqTable tab;               // n, tok0, nrb (row blocks per KV head), first
};

// Position of key kk (0..31) of a sub-tile in V^T: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_slot(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D>
__global__ void __launch_bounds__(AT_THREADS) attn_fwd_kernel(const AttnArgs a) {
  using T = bf16_t;
  using Geo = TileGeom<T, D>;
  constexpr int HALF = Geo::ROW_BYTES / 2;
  constexpr int CPR = Geo::ROW_BYTES / 16;       // 16-byte chunks per row
  constexpr int NDT = D / 32;                    // head-dim tiles of O^T
  constexpr int KCH = AT_STAGE * CPR;            // K chunks per stage
  constexpr int KSV = KCH / AT_THREADS;          // per thread
  constexpr int VPAIRS = AT_STAGE / 2 * CPR;     // (key pair, chunk) units per stage
  constexpr int VSV = VPAIRS / AT_THREADS;       // per thread
  constexpr int VT_W = AT_STAGE / 2 + 4;         // 32-bit words per V^T row (padded)
  constexpr int NR = KSV + 2 * VSV;              // ring vectors per stage and thread
  static_assert(KCH % AT_THREADS == 0 && VPAIRS % AT_THREADS == 0, "staging split");
  __shared__ __attribute__((aligned(16))) unsigned char lk[2][AT_SUB][Geo::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t lv[3][D][VT_W];

  const SeqTable& tab = a.tab;
  const int item = blockIdx.x;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int hkv = a.hkv, G = a.G;
  const int h = local % hkv;
  const int rb = tab.nrb[p] - 1 - local / hkv;   // longest key ranges first
  const int N = tab.n[p];
  const int PR = G * N;
  const int64_t tok0 = tab.tok0[p];
  const int rbase = rb * AT_ROWS;
  const int kend = (min(rbase + AT_ROWS, PR) - 1) / G + 1;   // keys the block sees
  const int nsub = (kend + TILE - 1) / TILE;
  const int nst = (nsub + AT_SUB - 1) / AT_SUB;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const float cl2 = a.scale_log2;

  // Row tiles wave + AT_WAVES t: this lane's row of each and its Q fragments.
  int tlo[AT_TW], thi[AT_TW], qpos[AT_TW], grow[AT_TW];
  bool row_ok[AT_TW];
  u32x4 qf[AT_TW][Geo::NV];
#pragma unroll
  for (int t = 0; t < AT_TW; ++t) {
    const int r0 = rbase + (wave + AT_WAVES * t) * TILE;
    tlo[t] = min(r0, PR - 1) / G;
    thi[t] = (min(r0 + TILE, PR) - 1) / G;
    const int row = r0 + col;
    row_ok[t] = row < PR;
    qpos[t] = row_ok[t] ? row / G : -1;          // -1: padding, every key masked
    grow[t] = h * G + (row_ok[t] ? row % G : 0);
    const int qq = row_ok[t] ? qpos[t] : 0;
    const unsigned char* src = static_cast<const unsigned char*>(a.q) +
                               ((tok0 + qq) * a.st.q_tok + (int64_t)grow[t] * a.st.q_head) * Geo::ELT +
                               hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) {
      const u32x4 x = ld16(src + 16 * v);
      qf[t][v] = row_ok[t] ? x : u32x4{0u, 0u, 0u, 0u};
      // Q lives in AGPRs for the whole item: the S^T MFMAs read their B
      // operand from there directly, leaving the VGPRs to K, P and the ring
      asm volatile("" : "+a"(qf[t][v]));
    }
  }

  // K/V staging: buffer resources over head h's rows of this sequence; the
  // hardware range check returns zeros past the sequence.
  const int row_bytes = (int)(a.st.kv_tok * Geo::ELT);
  const int64_t head0 = (tok0 * a.st.kv_tok + (int64_t)h * a.st.kv_head) * Geo::ELT;
  const int krange = (int)min((int64_t)N * row_bytes, (int64_t)0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(a.k) + head0), 0, krange,
      BUFFER_RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(a.v) + head0), 0, krange,
      BUFFER_RSRC_WORD3);
  int koff[KSV], voff[VSV], vch[VSV], vword[VSV];
#pragma unroll
  for (int i = 0; i < KSV; ++i) {
    const int cid = tid + i * AT_THREADS;
    koff[i] = (cid / CPR) * row_bytes + (cid % CPR) * 16;
  }
#pragma unroll
  for (int i = 0; i < VSV; ++i) {
    const int u = tid + i * AT_THREADS;
    const int kk = 2 * (u % (AT_STAGE / 2));     // first key of the pair in the stage
    vch[i] = u / (AT_STAGE / 2);
    voff[i] = kk * row_bytes + vch[i] * 16;
    vword[i] = ((kk / TILE) * TILE + vt_slot(kk % TILE)) / 2;
  }
  u32x4 ring[AT_RING][NR];
  auto issue = [&](int stage, u32x4* dst) __attribute__((always_inline)) {
    const int sbase = min(stage, nst - 1) * AT_STAGE * row_bytes;
#pragma unroll
    for (int i = 0; i < KSV; ++i)
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff[i] + sbase, 0, 0));
#pragma unroll
    for (int i = 0; i < VSV; ++i) {
      dst[KSV + 2 * i] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i] + sbase, 0, 0));
      dst[KSV + 2 * i + 1] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff[i] + row_bytes + sbase, 0, 0));
    }
  };
  auto commit = [&](int kb, int vb, const u32x4* src) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KSV; ++i) {
      const int cid = tid + i * AT_THREADS;
      const int r = cid / CPR;
      st16(lk[kb][r / TILE] + (r % TILE) * Geo::LDS_STRIDE + (cid % CPR) * 16, src[i]);
    }
#pragma unroll
    for (int i = 0; i < VSV; ++i) {
      const u32x4 x0 = src[KSV + 2 * i], x1 = src[KSV + 2 * i + 1];  // keys kk, kk + 1
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        lv[vb][8 * vch[i] + 2 * w][vword[i]] = __builtin_amdgcn_perm(x1[w], x0[w], 0x05040100u);
        lv[vb][8 * vch[i] + 2 * w + 1][vword[i]] = __builtin_amdgcn_perm(x1[w], x0[w], 0x07060302u);
      }
    }
  };

  f32x16 acc_s[AT_TW];
  f32x16 acc_o[AT_TW][NDT];
  float mref[AT_TW], lsum[AT_TW];
  bf16x8 pb[AT_TW][2];          // P^T operands of the previous sub-tile
#pragma unroll
  for (int t = 0; t < AT_TW; ++t) {
#pragma unroll
    for (int d = 0; d < NDT; ++d) acc_o[t][d] = f32x16{};
    // padding rows (never written) keep a finite reference, so that they
    // never send a sub-tile down the rare path
    mref[t] = row_ok[t] ? -INFINITY : 0.f;
    lsum[t] = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s) pb[t][s] = bf16x8{};
  }
  u32x4 kf[Geo::NV];

  // Softmax of sub-tile j (acc_s) into the bf16 P^T operands pb.  diag
  // (wave-uniform): the sub-tile may reach past a row's position.  The fast
  // path has no masks: a diagonal sub-tile (about one in a hundred) goes
  // through the rare path, which recomputes its exponentials with keys after
  // each row's position masked; a tile whose rows all precede the sub-tile
  // gets P = 0 there.
  auto epilogue = [&](int j, bool diag) __attribute__((always_inline)) {
    const int ktj = j * TILE;
    // masked logit (log2 units) for the rare path
    auto logit = [&](int t, int v) __attribute__((always_inline)) {
      const float s = acc_s[t][v] * cl2;
      return (diag && ktj + out_row(v, hf) > qpos[t]) ? -INFINITY : s;
    };
    float pv[AT_TW][16], lold[AT_TW];
#pragma unroll
    for (int t = 0; t < AT_TW; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) pv[t][v] = fast_exp2(fmaf(acc_s[t][v], cl2, -mref[t]));
    bool ok = !diag;
#pragma unroll
    for (int t = 0; t < AT_TW; ++t) {
      lold[t] = lsum[t];
      const float ln = lsum[t] + sum16(pv[t]);
      ok = ok && ln < 0x1p64f;
      lsum[t] = ln;
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) != 0, 0)) {
      // Rare (a diagonal sub-tile, a row's first keys, or a much larger
      // score later): move the reference of both lanes of every row to their
      // common max and rescale what was summed against the old one.
#pragma unroll
      for (int t = 0; t < AT_TW; ++t) {
        lsum[t] = lold[t];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, logit(t, v));
        mx = fmaxf(mx, wave_xor32(mx));
        const float mnew = fmaxf(mref[t], mx);
        if (mnew == -INFINITY) {
          lsum[t] = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) pv[t][v] = 0.f;
        } else {
          if (mref[t] == -INFINITY) {
            lsum[t] = 0.f;
          } else if (mnew != mref[t]) {
            const float alpha = fast_exp2(mref[t] - mnew);
#pragma unroll
            for (int d = 0; d < NDT; ++d)
#pragma unroll
              for (int v = 0; v < 16; ++v) acc_o[t][d][v] *= alpha;
            lsum[t] *= alpha;
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) pv[t][v] = fast_exp2(logit(t, v) - mnew);
          lsum[t] += sum16(pv[t]);
          mref[t] = mnew;
        }
      }
    }
#pragma unroll
    for (int t = 0; t < AT_TW; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[t][s][e] = (__bf16)pv[t][8 * s + e];
  };

  // O^T += V^T P^T with pb, for sub-tile u of V buffer vb.
  auto pv_mma = [&](int vb, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, ld16(&lv[vb][32 * d + col][16 * u + 8 * s + 4 * hf]));
#pragma unroll
        for (int t = 0; t < AT_TW; ++t)
          acc_o[t][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[t][s], acc_o[t][d], 0, 0, 0);
      }
  };

  // Sub-tile g (slot u of K buffer kb): its S^T MFMAs, then P V^T of sub-tile
  // g - 1 (V buffer vb_prev, slot u_prev, operands pb) in the same basic
  // block as the softmax of sub-tile g, which writes the next pb.  Sub-tiles
  // below every row of the wave (the common case) need no mask.
  auto subtile = [&](int kb, int u, int g, int vb_prev, int u_prev) __attribute__((always_inline)) {
    const bool diag = g * TILE + TILE - 1 > tlo[0];     // tile 0 holds the wave's lowest rows
    {
      const unsigned char* krow = lk[kb][u] + col * Geo::LDS_STRIDE + hf * HALF;
#pragma unroll
      for (int v = 0; v < Geo::NV; ++v) kf[v] = ld16(krow + 16 * v);
#pragma unroll
      for (int t = 0; t < AT_TW; ++t) acc_s[t] = f32x16{};
      if constexpr (AT_TW == 2) mma_tile2<T, D, true>(acc_s[0], acc_s[1], qf[0], qf[1], kf);
      else mma_tile<T, D>(acc_s[0], kf, qf[0]);
    }
    pv_mma(vb_prev, u_prev);
    epilogue(g, diag);
  };

  vm_wait_all();
#pragma unroll
  for (int s = 0; s < AT_RING; ++s) issue(s, ring[s]);
  commit(0, 0, ring[0]);
  issue(AT_RING, ring[0]);
  __syncthreads();
  // stage 0 (P V^T of "sub-tile -1" adds the zero operands)
  subtile(0, 0, 0, 0, 0);
  subtile(0, 1, 1, 0, 0);
  commit(1, 1, ring[1 % AT_RING]);
  issue(AT_RING + 1, ring[1 % AT_RING]);
  __syncthreads();

  // Stages 1 .. nst_pad: the last one only finishes the block's last real
  // sub-tile (its own sub-tiles lie past every key and get P = 0).
  const int nst_pad = (nst + AT_RING - 1) / AT_RING * AT_RING;
  for (int st0 = 1; st0 < 1 + nst_pad; st0 += AT_RING) {
#pragma unroll
    for (int s = 0; s < AT_RING; ++s) {
      const int st = st0 + s;
      const int kb = st & 1;
      const int vb = st % 3, vb_prev = (st + 2) % 3;
      subtile(kb, 0, st * AT_SUB, vb_prev, AT_SUB - 1);
      subtile(kb, 1, st * AT_SUB + 1, vb, 0);
      {
        const int nxt = (2 + s) % AT_RING;  // == (st + 1) % AT_RING
        commit(kb ^ 1, (st + 1) % 3, ring[nxt]);
        issue(st + 1 + AT_RING, ring[nxt]);
      }
      __syncthreads();
    }
  }

  // Normalise and write this lane's half of each row.
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int t = 0; t < AT_TW; ++t) {
    const float ltot = lsum[t] + wave_xor32(lsum[t]);
    if (!row_ok[t]) continue;
    const int64_t tk = tok0 + qpos[t];
    const float inv = 1.f / ltot;
    unsigned char* dst = reinterpret_cast<unsigned char*>(a.out + (tk * a.hq + grow[t]) * D);
#pragma unroll
    for (int d = 0; d < NDT; ++d)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc_o[t][d][4 * v4 + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + (32 * d + out_row(4 * v4, hf)) * 2) = o4;
      }
    if (hf == 0 && a.lse) a.lse[(int64_t)grow[t] * a.ntok + tk] = (mref[t] + log2f(ltot)) * LN2;
  }
}

}  // namespace waits
