// Pass 2 for heads with many processed rows: column-owner workgroups
// (WAITS README, introduction: each key's score is the forgetting-curve
// weighted sum over query rows of its causal attention probability):
//   s[h, k] = sum_{g in group h} sum_{q >= k} w[q] exp(scale <Q[g,q], K[h,k]> - lse[g,q])
// with w folded into one exponent offset per row,
//   off[q] = lse[g,q] * log2 e + log2(1 + exp(-a (q - c))),   p = exp2(dot * scale*log2 e - off).
//
// Work item = (sequence, KV head h, block of KB_KEYS keys, row chunk).  8
// waves; wave w owns the 32-key tiles k0 + 32 w and k0 + 256 + 32 w, whose
// K rows sit in registers as MFMA B operands for the whole item.  The packed
// query rows of the chunk (the G query heads of h interleaved, starting at
// the first row whose query can see k0) stream past them in stages of two
// 32-row tiles, with each row's exponent offset and position:
// HBM -> registers (KB_RING stages of loads in flight) -> LDS (double buffer,
// one barrier per stage) -> every wave.  MFMA(A = Q rows, B = K tile): each
// lane owns one key column and 16 rows of a tile, so a key's sum is in-lane
// work plus, at the end, one exchange between the lane halves; no wave
// shares keys with another.  Each wave issues the MFMAs of row tile g in the
// same basic block as the epilogue of row tile g - 1.
//
// A block whose rows form one chunk writes its scores directly; otherwise
// every chunk writes its partial sums and colsum_reduce_kernel adds them in
// chunk order -- no atomics, bitwise reproducible.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int KB_WAVES = 8;
constexpr int KB_THREADS = KB_WAVES * WAVE;
constexpr int KB_KEYS = KB_WAVES * 2 * TILE;  // 512 keys per block
constexpr int KB_STAGE = 2 * TILE;            // packed rows per stage
constexpr int KB_RING = 2;                    // stages of loads in flight

struct BlockArgs {
  const void* q;
  const void* k;
  const float* lse;           // [Hq, T]
  float* scores;              // [Hkv, T]
  float* part;                // [row chunk][Hkv][T] partial sums (blocks with several chunks)
  Strides st;
  int64_t T;
  int32_t G;
  int32_t hkv;
  float scale_log2;
  SeqTable tab;               // nc: row chunks per key block; first[]: items
};

template <typename T, int D>
__global__ void __launch_bounds__(KB_THREADS)
key_block_kernel(const BlockArgs args) {
  using Geo = TileGeom<T, D>;
  constexpr int HALF = Geo::ROW_BYTES / 2;
  constexpr int CPR = Geo::ROW_BYTES / 16;                  // 16-byte chunks per Q row
  constexpr int CHUNKS = KB_STAGE * CPR;                     // per stage
  constexpr int SV = (CHUNKS + KB_THREADS - 1) / KB_THREADS; // chunks per thread per stage
  static_assert(KB_RING % 2 == 0, "LDS buffer parity follows the unrolled stage index");
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][2][Geo::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float s_off[2][KB_STAGE];

  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int hkv = args.hkv, G = args.G;
  const int h = local % hkv;
  const int rest = local / hkv;
  const int nrc = tab.nc[p];
  const int kblk = rest / nrc;  // ascending: blocks seen by more rows first
  const int rc = rest - kblk * nrc;
  const int N = tab.n[p], q0 = tab.q0[p];
  const int PR = G * (N - q0);
  const int64_t tok0 = tab.tok0[p];
  const float a = tab.a[p], c = tab.c[p];
  const int k0 = kblk * KB_KEYS;

  // Rows of this chunk: the rows from the first one whose query reaches k0
  // to the last, cut into nrc chunks of whole stages.
  const int r_lo = G * max(0, k0 - q0);
  const int span = PR - r_lo;
  const int cr = ((span + nrc - 1) / nrc + KB_STAGE - 1) / KB_STAGE * KB_STAGE;
  const int rbeg = r_lo + rc * cr;
  const int rend = min(rbeg + cr, PR);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 31, hf = lane >> 5;
  const int kt[2] = {k0 + wave * TILE, k0 + (wave + KB_WAVES) * TILE};
  float* const out = nrc == 1 ? args.scores + (int64_t)h * args.T + tok0
                              : args.part + ((int64_t)rc * hkv + h) * args.T + tok0;

  if (rbeg >= rend) {  // a chunk past the block's rows: its partials are zero
    if (hf == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (kt[t] + col < N) out[kt[t] + col] = 0.f;
    }
    return;
  }
  const int nst = (rend - rbeg + KB_STAGE - 1) / KB_STAGE;

  const unsigned char* qb = static_cast<const unsigned char*>(args.q);
  const unsigned char* kb = static_cast<const unsigned char*>(args.k);
  const float cl2 = args.scale_log2;

  // Stationary K fragments: this lane's key of each of the wave's two tiles.
  u32x4 kf[2][Geo::NV];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int key = kt[t] + col;
    const bool ok = key < N;
    const unsigned char* src =
        kb + ((tok0 + (ok ? key : N - 1)) * args.st.kv_tok + (int64_t)h * args.st.kv_head) * Geo::ELT +
        hf * HALF;
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) {
      const u32x4 x = ld16(src + 16 * v);
      kf[t][v] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Q staging: buffer loads over the chunk's queries of the G heads of group
  // h (the host keeps that span below 2^31 bytes); rows past the chunk load a
  // clamped row and carry off = +inf, so they add exactly 0.  Stages past
  // the chunk re-read its last one, so every thread issues the same loads per
  // stage.
  const int qbase = q0 + rbeg / G;  // first query of the chunk
  const unsigned char* qseq =
      qb + ((tok0 + qbase) * args.st.q_tok + (int64_t)h * G * args.st.q_head) * Geo::ELT;
  const int qrange = (int)min(((int64_t)(N - 1 - qbase) * args.st.q_tok + (int64_t)(G - 1) * args.st.q_head) *
                                      Geo::ELT + Geo::ROW_BYTES,
                              (int64_t)0x7FFFFFFF);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(qseq), 0, qrange, BUFFER_RSRC_WORD3);
  u32x4 ring[KB_RING][SV];
  float lring[KB_RING];
  auto row_of = [&](int stage, int i) { return min(rbeg + min(stage, nst - 1) * KB_STAGE + i, rend - 1); };
  auto issue = [&](int stage, u32x4* dst, float& ldst) {
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int cid = min(tid + i * KB_THREADS, CHUNKS - 1);
      const int r = row_of(stage, cid / CPR);
      const int j = r / G;
      const int gi = r - j * G;  // query head within the group
      const int off = (int)(((int64_t)(q0 + j - qbase) * args.st.q_tok + (int64_t)gi * args.st.q_head) *
                            Geo::ELT) + (cid % CPR) * 16;
      dst[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
    }
    {
      const int r = row_of(stage, tid & (KB_STAGE - 1));
      const int j = r / G;
      ldst = args.lse[(int64_t)(h * G + (r - j * G)) * args.T + tok0 + q0 + j];
    }
  };
  auto commit = [&](int buf, int stage, const u32x4* src, float lv) {
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int cid = tid + i * KB_THREADS;
      if (cid < CHUNKS) {
        const int row = cid / CPR;
        st16(lds[buf][row / TILE] + (row % TILE) * Geo::LDS_STRIDE + (cid % CPR) * 16, src[i]);
      }
    }
    if (tid < KB_STAGE) {
      const int r = rbeg + stage * KB_STAGE + tid;
      const bool ok = stage < nst && r < rend;
      const int q = q0 + r / G;
      const float e = expf(-a * ((float)q - c));  // w = 1 / (1 + e)
      s_off[buf][tid] = ok ? fmaf(lv, LOG2E, log2f(1.f + e)) : INFINITY;
    }
  };

  float csum[2] = {0.f, 0.f};
  f32x16 acc[2][2];
  float off[2][16];
  // Row tile g (stage g / 2, tile u = g % 2): MFMAs into acc[u]; epilogue of
  // row tile g - 1 from acc[u ^ 1] with its offsets off[u ^ 1] (registers:
  // another wave may already be refilling that tile's LDS buffer) and its
  // rows' query positions derived from the row indices.
  auto rowtile = [&](int buf, int u, int g) {
    const unsigned char* arow = lds[buf][u] + col * Geo::LDS_STRIDE + hf * HALF;
    u32x4 af[Geo::NV];
#pragma unroll
    for (int v = 0; v < Geo::NV; ++v) af[v] = ld16(arow + 16 * v);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 ov = *reinterpret_cast<const f32x4*>(&s_off[buf][u * TILE + 8 * jj + 4 * hf]);
#pragma unroll
      for (int e = 0; e < 4; ++e) off[u][4 * jj + e] = ov[e];
    }
    const int pg = g - 1;
    const int pu = u ^ 1;
    const int r_first = rbeg + pg * TILE;
    const int r_last = min(r_first + TILE, rend) - 1;
    const bool live = pg >= 0 && r_first < rend;
    const int qlo = q0 + r_first / G, qhi = q0 + r_last / G;
    // per key tile: 0 nothing visible, 1 fully visible, 2 crossing the diagonal
    int kind[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) kind[t] = !live || kt[t] > qhi ? 0 : (kt[t] + TILE - 1 <= qlo ? 1 : 2);
    acc[u][0] = f32x16{};
    acc[u][1] = f32x16{};
    mma_tile2<T, D, true>(acc[u][0], acc[u][1], kf[0], kf[1], af);
    if (kind[0] == 1 && kind[1] == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float pv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(acc[pu][t][v], cl2, -off[pu][v]));
        csum[t] += sum16(pv);
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if (kind[t] == 0) continue;
        float pv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = fast_exp2(fmaf(acc[pu][t][v], cl2, -off[pu][v]));
        if (kind[t] == 2) {  // rows past the chunk already carry off = +inf
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (kt[t] + col > q0 + (r_first + out_row(v, hf)) / G) pv[v] = 0.f;
        }
        csum[t] += sum16(pv);
      }
    }
  };

  // Prologue: stage 0 to LDS, row tiles 0 and 1, stage 1 to LDS.
  vm_wait_all();
#pragma unroll
  for (int s = 0; s < KB_RING; ++s) issue(s, ring[s], lring[s]);
  commit(0, 0, ring[0], lring[0]);
  issue(KB_RING, ring[0], lring[0]);
  __syncthreads();
  rowtile(0, 0, 0);
  rowtile(0, 1, 1);
  commit(1, 1, ring[1], lring[1]);
  issue(KB_RING + 1, ring[1], lring[1]);
  __syncthreads();

  // Stage st: row tiles 2 st and 2 st + 1, then stage st + 1 goes to LDS.
  // The loop runs a multiple of KB_RING stages, one past the chunk's last so
  // its last row tile gets its epilogue, with no early exit.
  const int nst_pad = (nst + KB_RING - 1) / KB_RING * KB_RING;
  for (int st0 = 1; st0 < 1 + nst_pad; st0 += KB_RING) {
#pragma unroll
    for (int s = 0; s < KB_RING; ++s) {
      const int st = st0 + s;
      const int buf = (1 + s) & 1;  // == st & 1
      rowtile(buf, 0, 2 * st);
      rowtile(buf, 1, 2 * st + 1);
      const int nxt = (2 + s) % KB_RING;  // == (st + 1) % KB_RING
      commit(buf ^ 1, st + 1, ring[nxt], lring[nxt]);
      issue(st + 1 + KB_RING, ring[nxt], lring[nxt]);
      __syncthreads();
    }
  }

#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float sc = csum[t] + wave_xor32(csum[t]);
    if (hf == 0 && kt[t] + col < N) out[kt[t] + col] = sc;
  }
}

// scores[h, k] = sum over row chunks (in order) of the partial sums, for the
// sequences whose key blocks were split.  first[] counts (KV head, key) pairs.
struct ReduceArgs {
  const float* part;
  float* scores;
  int64_t T;
  int32_t hkv;
  SeqTable tab;               // nc: row chunks
};

__global__ void __launch_bounds__(256)
colsum_reduce_kernel(const ReduceArgs args) {
  const SeqTable& tab = args.tab;
  const int item = blockIdx.x * 256 + threadIdx.x;
  if (item >= tab.first[tab.nb]) return;
  const int p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[p];
  const int N = tab.n[p];
  const int h = local / N;
  const int key = local - h * N;
  const int64_t at = (int64_t)h * args.T + tab.tok0[p] + key;
  const int64_t stride = (int64_t)args.hkv * args.T;
  args.scores[at] = ordered_strided_sum(args.part + at, stride, tab.nc[p]);
}

}  // namespace waits
