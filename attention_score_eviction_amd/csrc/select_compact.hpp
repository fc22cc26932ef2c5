// Top-k selection and K/V compaction (WAITS README: the top-k selector of
// "Repository layout" keeps the highest-scoring keys per KV head; the
// introduction's retained key-value pairs are then gathered).
//
// select_kernel: one 1024-thread workgroup per (sequence, KV head).  Scores
// are non-negative fp32, so their bit patterns order like the values; an
// MSB-first radix select (4 digits of 8 bits) finds the bit pattern T of the
// budget-th largest score and how many of the kept keys must equal T.  Keys
// above T, then the lowest-positioned keys equal to T (ties go to the lower
// position), are written in ascending position order.
//
// Layout: wave w owns the contiguous key segment [w * seg, (w + 1) * seg)
// (seg a multiple of 64), lane l its keys w * seg + 64 i + l, so every load
// is coalesced and position order is (wave, i, lane) order.  Segments of up
// to 64 * PTC keys stay in registers across the passes; longer ones are
// re-read (from L2) on every pass.
//
// Histograms: the first digit is shared by almost every key, so its counts
// go to per-(digit, lane % 32) words (the lanes of one atomic hit distinct
// words instead of serialising on one) and are then folded into 256 digit
// counts; later passes see few matching keys and count directly.  Every wave
// derives the picked digit from the histogram itself: one barrier per pass
// (two for the first).
//
// Output: a key's slot is (#kept keys above T before it) + min(#keys equal
// to T before it, the number of T-equal keys kept), from wave ballots, their
// prefix within the wave and a prefix over the 16 wave totals; no block
// scan, no atomics.
//
// FUSE: the same workgroup then gathers the kept K and V rows (bit copies,
// 16-byte vectors; zero rows past the kept count), so select and compact are
// one launch.
//
// compact_kernel: one 16-byte vector per thread, rows of K and V copied bit
// for bit; empty slots (-1) are zero-filled.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int SEL_SUB = 32;          // sub-counters per digit
constexpr int SEL_FUSE_MAX = 8192;   // largest budget the fused gather keeps in LDS
constexpr int SEL_BATCH = 16;        // keys per lane loaded together (no register cache)

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Wave-uniform pick from a 256-bin histogram: the digit d whose keys hold the
// krem-th largest (counting from the highest digit), and how many keys lie
// in higher digits.  Every wave computes it, so no barrier hands it out.
__device__ __forceinline__ void pick_digit(const int* hist, int krem, int lane, int& digit,
                                           int& above_out) {
  // lane L holds digits 255-4L .. 252-4L (highest digits first)
  int hv[4], lsum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hv[j] = hist[255 - 4 * lane - j];
    lsum += hv[j];
  }
  int above = wave_incl_scan(lsum) - lsum, myd = -1, mya = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (above < krem && krem <= above + hv[j]) {
      myd = 255 - 4 * lane - j;
      mya = above;
    }
    above += hv[j];
  }
  const int src = __builtin_ctzll(__ballot(myd >= 0));  // exactly one lane
  digit = __builtin_amdgcn_readlane(myd, src);
  above_out = __builtin_amdgcn_readlane(mya, src);
}

template <int PTC, bool FUSE>
__global__ void __launch_bounds__(SEL_THREADS)
select_kernel(const SelectArgs args) {
  __shared__ __attribute__((aligned(16))) int sub[256 * SEL_SUB];
  __shared__ int hist[4][256];
  __shared__ int wtot[2][SEL_WAVES];
  __shared__ int sel[FUSE ? SEL_FUSE_MAX : 1];

  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  const int p = item / args.hkv;
  const int h = item - p * args.hkv;
  const int N = tab.n[p];
  const int budget = args.budget;
  const int keep = min(budget, N);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t* out = args.idx + ((int64_t)p * args.hkv + h) * budget;
  for (int j = keep + tid; j < budget; j += SEL_THREADS) out[j] = -1;

  if (keep == N) {  // every key is kept
    for (int j = tid; j < N; j += SEL_THREADS) {
      out[j] = j;
      if constexpr (FUSE) sel[j] = j;
    }
  } else {
    const uint32_t* s = reinterpret_cast<const uint32_t*>(args.scores + (int64_t)h * args.T + tab.tok0[p]);
    const int seg = (N + SEL_THREADS - 1) / SEL_THREADS * WAVE;  // keys per wave, multiple of 64
    const int iters = seg / WAVE;
    const int e0 = wave * seg + lane;
    uint32_t cache[PTC > 0 ? PTC : 1];
    if constexpr (PTC > 0) {
#pragma unroll
      for (int i = 0; i < PTC; ++i) {
        const int e = e0 + i * WAVE;
        cache[i] = (i < iters && e < N) ? s[e] : 0u;
      }
    }
    for (int i = tid; i < 256 * SEL_SUB / 4; i += SEL_THREADS)
      reinterpret_cast<int4*>(sub)[i] = int4{0, 0, 0, 0};
    hist[tid >> 8][tid & 255] = 0;
    static_assert(SEL_THREADS == 4 * 256, "one histogram word per thread");
    __syncthreads();

    // f(i, valid, bits) over this lane's keys, in position order.  `live`
    // (wave-uniform) skips keys no lane still needs: bit i stands for the
    // lane's i-th key with a register cache, for its i-th group of SEL_BATCH
    // keys without one (all bits set past 64 groups).  Without a cache the
    // keys are loaded SEL_BATCH at a time, all loads in flight together.
    uint64_t live = ~0ull;
    auto each_key = [&](auto&& f) {
      if constexpr (PTC > 0) {
#pragma unroll
        for (int i = 0; i < PTC; ++i)
          if (i < iters && ((live >> i) & 1u)) f(i, e0 + i * WAVE < N, cache[i]);  // wave-uniform
      } else {
        for (int i0 = 0; i0 < iters; i0 += SEL_BATCH) {
          const int grp = i0 / SEL_BATCH;
          if (grp < 64 && !((live >> grp) & 1u)) continue;  // wave-uniform
          uint32_t c[SEL_BATCH];
#pragma unroll
          for (int i = 0; i < SEL_BATCH; ++i) {
            const int e = e0 + (i0 + i) * WAVE;
            c[i] = (i0 + i < iters && e < N) ? s[e] : 0u;
          }
#pragma unroll
          for (int i = 0; i < SEL_BATCH; ++i)
            if (i0 + i < iters) f(i0 + i, e0 + (i0 + i) * WAVE < N, c[i]);
        }
      }
    };
    // the `live` bit of the lane's i-th key
    auto live_bit = [&](int i) -> uint64_t {
      const int b = PTC > 0 ? i : i / SEL_BATCH;
      return b < 64 ? 1ull << b : 0ull;
    };

    // pass 1 (top digit, shared by almost every key): per-(digit, lane % 32)
    // counters keep the lanes of one atomic on distinct words
    {
      int* mysub = sub + (lane & (SEL_SUB - 1));
      each_key([&](int, bool ok, uint32_t u) {
        if (ok) atomicAdd(mysub + (u >> 24) * SEL_SUB, 1);
      });
      __syncthreads();
      const int d = tid >> 2, part = tid & 3;
      const int4* q4 = reinterpret_cast<const int4*>(sub + d * SEL_SUB + part * 8);
      const int4 x = q4[0], y = q4[1];
      const int c = quad_sum((x.x + x.y) + (x.z + x.w) + (y.x + y.y) + (y.z + y.w));
      if (part == 0) hist[0][d] = c;
      __syncthreads();
    }
    int dgt, above;
    pick_digit(hist[0], keep, lane, dgt, above);
    uint32_t prefix = (uint32_t)dgt << 24, pmask = 0xFF000000u;
    int krem = keep - above;

    // passes 2-4: few keys still match, so plain atomics on one histogram
    // per pass (cleared at the start: no clearing between passes)
#pragma unroll
    for (int pass = 1; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint64_t nlive = iters > 64 * SEL_BATCH && PTC == 0 ? ~0ull : 0ull;
      each_key([&](int i, bool ok, uint32_t u) {
        const bool take = ok && (u & pmask) == prefix;
        const uint64_t m = __ballot(take);
        if (m != 0) nlive |= live_bit(i);
        if (take) atomicAdd(&hist[pass][(u >> shift) & 255u], 1);
      });
      live = nlive;
      __syncthreads();
      pick_digit(hist[pass], krem, lane, dgt, above);
      krem -= above;
      prefix |= (uint32_t)dgt << shift;
      pmask |= 255u << shift;
    }
    const uint32_t thr = prefix;
    const int need_eq = krem;  // keys equal to thr that are kept (lowest positions)
    live = ~0ull;

    int n_gt = 0, n_eq = 0;  // wave totals (uniform)
    each_key([&](int, bool ok, uint32_t u) {
      n_gt += __builtin_popcountll(__ballot(ok && u > thr));
      n_eq += __builtin_popcountll(__ballot(ok && u == thr));
    });
    if (lane == 0) {
      wtot[0][wave] = n_gt;
      wtot[1][wave] = n_eq;
    }
    __syncthreads();
    // keys above / equal to thr in earlier waves
    int gb = wave_incl_scan(lane < wave ? wtot[0][lane] : 0);
    int eb = wave_incl_scan(lane < wave ? wtot[1][lane] : 0);
    gb = __builtin_amdgcn_readlane(gb, SEL_WAVES - 1);
    eb = __builtin_amdgcn_readlane(eb, SEL_WAVES - 1);
    each_key([&](int i, bool ok, uint32_t u) {
      const bool gt = ok && u > thr, eq = ok && u == thr;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      if ((mg | me) == 0) return;  // wave-uniform
      const int g_before = gb + lanes_below(mg);
      const int e_before = eb + lanes_below(me);
      if (gt || (eq && e_before < need_eq)) {
        const int slot = g_before + min(e_before, need_eq);
        const int e = e0 + i * WAVE;
        out[slot] = e;
        if constexpr (FUSE) sel[slot] = e;
      }
      gb += __builtin_popcountll(mg);
      eb += __builtin_popcountll(me);
    });
  }

  if constexpr (FUSE) {
    __syncthreads();
    const int vs = args.row_shift;
    const int rb = 16 << vs;  // row bytes
    const int total = budget << vs;
    const int64_t obase = ((int64_t)p * args.hkv + h) * budget * rb;
    const int64_t kbase = ((int64_t)tab.tok0[p] * args.st.kv_tok + (int64_t)h * args.st.kv_head) * args.elt;
    for (int x = tid; x < total; x += SEL_THREADS) {
      const int j = x >> vs, c = x & ((1 << vs) - 1);
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (j < keep) {
        const int64_t src = kbase + (int64_t)sel[j] * args.st.kv_tok * args.elt + c * 16;
        kv = ld16(args.k + src);
        vv = ld16(args.v + src);
      }
      st16(args.k_out + obase + (int64_t)j * rb + c * 16, kv);
      st16(args.v_out + obase + (int64_t)j * rb + c * 16, vv);
    }
  }
}

__global__ void __launch_bounds__(256)
compact_kernel(const CompactArgs args, int row_bytes) {
  const int vpr = row_bytes >> 4;  // 16-byte vectors per row
  const int rows_per_block = 256 / vpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / vpr;
  const int vec = threadIdx.x % vpr;
  if (threadIdx.x >= rows_per_block * vpr || row >= args.rows) return;
  const int per_seq = args.hkv * args.budget;
  const int p = (int)(row / per_seq);
  const int h = (int)(row - (int64_t)p * per_seq) / args.budget;
  const int j = args.idx[row];
  const int64_t dst = row * row_bytes + vec * 16;
  if (j < 0) {
    st16(args.k_out + dst, u32x4{0u, 0u, 0u, 0u});
    st16(args.v_out + dst, u32x4{0u, 0u, 0u, 0u});
    return;
  }
  const int64_t src =
      ((args.tab.tok0[p] + j) * args.st.kv_tok + (int64_t)h * args.st.kv_head) * args.elt + vec * 16;
  const u32x4 kv = ld16(args.k + src);
  const u32x4 vv = ld16(args.v + src);
  st16(args.k_out + dst, kv);
  st16(args.v_out + dst, vv);
}

}  // namespace waits
