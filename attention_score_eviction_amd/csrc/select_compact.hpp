// Top-k selection and K/V compaction (WAITS README: the top-k selector of
// "Repository layout" keeps the highest-scoring keys per KV head; the
// introduction's retained key-value pairs are then gathered).
//
// select_kernel: one 1024-thread workgroup per (sequence, KV head).  Scores
// are non-negative fp32, so their bit patterns order like the values (a
// pattern with the sign bit set, -0 included, counts as +0); an
// MSB-first radix select (4 digits of 8 bits) finds the bit pattern T of the
// budget-th largest score and how many of the kept keys must equal T.  Keys
// above T, then the lowest-positioned keys equal to T (ties go to the lower
// position), are written in ascending position order.
//
// Layout: wave w owns the key segment [w * 64 PTC, (w + 1) * 64 PTC), lane l
// its keys w * 64 PTC + 64 i + l (i < PTC), held in registers for the whole
// select; every load is coalesced and position order is (wave, i, lane)
// order.  Slots at or past N read as score 0.  They follow every real key in
// position order, so they are never kept: a kept key equal to 0 is one of the
// lowest-positioned zeros, and N > budget real keys come first.  That lets
// every pass run over all slots with no bounds test.
//
// Pass 1 (top byte, shared by almost every key): per-(digit, lane % 32)
// counters keep the lanes of one atomic on distinct words, folded into 256
// digit counts.  Pass 2 (second byte): branch-free, keys outside the top-byte
// bucket count into a per-lane spare word.  Pass 3 (third byte): few keys
// still match the 16-bit prefix P; the pass also counts the keys above P and
// marks the (wave-uniform) slot indices holding keys in P, the only ones pass
// 4 and the final counts visit.  Every wave derives the picked digit from
// the histogram itself: one barrier per pass (two for the first).
//
// Output: a key's slot is (#kept keys above T before it) + min(#keys equal
// to T before it, the number of T-equal keys kept), from wave ballots, their
// prefix within the wave and a prefix over the 16 wave totals; no block
// scan, no atomics.
//
// FUSE: the same workgroup then gathers the kept K and V rows (bit copies,
// 16-byte vectors, four per thread in flight; zero rows past the kept
// count), so select and compact are one launch.  Once P is known (after
// pass 3), each lane requests into L2 the K and V rows of one of its keys
// at or above P (kept, or still undecided):
// plain loads whose values are consumed only after the gather, so pass 4,
// the counts and the output run while they are in flight and the gather
// finds most rows in L2.  A lane with several such keys (rare: about one key
// in a hundred is kept) requests one of them.
//
// compact_kernel: one 16-byte vector per thread, rows of K and V copied bit
// for bit; empty slots (-1) are zero-filled.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

// Phase marks for the microbenchmark library, which defines WAITS_SELECT_MARK
// to record a timestamp per phase; empty in the WAITS library.
#ifndef WAITS_SELECT_MARK
#define WAITS_SELECT_MARK(k)
#endif

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;
constexpr int SEL_SUB = 32;          // sub-counters per digit
constexpr int SEL_FUSE_MAX = 8192;   // largest budget the fused gather keeps in LDS

// The order key of a score's bit pattern: non-negative floats order like
// their bit patterns; anything with the sign bit set (-0, and values outside
// the scores' domain) counts as +0.
__device__ __forceinline__ uint32_t sel_key(uint32_t u) { return (int32_t)u < 0 ? 0u : u; }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Row copies of the gather: 16-byte vectors x in [x0, total) stepping by
// `stride`, U per trip with every load issued before the first store (a
// workgroup that keeps many rows would otherwise wait one memory round trip
// per vector).  src(x), dst(x): byte offsets of vector x in K and V and in
// the outputs; src(x) < 0 writes a zero vector.
template <int U, typename SrcF, typename DstF>
__device__ __forceinline__ void gather_vectors(const unsigned char* k, const unsigned char* v,
                                               unsigned char* k_out, unsigned char* v_out, int x0,
                                               int total, int stride, SrcF src, DstF dst) {
  for (int xb = x0; xb < total; xb += U * stride) {
    u32x4 kv[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = xb + u * stride;
      kv[u] = u32x4{0u, 0u, 0u, 0u};
      vv[u] = u32x4{0u, 0u, 0u, 0u};
      if (x < total) {
        const int64_t sx = src(x);
        if (sx >= 0) {
          kv[u] = ld16(k + sx);
          vv[u] = ld16(v + sx);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = xb + u * stride;
      if (x < total) {
        const int64_t dx = dst(x);
        st16(k_out + dx, kv[u]);
        st16(v_out + dx, vv[u]);
      }
    }
  }
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
  static_assert(PTC >= 1 && PTC <= 32, "slot marks are 32-bit masks");
  __shared__ __attribute__((aligned(16))) int sub[256 * SEL_SUB];
  __shared__ int hist[4][256];
  __shared__ int spare[WAVE];
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
  const int vs = args.row_shift;
  const int rb = 16 << vs;  // row bytes
  const int64_t kbase = ((int64_t)tab.tok0[p] * args.st.kv_tok + (int64_t)h * args.st.kv_head) * args.elt;
  const int64_t kv_row = args.st.kv_tok * args.elt;

  uint32_t pfv[4] = {0u, 0u, 0u, 0u};  // L2 requests (values unused)
  WAITS_SELECT_MARK(0);

  if (keep == N) {  // every key is kept
    for (int j = tid; j < N; j += SEL_THREADS) {
      out[j] = j;
      if constexpr (FUSE) sel[j] = j;
    }
  } else {
    // Range-checked buffer loads: a slot at or past N reads 0 without a
    // branch, so the PTC loads issue back to back.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(args.scores + (int64_t)h * args.T + tab.tok0[p]), 0, N * 4, BUFFER_RSRC_WORD3);
    const int e0 = wave * (PTC * WAVE) + lane;  // slot i of this lane: key e0 + 64 i
    uint32_t u[PTC];
#pragma unroll
    for (int i = 0; i < PTC; ++i)
      u[i] = sel_key((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (e0 + i * WAVE) * 4, 0, 0));
    for (int i = tid; i < 256 * SEL_SUB / 4; i += SEL_THREADS)
      reinterpret_cast<int4*>(sub)[i] = int4{0, 0, 0, 0};
    hist[tid >> 8][tid & 255] = 0;
    static_assert(SEL_THREADS == 4 * 256, "one histogram word per thread");
    __syncthreads();
    WAITS_SELECT_MARK(1);

    // pass 1: top byte
    {
      int* mysub = sub + (lane & (SEL_SUB - 1));
#pragma unroll
      for (int i = 0; i < PTC; ++i) atomicAdd(mysub + (u[i] >> 24) * SEL_SUB, 1);
      __syncthreads();
      const int d = tid >> 2, part = tid & 3;
      const int4* q4 = reinterpret_cast<const int4*>(sub + d * SEL_SUB + part * 8);
      const int4 x = q4[0], y = q4[1];
      const int c = quad_sum((x.x + x.y) + (x.z + x.w) + (y.x + y.y) + (y.z + y.w));
      if (part == 0) hist[0][d] = c;
      __syncthreads();
      WAITS_SELECT_MARK(2);
    }
    int dgt, above;
    pick_digit(hist[0], keep, lane, dgt, above);
    int krem = keep - above;
    const uint32_t d1 = (uint32_t)dgt;

    // pass 2: second byte of the keys in the top-byte bucket
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      int* a = (u[i] >> 24) == d1 ? &hist[1][(u[i] >> 16) & 255u] : &spare[lane];
      atomicAdd(a, 1);
    }
    __syncthreads();
    WAITS_SELECT_MARK(3);
    pick_digit(hist[1], krem, lane, dgt, above);
    krem -= above;
    const uint32_t P16 = (d1 << 8) | (uint32_t)dgt;

    // pass 3: third byte of the keys in P16; keys above P16 counted per lane
    int n_hi = 0;
    uint32_t cand = 0;  // bit i: slot i of some lane of this wave holds a key in P16
    int pf = -1;        // a slot of this lane at or above P16
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      const uint32_t t16 = u[i] >> 16;
      n_hi += t16 > P16 ? 1 : 0;
      if constexpr (FUSE) pf = t16 >= P16 ? i : pf;
      const bool in = t16 == P16;
      if (__ballot(in) != 0) {  // wave-uniform
        cand |= 1u << i;
        if (in) atomicAdd(&hist[2][(u[i] >> 8) & 255u], 1);
      }
    }
    cand = __builtin_amdgcn_readfirstlane(cand);  // uniform: keeps the tests below scalar branches
    if constexpr (FUSE) {
      // P16 > 0: slots past N (score 0) are below it, so pf names a real key
      if (P16 != 0 && pf >= 0) {
        const unsigned char* kr = args.k + kbase + (int64_t)(e0 + pf * WAVE) * kv_row;
        const unsigned char* vr = args.v + kbase + (int64_t)(e0 + pf * WAVE) * kv_row;
        const int second = rb > 128 ? 128 : 0;  // the row's second 128-byte line, if any
        pfv[0] = *reinterpret_cast<const uint32_t*>(kr);
        pfv[1] = *reinterpret_cast<const uint32_t*>(kr + second);
        pfv[2] = *reinterpret_cast<const uint32_t*>(vr);
        pfv[3] = *reinterpret_cast<const uint32_t*>(vr + second);
      }
    }
    __syncthreads();
    WAITS_SELECT_MARK(4);
    pick_digit(hist[2], krem, lane, dgt, above);
    krem -= above;
    const uint32_t P24 = (P16 << 8) | (uint32_t)dgt;

    // pass 4: last byte, slots marked in pass 3 only
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      if ((cand >> i) & 1u) {
        asm volatile("");  // keeps this a scalar branch (not merged into the lane test below)
        if ((u[i] >> 8) == P24) atomicAdd(&hist[3][u[i] & 255u], 1);
      }
    }
    __syncthreads();
    WAITS_SELECT_MARK(5);
    pick_digit(hist[3], krem, lane, dgt, above);
    krem -= above;
    const uint32_t thr = (P24 << 8) | (uint32_t)dgt;
    const int need_eq = krem;  // keys equal to thr that are kept (lowest positions)

    // wave totals: keys above thr (above P16, or in P16 and above thr) and equal to thr
    int n_gt = __builtin_amdgcn_readlane(wave_incl_scan(n_hi), WAVE - 1);
    int n_eq = 0;
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      if ((cand >> i) & 1u) {
        asm volatile("");
        n_gt += __builtin_popcountll(__ballot((u[i] >> 16) == P16 && u[i] > thr));
        n_eq += __builtin_popcountll(__ballot(u[i] == thr));
      }
    }
    if (lane == 0) {
      wtot[0][wave] = n_gt;
      wtot[1][wave] = n_eq;
    }
    __syncthreads();
    WAITS_SELECT_MARK(6);
    // keys above / equal to thr in earlier waves
    int gb = wave_incl_scan(lane < wave ? wtot[0][lane] : 0);
    int eb = wave_incl_scan(lane < wave ? wtot[1][lane] : 0);
    gb = __builtin_amdgcn_readlane(gb, SEL_WAVES - 1);
    eb = __builtin_amdgcn_readlane(eb, SEL_WAVES - 1);
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      if (__ballot(u[i] >= thr) == 0) continue;  // wave-uniform
      const bool gt = u[i] > thr, eq = u[i] == thr;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
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
    }
  }

  WAITS_SELECT_MARK(7);
  if constexpr (FUSE) {
    __syncthreads();
    const int total = budget << vs;
    const int64_t obase = ((int64_t)p * args.hkv + h) * budget * rb;
    const int cm = (1 << vs) - 1;
    gather_vectors<4>(
        args.k, args.v, args.k_out, args.v_out, tid, total, SEL_THREADS,
        [&](int x) { return (x >> vs) < keep ? kbase + (int64_t)sel[x >> vs] * kv_row + (x & cm) * 16 : (int64_t)-1; },
        [&](int x) { return obase + (int64_t)(x >> vs) * rb + (x & cm) * 16; });
    // keeps the L2 requests alive; budget >= 1, so nothing is written
    if (budget < 0) out[tid] = (int32_t)(pfv[0] ^ pfv[1] ^ pfv[2] ^ pfv[3]);
    WAITS_SELECT_MARK(8);
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
