// Top-k selection and K/V compaction (WAITS README: the top-k selector of
// "Repository layout" keeps the highest-scoring keys per KV head; the
// introduction's retained key-value pairs are then gathered).
//
// select_kernel: one 1024-thread workgroup per (sequence, KV head).  Scores
// are non-negative fp32, so their bit patterns order like the values; an
// MSB-first radix select (4 digits of 8 bits, LDS histograms) finds the bit
// pattern T of the budget-th largest score and how many of the kept keys
// must equal T.  An ordered pass then keeps every key above T plus the
// lowest-positioned keys equal to T (ties go to the lower position), writing
// positions in ascending order.  Each thread owns a contiguous run of
// positions; runs of up to PTC scores stay in registers across the passes,
// longer runs are re-read (from L2) on every pass.
//
// compact_kernel: one 16-byte vector per thread, rows of K and V copied bit
// for bit; empty slots (-1) are zero-filled.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / WAVE;

// Exclusive prefix sum over the workgroup in thread order; returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int x = lane < SEL_WAVES ? sh[lane] : 0;
    int xi = x;
#pragma unroll
    for (int d = 1; d < SEL_WAVES; d <<= 1) {
      const int y = __shfl_up(xi, d, 64);
      if (lane >= d) xi += y;
    }
    if (lane < SEL_WAVES) sh[lane] = xi - x;
    if (lane == SEL_WAVES - 1) sh[SEL_WAVES] = xi;
  }
  __syncthreads();
  const int out = incl - v + sh[wave];
  total = sh[SEL_WAVES];
  __syncthreads();
  return out;
}

// hist[d] += 1 for every active lane whose value matches; lanes that agree
// with the wave's first candidate digit are counted with one atomic (the
// leading radix digits of similar-magnitude scores are shared by almost all
// keys, so per-lane atomics would serialise on one LDS word).
__device__ __forceinline__ void hist_add(int* hist, bool take, uint32_t d) {
  const uint64_t cand = __ballot(take);
  if (cand == 0) return;
  const int leader = __builtin_ctzll(cand);
  const uint32_t ld = __shfl(d, leader, 64);
  const uint64_t same = __ballot(take && d == ld);
  const int lane = threadIdx.x & 63;
  if (lane == leader) atomicAdd(&hist[ld], __builtin_popcountll(same));
  else if (take && d != ld) atomicAdd(&hist[d], 1);
}

template <int PTC>
__global__ void __launch_bounds__(SEL_THREADS)
select_kernel(const SelectArgs args) {
  __shared__ int hist[256];
  __shared__ int scan_sh[SEL_WAVES + 1];
  __shared__ int pick[2];

  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  const int p = item / args.hkv;
  const int h = item - p * args.hkv;
  const int N = tab.n[p];
  const int budget = args.budget;
  const int keep = min(budget, N);
  const int tid = threadIdx.x;
  int32_t* out = args.idx + ((int64_t)p * args.hkv + h) * budget;
  for (int j = keep + tid; j < budget; j += SEL_THREADS) out[j] = -1;
  if (keep == N) {  // every key is kept
    for (int j = tid; j < N; j += SEL_THREADS) out[j] = j;
    return;
  }
  const uint32_t* s = reinterpret_cast<const uint32_t*>(args.scores + (int64_t)h * args.T + tab.tok0[p]);

  const int per = ((N + SEL_THREADS - 1) / SEL_THREADS + 3) & ~3;  // multiple of 4
  const int beg = min(tid * per, N);
  const int cnt = min(per, N - beg);
  uint32_t cache[PTC > 0 ? PTC : 1];
  // runs start at multiples of 4 scores: 16-byte aligned when the head's row is
  const bool vec_ok = (reinterpret_cast<uintptr_t>(s) & 15u) == 0;
  if constexpr (PTC > 0) {
#pragma unroll
    for (int i = 0; i < PTC; i += 4) {
      if (vec_ok && i + 4 <= cnt) {
        const u32x4 v = ld16(s + beg + i);
        cache[i] = v[0]; cache[i + 1] = v[1]; cache[i + 2] = v[2]; cache[i + 3] = v[3];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) cache[i + e] = (i + e < cnt) ? s[beg + i + e] : 0u;
      }
    }
  }
  auto val = [&](int i) -> uint32_t {
    if constexpr (PTC > 0) return cache[i];
    else return s[beg + i];
  };

  uint32_t prefix = 0, pmask = 0;
  int krem = keep;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    if constexpr (PTC > 0) {
#pragma unroll
      for (int i = 0; i < PTC; ++i) {
        const uint32_t u = cache[i];
        hist_add(hist, i < cnt && (u & pmask) == prefix, (u >> shift) & 255u);
      }
    } else {
      for (int i = 0; i < per; ++i) {  // same trip count in every lane (wave votes)
        const uint32_t u = i < cnt ? val(i) : 0u;
        hist_add(hist, i < cnt && (u & pmask) == prefix, (u >> shift) & 255u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane L holds digits 255-4L .. 252-4L (highest digits first)
      int hv[4], lsum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hv[j] = hist[255 - 4 * tid - j];
        lsum += hv[j];
      }
      int incl = lsum;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (tid >= d) incl += y;
      }
      int above = incl - lsum;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < krem && krem <= above + hv[j]) {
          pick[0] = 255 - 4 * tid - j;
          pick[1] = above;
        }
        above += hv[j];
      }
    }
    __syncthreads();
    const uint32_t dgt = (uint32_t)pick[0];
    krem -= pick[1];
    prefix |= dgt << shift;
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;
  const int need_eq = krem;  // keys equal to thr that are kept (lowest positions)

  int n_gt = 0, n_eq = 0;
  if constexpr (PTC > 0) {
#pragma unroll
    for (int i = 0; i < PTC; ++i) {
      if (i < cnt) {
        n_gt += cache[i] > thr;
        n_eq += cache[i] == thr;
      }
    }
  } else {
    for (int i = 0; i < cnt; ++i) {
      const uint32_t u = val(i);
      n_gt += u > thr;
      n_eq += u == thr;
    }
  }
  int tot;
  const int gt_before = block_exclusive_scan(n_gt, scan_sh, tot);
  const int eq_before = block_exclusive_scan(n_eq, scan_sh, tot);
  int pos = gt_before + min(eq_before, need_eq);
  int eq_rank = eq_before;
  auto emit = [&](int i, uint32_t u) {
    if (u > thr) {
      out[pos++] = beg + i;
    } else if (u == thr) {
      if (eq_rank < need_eq) out[pos++] = beg + i;
      ++eq_rank;
    }
  };
  if constexpr (PTC > 0) {
#pragma unroll
    for (int i = 0; i < PTC; ++i)
      if (i < cnt) emit(i, cache[i]);
  } else {
    for (int i = 0; i < cnt; ++i) emit(i, val(i));
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
