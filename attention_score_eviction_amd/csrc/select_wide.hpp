// Top-k select for long key ranges (more keys than one workgroup handles
// well): each (sequence, KV head) is cut into chunks of WIDE_CHUNK keys, one
// workgroup each, and the same MSB-first radix select as select_kernel runs
// over several launches that meet in a small workspace:
//   wide_zero_kernel        clears the per-(sequence, head) digit histograms;
//   wide_hist_kernel (x4)   digit d: every workgroup replays the picks of
//                           digits < d from the histograms, counts digit d of
//                           its keys that still match, and adds its counts to
//                           the head's histogram (global atomics, 256 words);
//   wide_count_kernel       replays all four picks (threshold T and how many
//                           keys equal to T are kept) and stores its chunk's
//                           count of keys above T and equal to T;
//   wide_emit_kernel        places its kept keys: slot = (kept keys above T
//                           before it) + min(keys equal to T before it, the
//                           T-equal keys kept), the "before" counts coming
//                           from the earlier chunks' counts plus wave ballots;
//                           optionally gathers its kept K/V rows (bit copies).
// Results equal select_kernel's bit for bit (ties to the lower position,
// ascending output, -1 / zero rows past the kept count).
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"
#include "select_compact.hpp"

namespace waits {

constexpr int WIDE_CHUNK = 4096;                       // keys per workgroup
constexpr int WIDE_PER = WIDE_CHUNK / SEL_THREADS;     // keys per lane
constexpr int WIDE_SEG = WIDE_PER * WAVE;              // keys per wave

// Chunks of a key range (an empty one still gets one: its workgroup writes
// the -1 slots and zero rows).
__host__ __device__ constexpr int wide_chunks(int n) {
  return n > 0 ? (n + WIDE_CHUNK - 1) / WIDE_CHUNK : 1;
}

struct WideArgs {
  const float* scores;        // [Hkv, T]
  int32_t* idx;               // this launch's slice [nb, Hkv, budget]
  int* hist;                  // workspace [nb, Hkv, 4, 256]
  int2* counts;               // workspace [items]: (keys above T, keys equal to T) per chunk
  int64_t T;
  int32_t hkv;
  int32_t budget;
  int32_t digit;              // wide_hist_kernel: 0 (top byte) .. 3
  const unsigned char* k;     // gather (wide_emit_kernel<true>)
  const unsigned char* v;
  unsigned char* k_out;       // this launch's slice [nb, Hkv, budget, d]
  unsigned char* v_out;
  Strides st;
  int32_t elt;
  int32_t row_shift;          // log2 of the 16-byte vectors per row
  SeqTable tab;               // first[]: items (head-major, then chunk) of each sequence
};

// Where a workgroup's chunk sits and what it loads.
struct WideItem {
  int p, h, ch, nch, N, keep, c0;
  __amdgpu_buffer_rsrc_t rs;  // the head's scores (loads past N read 0)
  int* hist;                  // the head's 4 x 256 histogram
};

__device__ __forceinline__ WideItem wide_item(const WideArgs& args) {
  WideItem w;
  const SeqTable& tab = args.tab;
  const int item = blockIdx.x;
  w.p = find_seq(tab.first, tab.nb, item);
  const int local = item - tab.first[w.p];
  w.N = tab.n[w.p];
  w.nch = wide_chunks(w.N);
  w.h = local / w.nch;
  w.ch = local - w.h * w.nch;
  w.keep = min(args.budget, w.N);
  w.c0 = w.ch * WIDE_CHUNK;
  const float* sc = args.scores + (int64_t)w.h * args.T + tab.tok0[w.p];
  w.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), 0, w.N * 4, BUFFER_RSRC_WORD3);
  w.hist = args.hist + ((int64_t)w.p * args.hkv + w.h) * 4 * 256;
  return w;
}

// This lane's keys of the chunk (wave w owns [c0 + w * WIDE_SEG, + WIDE_SEG),
// lane l its keys c0 + w * WIDE_SEG + 64 i + l): validity and order keys.
// Range-checked buffer loads (0 past N) keep the loads unconditional, so all
// of a lane's loads are in flight together.
__device__ __forceinline__ void wide_load(const WideItem& w, int wave, int lane, uint32_t* u, bool* ok) {
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i) {
    const int e = w.c0 + wave * WIDE_SEG + i * WAVE + lane;
    ok[i] = e < w.N;
    u[i] = sel_key((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(w.rs, e * 4, 0, 0));
  }
}

// Replays the picks of digits [0, nd) from the head's histograms.
__device__ __forceinline__ void wide_replay(const int* hist, int nd, int keep, int lane,
                                            uint32_t& prefix, uint32_t& pmask, int& krem) {
  prefix = 0;
  pmask = 0;
  krem = keep;
  for (int d = 0; d < nd; ++d) {
    int dgt, above;
    pick_digit(hist + d * 256, krem, lane, dgt, above);
    krem -= above;
    prefix |= (uint32_t)dgt << (24 - 8 * d);
    pmask |= 255u << (24 - 8 * d);
  }
}

__global__ void __launch_bounds__(256)
wide_zero_kernel(int* hist, int64_t words) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < words; i += (int64_t)gridDim.x * 256) hist[i] = 0;
}

__global__ void __launch_bounds__(SEL_THREADS)
wide_hist_kernel(const WideArgs args) {
  __shared__ __attribute__((aligned(16))) int sub[256 * SEL_SUB];
  __shared__ int lhist[256];
  const WideItem w = wide_item(args);
  if (w.keep == w.N) return;  // every key is kept: nothing to select
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = args.digit;
  uint32_t u[WIDE_PER];
  bool ok[WIDE_PER];
  wide_load(w, wave, lane, u, ok);
  uint32_t prefix, pmask;
  int krem;
  wide_replay(w.hist, d, w.keep, lane, prefix, pmask, krem);
  const int shift = 24 - 8 * d;
  if (d == 0) {
    // the top digit is shared by almost every key: per-(digit, lane % 32) words
    for (int i = tid; i < 256 * SEL_SUB / 4; i += SEL_THREADS)
      reinterpret_cast<int4*>(sub)[i] = int4{0, 0, 0, 0};
    __syncthreads();
    int* mysub = sub + (lane & (SEL_SUB - 1));
#pragma unroll
    for (int i = 0; i < WIDE_PER; ++i)
      if (ok[i]) atomicAdd(mysub + (u[i] >> 24) * SEL_SUB, 1);
    __syncthreads();
    const int dd = tid >> 2, part = tid & 3;
    const int4* q4 = reinterpret_cast<const int4*>(sub + dd * SEL_SUB + part * 8);
    const int4 x = q4[0], y = q4[1];
    const int c = quad_sum((x.x + x.y) + (x.z + x.w) + (y.x + y.y) + (y.z + y.w));
    if (part == 0 && c != 0) atomicAdd(w.hist + dd, c);
  } else {
    if (tid < 256) lhist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WIDE_PER; ++i)
      if (ok[i] && (u[i] & pmask) == prefix) atomicAdd(&lhist[(u[i] >> shift) & 255u], 1);
    __syncthreads();
    if (tid < 256 && lhist[tid] != 0) atomicAdd(w.hist + d * 256 + tid, lhist[tid]);
  }
}

__global__ void __launch_bounds__(SEL_THREADS)
wide_count_kernel(const WideArgs args) {
  __shared__ int wtot[2][SEL_WAVES];
  const WideItem w = wide_item(args);
  if (w.keep == w.N) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t u[WIDE_PER];
  bool ok[WIDE_PER];
  wide_load(w, wave, lane, u, ok);
  uint32_t thr, pmask;
  int need_eq;
  wide_replay(w.hist, 4, w.keep, lane, thr, pmask, need_eq);
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i) {
    n_gt += __builtin_popcountll(__ballot(ok[i] && u[i] > thr));
    n_eq += __builtin_popcountll(__ballot(ok[i] && u[i] == thr));
  }
  if (lane == 0) {
    wtot[0][wave] = n_gt;
    wtot[1][wave] = n_eq;
  }
  __syncthreads();
  if (wave == 0) {
    const int g = wave_incl_scan(lane < SEL_WAVES ? wtot[0][lane] : 0);
    const int e = wave_incl_scan(lane < SEL_WAVES ? wtot[1][lane] : 0);
    if (lane == SEL_WAVES - 1) args.counts[blockIdx.x] = make_int2(g, e);
  }
}

template <bool FUSE>
__global__ void __launch_bounds__(SEL_THREADS)
wide_emit_kernel(const WideArgs args) {
  __shared__ int wtot[2][SEL_WAVES];
  __shared__ int base[2];
  __shared__ int slot_of[FUSE ? WIDE_CHUNK : 1];
  __shared__ int pos_of[FUSE ? WIDE_CHUNK : 1];
  __shared__ int nkept;
  const WideItem w = wide_item(args);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int budget = args.budget;
  int32_t* out = args.idx + ((int64_t)w.p * args.hkv + w.h) * budget;
  const int vs = args.row_shift;
  const int rb = 16 << vs;  // row bytes
  const int64_t obase = ((int64_t)w.p * args.hkv + w.h) * budget * rb;
  const int64_t kbase =
      ((int64_t)args.tab.tok0[w.p] * args.st.kv_tok + (int64_t)w.h * args.st.kv_head) * args.elt;

  if (w.ch == 0) {  // slots past the kept count
    for (int j = w.keep + tid; j < budget; j += SEL_THREADS) out[j] = -1;
    if constexpr (FUSE) {
      for (int x = (w.keep << vs) + tid; x < (budget << vs); x += SEL_THREADS) {
        const int j = x >> vs, c = x & ((1 << vs) - 1);
        st16(args.k_out + obase + (int64_t)j * rb + c * 16, u32x4{0u, 0u, 0u, 0u});
        st16(args.v_out + obase + (int64_t)j * rb + c * 16, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }
  if (tid == 0) nkept = 0;

  uint32_t u[WIDE_PER];
  bool ok[WIDE_PER];
  wide_load(w, wave, lane, u, ok);
  uint32_t thr = 0, pmask = 0;
  int need_eq = 0;
  const bool all = w.keep == w.N;  // every key is kept, at its own position
  if (!all) {
    wide_replay(w.hist, 4, w.keep, lane, thr, pmask, need_eq);
    // keys above / equal to thr in the head's earlier chunks
    if (wave == 0) {
      const int2* cnt = args.counts + (blockIdx.x - w.ch);
      int g = 0, e = 0;
      for (int c = lane; c < w.ch; c += WAVE) {
        g += cnt[c].x;
        e += cnt[c].y;
      }
      g = wave_incl_scan(g);
      e = wave_incl_scan(e);
      if (lane == WAVE - 1) {
        base[0] = g;
        base[1] = e;
      }
    }
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < WIDE_PER; ++i) {
      n_gt += __builtin_popcountll(__ballot(ok[i] && u[i] > thr));
      n_eq += __builtin_popcountll(__ballot(ok[i] && u[i] == thr));
    }
    if (lane == 0) {
      wtot[0][wave] = n_gt;
      wtot[1][wave] = n_eq;
    }
  }
  __syncthreads();
  int gb = 0, eb = 0;
  if (!all) {
    gb = wave_incl_scan(lane < wave ? wtot[0][lane] : 0);
    eb = wave_incl_scan(lane < wave ? wtot[1][lane] : 0);
    gb = __builtin_amdgcn_readlane(gb, SEL_WAVES - 1) + base[0];
    eb = __builtin_amdgcn_readlane(eb, SEL_WAVES - 1) + base[1];
  }
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i) {
    const int e = w.c0 + wave * WIDE_SEG + i * WAVE + lane;
    int slot = -1;
    if (all) {
      if (ok[i]) slot = e;
    } else {
      const bool gt = ok[i] && u[i] > thr, eq = ok[i] && u[i] == thr;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const int g_before = gb + lanes_below(mg);
      const int e_before = eb + lanes_below(me);
      if (gt || (eq && e_before < need_eq)) slot = g_before + min(e_before, need_eq);
      gb += __builtin_popcountll(mg);
      eb += __builtin_popcountll(me);
    }
    if (slot >= 0) {
      out[slot] = e;
      if constexpr (FUSE) {
        const int at = atomicAdd(&nkept, 1);
        slot_of[at] = slot;
        pos_of[at] = e;
      }
    }
  }
  if constexpr (FUSE) {
    __syncthreads();
    const int total = nkept << vs;
    for (int x = tid; x < total; x += SEL_THREADS) {
      const int j = x >> vs, c = x & ((1 << vs) - 1);
      const int64_t src = kbase + (int64_t)pos_of[j] * args.st.kv_tok * args.elt + c * 16;
      const int64_t dst = obase + (int64_t)slot_of[j] * rb + c * 16;
      st16(args.k_out + dst, ld16(args.k + src));
      st16(args.v_out + dst, ld16(args.v + src));
    }
  }
}

}  // namespace waits
