// Top-k select for long key ranges (more keys than one workgroup handles
// well): each (sequence, KV head) is cut into chunks of WIDE_CHUNK keys, one
// workgroup each, and the same MSB-first radix select as select_kernel runs
// over five launches that meet in a small workspace.  No launch clears
// memory and no two workgroups write one word: every chunk writes its own
// histograms and counts, and the next launch sums the head's chunks.
//   wide_hist_kernel, digit 0   each chunk's histogram of the top byte;
//   wide_hist_kernel, digit d   (d = 1, 2, 3) sums digit d - 1's chunk
//                               histograms over the head, picks that digit
//                               (every workgroup of the head finds the same),
//                               stores the chunk's count of keys above the
//                               pick, and writes the histogram of digit d of
//                               its keys that match the d picked digits;
//   wide_emit_kernel            picks the last digit the same way (threshold
//                               T, and how many keys equal to T are kept),
//                               then places its kept keys: slot = (kept keys
//                               above T before it) + min(keys equal to T
//                               before it, the T-equal keys kept), the
//                               earlier chunks' part from their stored counts
//                               and last-digit histograms, the own part from
//                               wave ballots; optionally gathers its kept K/V
//                               rows (bit copies).
// Histograms hold 16-bit counts (a chunk has at most 4096 keys) in two
// buffers per chunk: digit d goes to buffer d & 1, so the launch reading
// digit d - 1 writes the other one.
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
constexpr int WIDE_HIST_BYTES = 2 * 256 * 2;           // per chunk: two 256-bin uint16 histograms
constexpr int WIDE_SUM_GROUPS = SEL_THREADS / 128;     // chunk groups of the cross-chunk sum
static_assert(WIDE_CHUNK <= 65535, "16-bit histogram counts");

// Chunks of a key range (an empty one still gets one: its workgroup writes
// the -1 slots and zero rows).
__host__ __device__ constexpr int wide_chunks(int n) {
  return n > 0 ? (n + WIDE_CHUNK - 1) / WIDE_CHUNK : 1;
}

struct WideArgs {
  const float* scores;        // [Hkv, T]
  int32_t* idx;               // this launch's slice [nb, Hkv, budget]
  uint16_t* chist;            // workspace [items][2][256]: each chunk's digit histograms
  int4* above;                // workspace [items]: each chunk's keys above picked digits 0, 1, 2
  int2* state;                // workspace [nb * Hkv][4]: (prefix of the first d picks, keys still to keep)
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
  int p, h, ch, nch, N, keep, c0, item0;  // item0: the work item of the head's chunk 0
  __amdgpu_buffer_rsrc_t rs;  // the head's scores (loads past N read 0)
  int2* state;                // the head's 4 (prefix, keys still to keep) pairs
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
  w.item0 = item - w.ch;
  w.keep = min(args.budget, w.N);
  w.c0 = w.ch * WIDE_CHUNK;
  const float* sc = args.scores + (int64_t)w.h * args.T + tab.tok0[w.p];
  w.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), 0, w.N * 4, BUFFER_RSRC_WORD3);
  w.state = args.state + ((int64_t)w.p * args.hkv + w.h) * 4;
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

// The head's histogram of digit d (buffer d & 1 of every chunk) into tot[256]
// and, with BEFORE, that of the chunks ahead of this one into bef[256].
// Thread t adds bins 2 (t % 128) and 2 (t % 128) + 1 of chunks t / 128 + 8 j
// with range-checked 32-bit loads (chunks past the head read 0, so eight
// loads go out together); red holds the WIDE_SUM_GROUPS partial sums.  Ends
// with a barrier.
template <bool BEFORE>
__device__ __forceinline__ void wide_sum(const WideArgs& args, const WideItem& w, int d, int* tot, int* bef,
                                         int (*red)[2][256]) {
  const int tid = threadIdx.x;
  const int bp = tid & 127, grp = tid >> 7;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      args.chist + (int64_t)w.item0 * (WIDE_HIST_BYTES / 2), 0, w.nch * WIDE_HIST_BYTES, BUFFER_RSRC_WORD3);
  const int off = (d & 1) * 512 + bp * 4;  // bytes: the bin pair inside a chunk's record
  int t0 = 0, t1 = 0, b0 = 0, b1 = 0;
  for (int c = grp; c < w.nch; c += 8 * WIDE_SUM_GROUPS) {
    uint32_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(hr, (c + j * WIDE_SUM_GROUPS) * WIDE_HIST_BYTES + off,
                                                            0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int lo = (int)(x[j] & 0xFFFFu), hi = (int)(x[j] >> 16);
      t0 += lo;
      t1 += hi;
      if constexpr (BEFORE) {
        const bool early = c + j * WIDE_SUM_GROUPS < w.ch;
        b0 += early ? lo : 0;
        b1 += early ? hi : 0;
      }
    }
  }
  red[grp][0][2 * bp] = t0;
  red[grp][0][2 * bp + 1] = t1;
  if constexpr (BEFORE) {
    red[grp][1][2 * bp] = b0;
    red[grp][1][2 * bp + 1] = b1;
  }
  __syncthreads();
  if (tid < 256) {
    int s = 0, sb = 0;
#pragma unroll
    for (int g = 0; g < WIDE_SUM_GROUPS; ++g) {
      s += red[g][0][tid];
      if constexpr (BEFORE) sb += red[g][1][tid];
    }
    tot[tid] = s;
    if constexpr (BEFORE) bef[tid] = sb;
  }
  __syncthreads();
}

__global__ void __launch_bounds__(SEL_THREADS)
wide_hist_kernel(const WideArgs args) {
  __shared__ __attribute__((aligned(16))) int sub[256 * SEL_SUB];
  __shared__ int red[WIDE_SUM_GROUPS][2][256];
  __shared__ int tot[256];
  __shared__ int lhist[256];
  __shared__ int wabove[SEL_WAVES];
  const WideItem w = wide_item(args);
  if (w.keep == w.N) return;  // every key is kept: nothing to select
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = args.digit;
  uint32_t u[WIDE_PER];
  bool ok[WIDE_PER];
  wide_load(w, wave, lane, u, ok);
  uint16_t* mine = args.chist + (int64_t)blockIdx.x * (WIDE_HIST_BYTES / 2) + (d & 1) * 256;
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
    if (part == 0) mine[dd] = (uint16_t)c;
    return;
  }
  // the first d - 1 picks, then digit d - 1 from the head's chunks
  int2 st = make_int2(0, w.keep);
  if (d >= 2) st = w.state[d - 1];
  if (tid < 256) lhist[tid] = 0;
  wide_sum<false>(args, w, d - 1, tot, nullptr, red);
  int dgt, abv;
  pick_digit(tot, st.y, lane, dgt, abv);
  const int dshift = 24 - 8 * (d - 1);                   // digit d - 1's lowest bit
  const uint32_t pmask = d >= 2 ? ~0u << (dshift + 8) : 0u;  // digits before it
  const uint32_t prefix = (uint32_t)st.x | ((uint32_t)dgt << dshift);
  if (w.ch == 0 && tid == 0) w.state[d] = make_int2((int)prefix, st.y - abv);
  // this chunk's keys above the pick (among those matching the earlier
  // picks), and digit d of its keys that match all d picks
  const uint32_t pmask_d = ~0u << dshift;
  int n_above = 0;
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i) {
    const bool in_prev = ok[i] && (u[i] & pmask) == (uint32_t)st.x;
    n_above += __builtin_popcountll(__ballot(in_prev && ((u[i] >> dshift) & 255u) > (uint32_t)dgt));
    if (ok[i] && (u[i] & pmask_d) == prefix) atomicAdd(&lhist[(u[i] >> (dshift - 8)) & 255u], 1);
  }
  if (lane == 0) wabove[wave] = n_above;
  __syncthreads();
  if (tid < 256) mine[tid] = (uint16_t)lhist[tid];
  if (wave == 0) {
    const int a = wave_incl_scan(lane < SEL_WAVES ? wabove[lane] : 0);
    if (lane == SEL_WAVES - 1) reinterpret_cast<int*>(args.above + blockIdx.x)[d - 1] = a;
  }
}

template <bool FUSE>
__global__ void __launch_bounds__(SEL_THREADS)
wide_emit_kernel(const WideArgs args) {
  __shared__ int red[WIDE_SUM_GROUPS][2][256];
  __shared__ int tot[256];
  __shared__ int bef[256];
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
  uint32_t thr = 0;
  int need_eq = 0;
  const bool all = w.keep == w.N;  // every key is kept, at its own position
  if (!all) {
    const int2 st = w.state[3];
    wide_sum<true>(args, w, 3, tot, bef, red);
    int dgt, abv;
    pick_digit(tot, st.y, lane, dgt, abv);
    thr = (uint32_t)st.x | (uint32_t)dgt;
    need_eq = st.y - abv;
    // keys above / equal to thr in the head's earlier chunks: their counts
    // above the first three picks, and their last-digit histograms
    if (wave == 0) {
      const int4* ab = args.above + w.item0;
      int g = 0;
      for (int c = lane; c < w.ch; c += WAVE) {
        const int4 a = ab[c];
        g += a.x + a.y + a.z;
      }
      for (int b = dgt + 1 + lane; b < 256; b += WAVE) g += bef[b];
      g = wave_incl_scan(g);
      if (lane == WAVE - 1) {
        base[0] = g;
        base[1] = bef[dgt];
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
    if (slot >= 0 && slot < w.keep) {  // always so; keeps every store inside the head's rows
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
