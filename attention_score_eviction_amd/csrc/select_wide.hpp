// Top-k select for long key ranges (more keys than one workgroup handles
// well): each (sequence, KV head) is cut into chunks of WIDE_CHUNK keys, one
// workgroup each, and the select runs in two launches that meet in the
// workspace (WAITS README: the top-k selector of "Repository layout"; the
// same order as select_kernel: bit patterns of the non-negative scores, ties
// to the lower position).
//
//   wide_sort_kernel    each chunk counting-sorts its keys by the top 12 bits
//                       of their order key (4096 bins, 1/16 of an octave):
//                       it writes the bins' start offsets (and every 64th of
//                       them again, contiguous) and its keys' order keys in
//                       bin order.  No atomics outside LDS, so the workspace
//                       needs no initial state.
//   wide_place_kernel   every chunk of a head reads all of the head's chunk
//                       records: the counts at or above each 64th bin, then
//                       at or above each bin of the one 64-bin group that
//                       holds the budget-th largest key, give that key's bin
//                       B and how many keys lie above it.  The keys of bin B
//                       (few, as a rule) are read back from the sorted
//                       lists, and three more radix digits over them
//                       (bits 18-11, 10-3, 2-0) give the threshold T and how
//                       many keys equal to T are kept.  Each chunk then
//                       places its own kept keys, slot = (kept keys above T
//                       before it) + min(keys equal to T before it, the
//                       T-equal keys kept), the earlier chunks' part from
//                       their records and bin-B keys, its own from wave
//                       ballots, and optionally gathers their K/V rows.
//
// Every chunk of a head derives the same B and T from the same records.
// Bin B's keys are held in LDS when they fit (WIDE_CACHE); past that (many
// equal or nearly equal scores) each pass reads them again from the
// workspace, which is slower but gives the same result.  For heads of up to
// WIDE_FINE_CHUNKS chunks the bin offsets read in the search stay in LDS and
// give every chunk's bin-B range without another round of loads.
// Results equal select_kernel's bit for bit (ascending output, -1 / zero
// rows past the kept count).
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"
#include "select_compact.hpp"

namespace waits {

constexpr int WIDE_CHUNK = 4096;                       // keys per workgroup
constexpr int WIDE_PER = WIDE_CHUNK / SEL_THREADS;     // keys per lane
constexpr int WIDE_SEG = WIDE_PER * WAVE;              // keys per wave
constexpr int WIDE_BINS = 4096;                        // bins of the 12-bit key prefix
constexpr int WIDE_SHIFT = 19;                         // order keys are 31 bits: prefix = bits 30..19
constexpr int WIDE_GROUP = 64;                         // bins per coarse group
constexpr int WIDE_GROUPS = WIDE_BINS / WIDE_GROUP;
constexpr int WIDE_SUMS = SEL_THREADS / WIDE_GROUP;    // chunk groups of the cross-chunk sums
constexpr int WIDE_MAX_CHUNKS = 1024;                  // chunks of the longest accepted head
constexpr int WIDE_CACHE = 4096;                       // bin-B keys held in LDS
constexpr int WIDE_FINE_CHUNKS = 64;                   // chunks whose searched offsets stay in LDS
constexpr int WIDE_U = 4;                              // chunk records per thread loaded together
// Chunk record: coarse offsets (u32, off[64 j] for j = 0..64), bin offsets
// (u16, off[b] for b = 0..4096; off[4096] = the chunk's key count), order
// keys in bin order (u32).  A bin-B key only adds to its chunk's counts, so
// its position is not kept: each chunk places its own keys from the scores.
constexpr int WREC_COARSE = 0;
constexpr int WREC_OFF = 272;
constexpr int WREC_VAL = WREC_OFF + 2 * 4104;
constexpr int WIDE_REC_BYTES = WREC_VAL + 4 * WIDE_CHUNK;
static_assert(WREC_OFF >= 4 * (WIDE_GROUPS + 1) && WREC_OFF % 16 == 0, "coarse offsets fit");
static_assert(WREC_VAL % 16 == 0 && WIDE_REC_BYTES % 16 == 0, "16-byte aligned record parts");
static_assert(WIDE_CHUNK <= 65535, "16-bit offsets");
static_assert(WIDE_BINS == 4 * SEL_THREADS, "four bins per thread in the chunk's scan");

// Chunks of a key range (an empty one still gets one: its workgroup writes
// the -1 slots and zero rows).
__host__ __device__ constexpr int wide_chunks(int n) {
  return n > 0 ? (n + WIDE_CHUNK - 1) / WIDE_CHUNK : 1;
}

struct WideArgs {
  const float* scores;        // [Hkv, T]
  int32_t* idx;               // this launch's slice [nb, Hkv, budget]
  unsigned char* rec;         // workspace [items][WIDE_REC_BYTES]: each chunk's record
  int64_t T;
  int32_t hkv;
  int32_t budget;
  const unsigned char* k;     // gather (wide_place_kernel<true>)
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
  const float* sc;            // the head's scores
  __amdgpu_buffer_rsrc_t rs;  // the same (loads past N read 0)
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
  w.sc = args.scores + (int64_t)w.h * args.T + tab.tok0[w.p];
  w.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(w.sc), 0, w.N * 4, BUFFER_RSRC_WORD3);
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

// Exclusive prefix of x over the workgroup (thread order) and the total.
// wsum: SEL_WAVES words; starts and ends with a barrier.
__device__ __forceinline__ int block_excl_scan(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  const int incl = wave_incl_scan(x);
  if (lane == WAVE - 1) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < SEL_WAVES; ++k) {
    const int v = wsum[k];
    base += k < wave ? v : 0;
    tot += v;
  }
  total = tot;
  __syncthreads();
  return base + incl - x;
}

__global__ void __launch_bounds__(SEL_THREADS)
wide_sort_kernel(const WideArgs args) {
  __shared__ __attribute__((aligned(16))) int cnt[WIDE_BINS];
  __shared__ int wsum[SEL_WAVES];
  __shared__ __attribute__((aligned(16))) uint32_t sval[WIDE_CHUNK];
  const WideItem w = wide_item(args);
  if (w.keep == w.N) return;  // every key is kept: the place kernel reads no record
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t u[WIDE_PER];
  bool ok[WIDE_PER];
  wide_load(w, wave, lane, u, ok);
  reinterpret_cast<int4*>(cnt)[tid] = int4{0, 0, 0, 0};
  __syncthreads();
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i)
    if (ok[i]) atomicAdd(&cnt[u[i] >> WIDE_SHIFT], 1);
  __syncthreads();
  // bins 4 tid .. 4 tid + 3: their start offsets
  const int4 c4 = reinterpret_cast<const int4*>(cnt)[tid];
  int total;
  const int o0 = block_excl_scan((c4.x + c4.y) + (c4.z + c4.w), wsum, total);
  const int o1 = o0 + c4.x, o2 = o1 + c4.y, o3 = o2 + c4.z;
  unsigned char* rec = args.rec + (int64_t)blockIdx.x * WIDE_REC_BYTES;
  *reinterpret_cast<uint2*>(rec + WREC_OFF + 8 * tid) =
      make_uint2((uint32_t)o0 | ((uint32_t)o1 << 16), (uint32_t)o2 | ((uint32_t)o3 << 16));
  if ((tid & (WIDE_GROUP / 4 - 1)) == 0)
    reinterpret_cast<uint32_t*>(rec + WREC_COARSE)[tid / (WIDE_GROUP / 4)] = (uint32_t)o0;
  if (tid == 0) {
    reinterpret_cast<uint16_t*>(rec + WREC_OFF)[WIDE_BINS] = (uint16_t)total;
    reinterpret_cast<uint32_t*>(rec + WREC_COARSE)[WIDE_GROUPS] = (uint32_t)total;
  }
  // the start offsets become the bins' write cursors
  reinterpret_cast<int4*>(cnt)[tid] = int4{o0, o1, o2, o3};
  __syncthreads();
#pragma unroll
  for (int i = 0; i < WIDE_PER; ++i) {
    if (ok[i]) {
      const int slot = atomicAdd(&cnt[u[i] >> WIDE_SHIFT], 1);
      sval[slot] = u[i];
    }
  }
  __syncthreads();
  // order keys in bin order, 16 bytes per thread (the slots past the key
  // count are never read)
  *reinterpret_cast<u32x4*>(rec + WREC_VAL + 16 * tid) = reinterpret_cast<const u32x4*>(sval)[tid];
}

template <bool FUSE>
__global__ void __launch_bounds__(SEL_THREADS)
wide_place_kernel(const WideArgs args) {
  __shared__ int red[WIDE_SUMS][WIDE_GROUP];
  __shared__ int acnt[WIDE_GROUP];
  __shared__ int ctot[WIDE_MAX_CHUNKS];      // each chunk's key count
  __shared__ int fine[WIDE_FINE_CHUNKS][WIDE_GROUP + 1];  // searched bin offsets (short heads)
  __shared__ int cs0[WIDE_MAX_CHUNKS];       // each chunk's first bin-B slot in its sorted list
  __shared__ int cabove[WIDE_MAX_CHUNKS];    // its keys in bins above B
  __shared__ int cstart[WIDE_MAX_CHUNKS];    // its first bin-B key among the head's
  __shared__ int gtc[WIDE_MAX_CHUNKS];       // its bin-B keys above T
  __shared__ int eqc[WIDE_MAX_CHUNKS];       // its keys equal to T
  __shared__ int hist[3][256];
  __shared__ int wsum[SEL_WAVES];
  __shared__ uint32_t cval[WIDE_CACHE];
  __shared__ uint16_t cchk[WIDE_CACHE];
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
  wide_load(w, wave, lane, u, ok);  // this chunk's keys, in flight during the search
  uint32_t thr = 0;
  int need_eq = 0;
  const bool all = w.keep == w.N;  // every key is kept, at its own position
  if (!all) {
    const int C = w.nch;
    const unsigned char* rec0 = args.rec + (int64_t)w.item0 * WIDE_REC_BYTES;
    auto coarse = [&](int c, int j) {
      return (int)reinterpret_cast<const uint32_t*>(rec0 + (int64_t)c * WIDE_REC_BYTES + WREC_COARSE)[j];
    };
    auto off = [&](int c, int b) {
      return (int)reinterpret_cast<const uint16_t*>(rec0 + (int64_t)c * WIDE_REC_BYTES + WREC_OFF)[b];
    };
    const int j = tid & (WIDE_GROUP - 1), g = tid / WIDE_GROUP;

    // keys of the head at or above bin 64 j (j < 64)
    // (WIDE_U chunks per thread with their loads in flight together)
    {
      int s = 0;
      for (int c0 = g; c0 < C; c0 += WIDE_U * WIDE_SUMS) {
        int tot[WIDE_U], at[WIDE_U];
#pragma unroll
        for (int u = 0; u < WIDE_U; ++u) {
          const int c = c0 + u * WIDE_SUMS;
          tot[u] = c < C ? coarse(c, WIDE_GROUPS) : 0;
          at[u] = c < C ? coarse(c, j) : 0;
        }
#pragma unroll
        for (int u = 0; u < WIDE_U; ++u) {
          const int c = c0 + u * WIDE_SUMS;
          if (c < C) {
            s += tot[u] - at[u];
            if (j == 0) ctot[c] = tot[u];
          }
        }
      }
      red[g][j] = s;
    }
    __syncthreads();
    if (tid < WIDE_GROUP) {
      int s = 0;
#pragma unroll
      for (int k = 0; k < WIDE_SUMS; ++k) s += red[k][tid];
      acnt[tid] = s;
    }
    __syncthreads();
    // the last group whose start has keep or more keys at or above it (group
    // 0 has all N > keep; the counts fall with j, so the lanes that pass are
    // a prefix)
    const int gsel = __builtin_popcountll(__ballot(acnt[lane] >= w.keep)) - 1;
    __syncthreads();
    // keys at or above bin 64 gsel + 1 + j (bin 4096 reads the key count:
    // none); short heads keep the offsets of bins 64 gsel .. 64 gsel + 64
    const bool keep_fine = C <= WIDE_FINE_CHUNKS;
    {
      const int b = WIDE_GROUP * gsel + 1 + j;
      int s = 0;
      for (int c0 = g; c0 < C; c0 += WIDE_U * WIDE_SUMS) {
        int o[WIDE_U], o0[WIDE_U];
#pragma unroll
        for (int u = 0; u < WIDE_U; ++u) {
          const int c = c0 + u * WIDE_SUMS;
          o[u] = c < C ? off(c, b) : 0;
          o0[u] = keep_fine && j == 0 && c < C ? off(c, b - 1) : 0;
        }
#pragma unroll
        for (int u = 0; u < WIDE_U; ++u) {
          const int c = c0 + u * WIDE_SUMS;
          if (c < C) {
            s += ctot[c] - o[u];
            if (keep_fine) {
              fine[c][1 + j] = o[u];
              if (j == 0) fine[c][0] = o0[u];
            }
          }
        }
      }
      red[g][j] = s;
    }
    __syncthreads();
    if (tid < WIDE_GROUP) {
      int s = 0;
#pragma unroll
      for (int k = 0; k < WIDE_SUMS; ++k) s += red[k][tid];
      acnt[tid] = s;
    }
    __syncthreads();
    // bin B: the last bin with keep or more keys at or above it.  Below 64:
    // the last bin of the group has fewer than keep (maximality of gsel, or
    // bin 4096).
    const int nge = __builtin_popcountll(__ballot(acnt[lane] >= w.keep));
    const int B = WIDE_GROUP * gsel + nge;
    const int above = acnt[nge];  // keys in bins above B
    int krem = w.keep - above;    // keys of bin B to keep (>= 1)

    // every chunk's bin-B range, and its keys above bin B
    int len = 0;
    for (int c = tid; c < C; c += SEL_THREADS) {
      const int bb = B - WIDE_GROUP * gsel;  // 0 .. 63
      const int s0 = keep_fine ? fine[c][bb] : off(c, B);
      const int s1 = keep_fine ? fine[c][bb + 1] : off(c, B + 1);
      cs0[c] = s0;
      cabove[c] = ctot[c] - s1;
      gtc[c] = 0;
      eqc[c] = 0;
      len = s1 - s0;  // one chunk per thread: C <= WIDE_MAX_CHUNKS = SEL_THREADS
    }
    static_assert(WIDE_MAX_CHUNKS == SEL_THREADS, "one chunk per thread in the range scan");
    int ncand;
    const int st0 = block_excl_scan(len, wsum, ncand);
    if (tid < C) cstart[tid] = st0;
    for (int x = tid; x < 3 * 256; x += SEL_THREADS) (&hist[0][0])[x] = 0;
    __syncthreads();

    // bin-B key e of the head: its order key and chunk (from LDS once cached)
    const bool cached = ncand <= WIDE_CACHE;
    auto fetch = [&](int e, uint32_t& val, int& c) __attribute__((always_inline)) {
      int lo = 0, hi = C - 1;  // the last chunk whose range starts at or before e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cstart[mid] <= e) lo = mid;
        else hi = mid - 1;
      }
      c = lo;
      val = reinterpret_cast<const uint32_t*>(rec0 + (int64_t)c * WIDE_REC_BYTES + WREC_VAL)
          [cs0[c] + e - cstart[c]];
    };

    // three more digits of the threshold over bin B's keys
    uint32_t P = (uint32_t)B;
    int sh = WIDE_SHIFT;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int dsh = r == 0 ? 11 : (r == 1 ? 3 : 0);
      const uint32_t dmask = r < 2 ? 255u : 7u;
      for (int e = tid; e < ncand; e += SEL_THREADS) {
        uint32_t val;
        int c;
        if (r > 0 && cached) {
          val = cval[e];
          c = cchk[e];
        } else {
          fetch(e, val, c);
          if (r == 0 && cached) {
            cval[e] = val;
            cchk[e] = (uint16_t)c;
          }
        }
        if ((val >> sh) == P) atomicAdd(&hist[r][(val >> dsh) & dmask], 1);
      }
      __syncthreads();
      int dgt, abv;
      pick_digit(hist[r], krem, lane, dgt, abv);
      krem -= abv;
      P = (P << (sh - dsh)) | (uint32_t)dgt;
      sh = dsh;
    }
    thr = P;
    need_eq = krem;

    // bin-B keys above / equal to thr, per chunk
    for (int e = tid; e < ncand; e += SEL_THREADS) {
      uint32_t val;
      int c;
      if (cached) {
        val = cval[e];
        c = cchk[e];
      } else {
        fetch(e, val, c);
      }
      if (val > thr) atomicAdd(&gtc[c], 1);
      else if (val == thr) atomicAdd(&eqc[c], 1);
    }
    __syncthreads();
    // kept keys above / equal to thr in the head's earlier chunks
    if (wave == 0) {
      int gs = 0, es = 0;
      for (int c = lane; c < w.ch; c += WAVE) {
        gs += cabove[c] + gtc[c];
        es += eqc[c];
      }
      gs = wave_incl_scan(gs);
      es = wave_incl_scan(es);
      if (lane == WAVE - 1) {
        base[0] = gs;
        base[1] = es;
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
    // eight vectors per thread in flight: the kept keys can crowd into a few
    // chunks (at a = 0 the first keys hold the largest scores)
    const int cm = (1 << vs) - 1;
    const int64_t kv_row = args.st.kv_tok * args.elt;
    gather_vectors<8>(
        args.k, args.v, args.k_out, args.v_out, tid, total, SEL_THREADS,
        [&](int x) { return kbase + (int64_t)pos_of[x >> vs] * kv_row + (x & cm) * 16; },
        [&](int x) { return obase + (int64_t)slot_of[x >> vs] * rb + (x & cm) * 16; });
  }
}

}  // namespace waits
