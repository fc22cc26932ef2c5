// Host side of the WAITS C ABI (include/waits.h): argument checks, launch
// planning and kernel launches on the caller's stream.  Nothing here
// allocates, synchronises or keeps state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "waits.h"
#include "device_common.hpp"
#include "kernel_args.hpp"
#include "pass1_lse.hpp"
#include "pass2_colsum.hpp"
#include "few_rows.hpp"
#include "few_rows16.hpp"
#include "few_rows_multi.hpp"
#include "key_blocks.hpp"
#include "select_compact.hpp"
#include "select_wide.hpp"
#include "attention.hpp"

// Scratch of waits_select_compact_noalloc (the wide select's per-chunk
// counting-sort records), one copy per GPU for the life of the process.  In host code `scratch` is a host-side stand-in, not a device
// address: kernels get the address hipGetSymbolAddress reports for their
// device (device_scratch below).
constexpr size_t STATIC_SCRATCH_BYTES = WAITS_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

namespace waits {
namespace {

// Tile configuration (stationary 32-row tiles per wave).
constexpr int SW1 = 2;                            // pass 1: 64 query rows per wave
constexpr int SW2 = 2;                            // pass 2: 64 keys per wave
constexpr int WGROWS1 = NWAVES * SW1 * TILE;      // 256 packed rows per workgroup
constexpr int WGKEYS2 = NWAVES * SW2 * TILE;      // 256 keys per workgroup
constexpr int NUM_CU = 256;
constexpr int MAX_SEQ_LEN = (1 << 22) - 1;        // keeps N - b - 0.5 exact in fp32
constexpr int MAX_B = 1 << 22;
constexpr float LIVE_EXP_LIMIT = 89.0f;           // expf overflows above ~88.7228
constexpr int FR_MIN_CHUNK = 256;                 // few-rows: shortest key chunk
constexpr int BIG_MIN_CHUNK = 1024;               // row blocks: shortest pass-1 key chunk
constexpr int KB_MIN_ROWS = 256;                  // key blocks: fewest rows per chunk
constexpr int KB_MAX_CHUNKS = 64;                 // key blocks: most row chunks
constexpr int64_t SPAN_BYTES = int64_t(1) << 30;  // buffer-load span of one chunk (< 2^31)
constexpr int SEL_WIDE_MIN = SEL_THREADS * 32;    // longer key ranges: select over several workgroups
// BIG pass 2 in row blocks while one launch group's partials take at most
// this much workspace (6 GiB: a = 0 with 8 KV heads and G = 4 up to N ~ 160K;
// it also keeps the reduce's per-group item count, sum of Hkv N, within int32)
constexpr int64_t RB_PART_MAX = int64_t(6) << 30;        // one sequence's partials
constexpr int64_t RB_PART_TOTAL = int64_t(6) << 30;      // ... and one launch group's

// Few-rows workgroup shapes: a head takes the smallest that holds its packed
// rows (row blocks of longer heads use the largest).  tiles: 32-row tiles per
// wave; t16: 16-row tiles per wave of the 16x16 MFMA kernel (bf16 heads of one
// row block only), which pads rows to 16 rather than to 256.  Its tiles cost
// more per row than 32-row tiles (twice the MFMA operand reads per flop), so
// it takes a head only while the busiest SIMD runs fewer rows than the
// 512-row shape gives it: at most 7 16-row tiles per SIMD, 448 rows.
struct FrShape {
  int rows, waves, tiles, t16;
};
constexpr FrShape FR_SHAPES[] = {{64, 2, 1, 0},  {128, 4, 1, 0}, {256, 8, 1, 0},
                                 {384, 8, 0, 3}, {448, 8, 0, 4}, {512, 8, 2, 0}};
constexpr int FR_NSHAPES = 6;
constexpr int FR_BIG_SHAPE = FR_NSHAPES - 1;
static_assert(FR_SHAPES[FR_BIG_SHAPE].rows == FR_ROWS, "row blocks use the largest shape");
// Pass 1 of bf16 head_dim 64 runs its row blocks on the one-tile 8-wave shape
// (256 rows): twice the blocks, so a batch needs fewer key splits (and
// partials) for balance, and the shape's own kernel (about 110 VGPRs) fits
// two workgroups per CU.  Measured 5-8% faster than 512-row blocks.  Pass 2
// keeps 512-row blocks: its per-block column sums would double.
constexpr int FR_P1_SHAPE64 = 2;
static_assert(FR_SHAPES[FR_P1_SHAPE64].waves == 8 && FR_SHAPES[FR_P1_SHAPE64].tiles == 1, "shape table");

// The workgroup shape of row blocks (heads of more than FR_ROWS packed rows) in pass 1 or 2.
int row_block_shape(const waits_shape* s, int pass) {
  return pass == 1 && s->head_dim == 64 && s->dtype == WAITS_BF16 ? FR_P1_SHAPE64 : FR_BIG_SHAPE;
}

// How a sequence's two passes run.
enum class Mode {
  NONE,   // no tokens
  FR,     // all packed rows of a KV head in one workgroup: few-rows kernel, both passes
  BIG,    // more rows: pass 1 on the few-rows kernel in row blocks; pass 2 on the same row blocks
          // (reduced in block order), or on key blocks for the longest heads
  WIDE,   // fp32 rows of head_dim 128 (too wide for those register budgets): lse/colsum kernels
};

struct Seq {
  int n = 0, q0 = 0, pr = 0;
  Mode mode = Mode::NONE;
  int rg = 0;                 // WIDE pass 1: row groups per KV head
  int frs = FR_BIG_SHAPE;     // FR / BIG: few-rows workgroup shape (FR_SHAPES index)
  int nrb = 0;                // FR / BIG pass 1: row blocks of that shape's rows
  int nkb = 0;                // BIG pass 2: key blocks of KB_KEYS keys
  int nrc = 1;                // BIG pass 2: row chunks per key block
  bool p2rb = false;          // BIG pass 2 in row blocks (few-rows kernel) instead of key blocks
  int nc = 1, kc = 32;        // key chunks: pass 1 (every mode), pass 2 (FR)
  int64_t tok0 = 0;
  float a = 0.f, c = 0.f;
};

bool is_aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elt_bytes(int dtype) { return dtype == WAITS_BF16 ? 2 : 4; }

int check_shape(const waits_shape* s, bool need_q) {
  if (!s || !s->cu_seqlens || s->batch < 1) return WAITS_EINVAL;
  if (s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads) return WAITS_EINVAL;
  if (s->cu_seqlens[0] != 0) return WAITS_EINVAL;
  for (int i = 0; i < s->batch; ++i) {
    const int64_t n = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    if (n < 0 || n > MAX_SEQ_LEN) return WAITS_EINVAL;
  }
  if (s->dtype != WAITS_BF16 && s->dtype != WAITS_F32) return WAITS_EINVAL;
  if (s->head_dim < 1) return WAITS_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return WAITS_EUNSUPPORTED;
  const int64_t e = elt_bytes(s->dtype);
  if (s->kv_stride_tok < 0 || s->kv_stride_head < 0) return WAITS_EINVAL;
  if ((s->kv_stride_tok * e) % 16 || (s->kv_stride_head * e) % 16) return WAITS_EINVAL;
  if (need_q) {
    if (s->q_stride_tok < 0 || s->q_stride_head < 0) return WAITS_EINVAL;
    if ((s->q_stride_tok * e) % 16 || (s->q_stride_head * e) % 16) return WAITS_EINVAL;
    if (!(std::isfinite(s->scale) && s->scale > 0.f)) return WAITS_EINVAL;
    if (s->pass2 != WAITS_PASS2_AUTO && s->pass2 != WAITS_PASS2_KEY_BLOCKS) return WAITS_EINVAL;
  }
  return WAITS_OK;
}

int check_curves(const waits_shape* s, const float* a, const int32_t* b) {
  if (!a || !b) return WAITS_EINVAL;
  for (int i = 0; i < s->batch; ++i) {
    if (std::isnan(a[i]) || a[i] < 0.f) return WAITS_EINVAL;
    if (b[i] < 1 || b[i] > MAX_B) return WAITS_EINVAL;
  }
  return WAITS_OK;
}

// First row whose fp32 weight can be nonzero.  w = 1 / (1 + expf(a (c - q)))
// is exactly 0 only where expf overflows, i.e. a (c - q) > 88.72..; rows are
// kept from the first q with a (c - q) <= 89 (fp32 product, as on the
// device), so every row left out has an fp32 weight of exactly 0 whatever the
// last-ulp behaviour of expf.  Row N - 1 always has w >= 1/2.
int first_live_row(int n, float a, int32_t b) {
  if (n <= 0) return 0;
  const float c = (float)n - (float)b - 0.5f;
  auto dead = [&](int q) { return a * (c - (float)q) > LIVE_EXP_LIMIT; };
  if (a == 0.f) return 0;
  int q;
  if (std::isinf(a)) {
    q = std::max(0, (int)std::ceil((double)c));
  } else {
    const double est = (double)c - (double)LIVE_EXP_LIMIT / (double)a;
    q = (int)std::max(0.0, std::min((double)n - 1, std::floor(est) - 2.0));
  }
  while (q > 0 && !dead(q - 1)) --q;
  while (q < n - 1 && dead(q)) ++q;
  return std::min(q, n - 1);
}

int round32(int x) { return (x + 31) / 32 * 32; }

int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

// Bytes from the first to the last byte of one token's rows of a query-head
// group (the key-block kernel addresses a chunk of queries of all G heads
// from one buffer base).
int64_t group_span(const waits_shape* s) {
  const int64_t e = elt_bytes(s->dtype);
  const int G = s->n_q_heads / s->n_kv_heads;
  return ((int64_t)(G - 1) * s->q_stride_head + s->head_dim) * e;
}

// Launch plan of pass 1 or pass 2.  A sequence whose packed rows fit one
// workgroup per KV head runs both passes on the few-rows kernel, its key
// range cut into chunks until the batch has about one workgroup per compute
// unit.  A longer one runs pass 1 on the same kernel in row blocks (512 rows;
// 256 for bf16 head_dim 64) with key chunks for balance.  Its pass 2 runs on
// 512-row blocks with key chunks planned the same way, each block writing its
// column sums for a fixed-order reduce, while the partials stay under
// RB_PART_MAX per sequence and RB_PART_TOTAL per launch group; other long
// sequences run pass 2 on key blocks (row chunks for balance), whose partials
// are [row chunk][Hkv][T].  Every chunk a buffer load
// addresses spans less than 2^31 bytes.
std::vector<Seq> plan_seqs(const waits_shape* s, const float* a, const int32_t* b, int pass) {
  const int G = s->n_q_heads / s->n_kv_heads;
  const int hkv = s->n_kv_heads;
  const bool fr_ok = !(s->dtype == WAITS_F32 && s->head_dim == 128);
  const int64_t krow = std::max<int64_t>(1, s->kv_stride_tok * elt_bytes(s->dtype));
  const int64_t qrow = std::max<int64_t>(1, s->q_stride_tok * elt_bytes(s->dtype));
  std::vector<Seq> v(s->batch);
  int64_t fr_units = 0, big_units1 = 0, big_units2 = 0, big_waves = 0, wide_rg = 0;
  for (int i = 0; i < s->batch; ++i) {
    Seq& q = v[i];
    q.n = (int)(s->cu_seqlens[i + 1] - s->cu_seqlens[i]);
    q.tok0 = s->cu_seqlens[i];
    q.a = a ? a[i] : 0.f;
    q.c = (float)q.n - (float)(b ? b[i] : 1) - 0.5f;
    q.q0 = a ? first_live_row(q.n, a[i], b[i]) : 0;
    q.pr = G * (q.n - q.q0);
    q.nc = 1;
    q.kc = std::max(32, round32(q.n));
    if (q.n == 0) {
      q.mode = Mode::NONE;
    } else if (!fr_ok) {
      q.mode = Mode::WIDE;
      q.rg = (q.pr + WGROWS1 - 1) / WGROWS1;
      wide_rg += (int64_t)hkv * q.rg;
    } else if (q.pr <= FR_ROWS) {
      q.mode = Mode::FR;
      q.nrb = 1;
      q.frs = 0;
      while (FR_SHAPES[q.frs].rows < q.pr || (FR_SHAPES[q.frs].t16 > 0 && s->dtype != WAITS_BF16))
        ++q.frs;
      fr_units += (int64_t)hkv * FR_SHAPES[q.frs].waves;
    } else {
      q.mode = Mode::BIG;
      q.frs = row_block_shape(s, pass);
      q.nrb = (q.pr + FR_SHAPES[q.frs].rows - 1) / FR_SHAPES[q.frs].rows;
      q.nkb = (q.n + KB_KEYS - 1) / KB_KEYS;
      big_units1 += (int64_t)hkv * q.nrb;
      big_units2 += (int64_t)hkv * q.nkb;
      big_waves += (int64_t)hkv * q.nrb * FR_SHAPES[q.frs].waves;
    }
  }
  for (Seq& q : v) {
    if (q.mode == Mode::FR) {
      // about 8 waves per compute unit over the batch's few-rows workgroups;
      // in pass 1 of a bf16 batch the row blocks share the launch and count
      // too, since a key split there costs the lse combine (pass 2's key
      // chunks need no reduce; fp32 shapes launch one after another)
      const int64_t busy = fr_units + (pass == 1 && s->dtype == WAITS_BF16 ? big_waves : 0);
      const int64_t want = std::max<int64_t>(1, ceil_div(8 * NUM_CU, busy));
      int64_t nc = std::max<int64_t>(1, std::min<int64_t>(want, ceil_div(q.n, FR_MIN_CHUNK)));
      nc = std::max(nc, ceil_div(q.n * krow, SPAN_BYTES));
      q.kc = round32((int)ceil_div(q.n, nc));
      q.nc = (q.n + q.kc - 1) / q.kc;
    } else if (q.mode == Mode::BIG) {
      // pass 1: key chunks of each row block (sized in the kernel)
      const int64_t want1 = std::max<int64_t>(1, ceil_div(4 * NUM_CU, big_units1));
      int64_t nc = std::max<int64_t>(1, std::min<int64_t>(want1, ceil_div(q.n, BIG_MIN_CHUNK)));
      q.nc = (int)std::max(nc, ceil_div(q.n * krow, SPAN_BYTES));
      q.kc = 0;
      // pass 2: row chunks of each key block
      const int64_t want2 = std::max<int64_t>(1, ceil_div(8 * NUM_CU, big_units2));
      int64_t nrc = std::min<int64_t>({want2, KB_MAX_CHUNKS, ceil_div(q.pr, KB_MIN_ROWS)});
      nrc = std::max<int64_t>(1, nrc);
      // each chunk's Q rows span less than 2^30 bytes (wider groups are refused in run_colsum)
      const int64_t room = SPAN_BYTES - group_span(s);
      if (room > 0) nrc = std::max(nrc, ceil_div((q.n - q.q0 + 1) * qrow, room));
      q.nrc = (int)nrc;
    }
  }
  if (wide_rg > 0 && wide_rg < 2 * NUM_CU) {
    const int want = (int)((4 * NUM_CU + wide_rg - 1) / wide_rg);
    for (Seq& q : v) {
      if (q.mode != Mode::WIDE) continue;
      const int nc = std::max(1, std::min(want, (q.n + 511) / 512));
      q.kc = round32((q.n + nc - 1) / nc);
      q.nc = (q.n + q.kc - 1) / q.kc;
    }
  }
  // BIG pass 2 on the pass-1 row blocks and key chunks, each block writing its
  // column sums for a reduce in block order, while the partials stay small
  // (per sequence, and summed over a launch group, in sequence order); the
  // other BIG sequences run pass 2 on key blocks, and so do all of them when
  // the caller asks for the key-block plan.
  const bool rb_ok = s->pass2 == WAITS_PASS2_AUTO;
  for (int lo = 0; rb_ok && lo < s->batch; lo += MAXB) {
    int64_t total = 0;
    for (int i = lo; i < std::min(s->batch, lo + MAXB); ++i) {
      Seq& q = v[i];
      if (q.mode != Mode::BIG) continue;
      const int64_t bytes = (int64_t)q.nrb * hkv * q.n * (int64_t)sizeof(float);
      q.p2rb = bytes <= RB_PART_MAX && total + bytes <= RB_PART_TOTAL;
      if (q.p2rb) total += bytes;
    }
  }
  return v;
}

// Pass-1 packed-row pitch of a sequence's partials (per KV head).
int partial_rows(const Seq& q) {
  return q.mode == Mode::WIDE ? q.rg * WGROWS1 : q.nrb * FR_SHAPES[q.frs].rows;
}

// Partial (float2) slots pass 1 needs for sequences [lo, hi).
int64_t partial_slots(const waits_shape* s, const std::vector<Seq>& v, int lo, int hi) {
  int64_t tot = 0;
  for (int i = lo; i < hi; ++i)
    if (v[i].nc > 1) tot += (int64_t)s->n_kv_heads * partial_rows(v[i]) * v[i].nc;
  return tot;
}

size_t lse_ws_bytes(const waits_shape* s, const std::vector<Seq>& v) {
  int64_t mx = 0;
  for (int lo = 0; lo < s->batch; lo += MAXB)
    mx = std::max(mx, partial_slots(s, v, lo, std::min(s->batch, lo + MAXB)));
  return (size_t)mx * sizeof(float2);
}

// Pass-2 partial sums.  Key blocks: [row chunk][Hkv][T] fp32 for the
// most-split sequence.  Then, from a 256-byte boundary, row blocks: per
// launch group, [row block][Hkv][N] fp32 per sequence, back to back.
size_t kb_part_bytes(const waits_shape* s, const std::vector<Seq>& v) {
  int mx = 0;
  for (const Seq& q : v)
    if (q.mode == Mode::BIG && !q.p2rb && q.nrc > 1) mx = std::max(mx, q.nrc);
  const size_t bytes = (size_t)mx * s->n_kv_heads * (size_t)s->cu_seqlens[s->batch] * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

int64_t rb_part_floats(const std::vector<Seq>& v, int lo, int hi, int hkv) {
  int64_t n = 0;
  for (int i = lo; i < hi; ++i)
    if (v[i].mode == Mode::BIG && v[i].p2rb) n += (int64_t)v[i].nrb * hkv * v[i].n;
  return n;
}

size_t colsum_ws_bytes(const waits_shape* s, const std::vector<Seq>& v) {
  int64_t rb = 0;
  for (int lo = 0; lo < s->batch; lo += MAXB)
    rb = std::max(rb, rb_part_floats(v, lo, std::min(s->batch, lo + MAXB), s->n_kv_heads));
  return kb_part_bytes(s, v) + (size_t)rb * sizeof(float);
}

size_t lse_buffer_bytes(const waits_shape* s) {
  const size_t bytes = (size_t)s->n_q_heads * (size_t)s->cu_seqlens[s->batch] * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

void fill_table(SeqTable& t, const std::vector<Seq>& v, int lo, int hi, int hkv) {
  std::memset(&t, 0, sizeof(t));
  t.nb = hi - lo;
  for (int i = lo; i < hi; ++i) {
    const Seq& q = v[i];
    const int j = i - lo;
    t.n[j] = q.n;
    t.q0[j] = q.q0;
    t.rg[j] = q.rg;
    t.nrb[j] = q.nrb;
    t.nc[j] = q.nc;
    t.kc[j] = q.kc;
    t.prow[j] = partial_rows(q);
    t.a[j] = q.a;
    t.c[j] = q.c;
    t.tok0[j] = q.tok0;
  }
  int64_t ws0 = 0;
  for (int i = lo; i < hi; ++i) {
    t.ws0[i - lo] = ws0;
    if (v[i].nc > 1) ws0 += (int64_t)hkv * partial_rows(v[i]) * v[i].nc;
  }
}

Strides strides_of(const waits_shape* s) {
  return Strides{s->q_stride_tok, s->q_stride_head, s->kv_stride_tok, s->kv_stride_head};
}

int launched() { return hipGetLastError() == hipSuccess ? WAITS_OK : WAITS_EDEVICE; }

template <typename T, int D>
void launch_lse(const LseArgs& args, int items, hipStream_t st) {
  hipLaunchKernelGGL((lse_kernel<T, D, SW1>), dim3(items), dim3(NTHREADS), 0, st, args);
}

template <typename T, int D>
void launch_colsum(const ColsumArgs& args, int items, hipStream_t st) {
  hipLaunchKernelGGL((colsum_kernel<T, D, SW2>), dim3(items), dim3(NTHREADS), 0, st, args);
}

template <bool PASS2, typename T, int D, int W, int TW>
void launch_fr(const FrArgs& args, int items, hipStream_t st) {
  hipLaunchKernelGGL((few_rows_kernel<T, D, PASS2, W, TW>), dim3(items), dim3(W * WAVE), 0, st, args);
}

template <bool PASS2, int W, int TW>
void dispatch_fr_shape(const waits_shape* s, const FrArgs& args, int items, hipStream_t st) {
  if (s->dtype == WAITS_BF16) {
    if (s->head_dim == 64) launch_fr<PASS2, bf16_t, 64, W, TW>(args, items, st);
    else launch_fr<PASS2, bf16_t, 128, W, TW>(args, items, st);
  } else {
    launch_fr<PASS2, float, 64, W, TW>(args, items, st);  // fp32 only at head_dim 64 (see plan_seqs)
  }
}

template <bool PASS2, int NT>
void dispatch_fr16(const waits_shape* s, const FrArgs& args, int items, hipStream_t st) {
  if (s->head_dim == 64)
    hipLaunchKernelGGL((few_rows16_kernel<64, PASS2, NT>), dim3(items), dim3(8 * WAVE), 0, st, args);
  else
    hipLaunchKernelGGL((few_rows16_kernel<128, PASS2, NT>), dim3(items), dim3(8 * WAVE), 0, st, args);
}

template <bool PASS2>
void dispatch_fr(const waits_shape* s, const FrArgs& args, int items, int shape, hipStream_t st) {
  static_assert(FR_SHAPES[0].waves == 2 && FR_SHAPES[0].tiles == 1, "shape table");
  static_assert(FR_SHAPES[1].waves == 4 && FR_SHAPES[1].tiles == 1, "shape table");
  static_assert(FR_SHAPES[2].waves == 8 && FR_SHAPES[2].tiles == 1, "shape table");
  static_assert(FR_SHAPES[3].waves == 8 && FR_SHAPES[3].t16 == 3 && FR_SHAPES[3].rows == 8 * 3 * 16,
                "shape table");
  static_assert(FR_SHAPES[4].waves == 8 && FR_SHAPES[4].t16 == 4 && FR_SHAPES[4].rows > 8 * 3 * 16 &&
                    FR_SHAPES[4].rows <= 8 * 4 * 16,
                "shape table");
  static_assert(FR_SHAPES[5].waves == 8 && FR_SHAPES[5].tiles == 2, "shape table");
  switch (shape) {
    case 0: dispatch_fr_shape<PASS2, 2, 1>(s, args, items, st); break;
    case 1: dispatch_fr_shape<PASS2, 4, 1>(s, args, items, st); break;
    case 2: dispatch_fr_shape<PASS2, 8, 1>(s, args, items, st); break;
    case 3: dispatch_fr16<PASS2, 3>(s, args, items, st); break;
    case 4: dispatch_fr16<PASS2, 4>(s, args, items, st); break;
    default: dispatch_fr_shape<PASS2, 8, 2>(s, args, items, st); break;
  }
}

static_assert(FR_MULTI_SHAPES == FR_NSHAPES, "one launch segment per shape");
static_assert(sizeof(FrMultiArgs) <= 4096, "kernel argument segment");

// The few-rows launches of one pass: items[sh] work items on shape sh,
// firsts[sh] the first item of each sequence among them.  Heads of several
// shapes in a bf16 batch go into one few_rows_multi_kernel launch;
// otherwise each shape has its own launch.
template <bool PASS2>
int launch_fr_shapes(const waits_shape* s, const FrArgs& f, const int* items,
                     const int32_t (*firsts)[MAXB + 1], int rb_shape, hipStream_t st) {
  int active = 0;
  for (int sh = 0; sh < FR_NSHAPES; ++sh) active += items[sh] > 0 ? 1 : 0;
  if (s->dtype == WAITS_BF16 && active > 1) {
    FrMultiArgs m;
    std::memset(&m, 0, sizeof(m));
    m.f = f;
    int at = 0;
    // few-rows heads first (largest shape first), the row blocks (shape
    // rb_shape) last: a sequence's row blocks run longest first, so the grid
    // ends on the shortest items (1-2% faster than row blocks first on the
    // 1B batch)
    int order[FR_NSHAPES], no = 0;
    for (int sh = FR_NSHAPES - 1; sh >= 0; --sh)
      if (sh != rb_shape) order[no++] = sh;
    order[no++] = rb_shape;
    for (int o = 0; o < FR_NSHAPES; ++o) {
      const int sh = order[o];
      m.begin[sh] = at;
      at += items[sh];
      m.end[sh] = at;
      std::memcpy(m.first[sh], firsts[sh], sizeof(m.first[sh]));
    }
    if (s->head_dim == 64)
      hipLaunchKernelGGL((few_rows_multi_kernel<64, PASS2>), dim3(at), dim3(8 * WAVE), 0, st, m);
    else
      hipLaunchKernelGGL((few_rows_multi_kernel<128, PASS2>), dim3(at), dim3(8 * WAVE), 0, st, m);
    return launched();
  }
  for (int sh = 0; sh < FR_NSHAPES; ++sh) {
    if (items[sh] == 0) continue;
    FrArgs g = f;
    std::memcpy(g.tab.first, firsts[sh], sizeof(g.tab.first));
    dispatch_fr<PASS2>(s, g, items[sh], sh, st);
    if (launched() != WAITS_OK) return WAITS_EDEVICE;
  }
  return WAITS_OK;
}

FrArgs fr_args(const waits_shape* s, const void* q, const void* k) {
  FrArgs f;
  std::memset(&f, 0, sizeof(f));
  f.q = q;
  f.k = k;
  f.st = strides_of(s);
  f.T = s->cu_seqlens[s->batch];
  f.G = s->n_q_heads / s->n_kv_heads;
  f.hkv = s->n_kv_heads;
  f.scale = s->scale;
  f.scale_log2 = s->scale * LOG2E;
  return f;
}

int run_lse(const waits_shape* s, const void* q, const void* k, const float* a, const int32_t* b,
            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  const std::vector<Seq> v = plan_seqs(s, a, b, 1);
  const size_t need = lse_ws_bytes(s, v);  // (max, sum) float2 partials
  if (ws_bytes < need || (need > 0 && (!ws || !is_aligned(ws, 8)))) return WAITS_EWORKSPACE;
  const int G = s->n_q_heads / s->n_kv_heads;
  const int hkv = s->n_kv_heads;
  for (int lo = 0; lo < s->batch; lo += MAXB) {
    const int hi = std::min(s->batch, lo + MAXB);
    SeqTable tab;
    fill_table(tab, v, lo, hi, hkv);

    // few-rows kernel: the heads of every workgroup shape
    {
      FrArgs f = fr_args(s, q, k);
      f.lse = lse;
      f.part = static_cast<float2*>(ws);
      f.tab = tab;
      int items[FR_NSHAPES] = {};
      int32_t firsts[FR_NSHAPES][MAXB + 1] = {};
      for (int shape = 0; shape < FR_NSHAPES; ++shape) {
        for (int i = lo; i < hi; ++i) {
          firsts[shape][i - lo] = items[shape];
          if ((v[i].mode == Mode::FR || v[i].mode == Mode::BIG) && v[i].frs == shape)
            items[shape] += hkv * v[i].nrb * v[i].nc;
        }
        firsts[shape][hi - lo] = items[shape];
      }
      if (launch_fr_shapes<false>(s, f, items, firsts, row_block_shape(s, 1), stream) != WAITS_OK)
        return WAITS_EDEVICE;
    }

    // fp32 rows of head_dim 128
    LseArgs args;
    args.q = q;
    args.k = k;
    args.lse = lse;
    args.part = static_cast<float2*>(ws);
    args.st = strides_of(s);
    args.T = s->cu_seqlens[s->batch];
    args.G = G;
    args.hkv = hkv;
    args.scale = s->scale;
    args.scale_log2 = s->scale * LOG2E;
    args.tab = tab;
    int items = 0;
    for (int i = lo; i < hi; ++i) {
      args.tab.first[i - lo] = items;
      if (v[i].mode == Mode::WIDE) items += hkv * v[i].rg * v[i].nc;
    }
    args.tab.first[hi - lo] = items;
    if (items > 0) {
      launch_lse<float, 128>(args, items, stream);
      if (launched() != WAITS_OK) return WAITS_EDEVICE;
    }

    // merge split key ranges
    CombineArgs cargs;
    cargs.lse = lse;
    cargs.part = static_cast<const float2*>(ws);
    cargs.T = args.T;
    cargs.G = G;
    cargs.hkv = hkv;
    cargs.tab = tab;
    // a team of lanes per row, sized to the sequence's chunk count; every
    // sequence's threads start on a wave boundary (one lane per row if the
    // teams would not fit the 32-bit thread index)
    auto plan_combine = [&](bool teams) {
      int64_t threads = 0;
      for (int i = lo; i < hi; ++i) {
        int team = 1;
        while (teams && team < 64 && team < v[i].nc / 2) team *= 2;
        cargs.team[i - lo] = team;
        cargs.tab.first[i - lo] = (int32_t)std::min<int64_t>(threads, INT32_MAX);
        if (v[i].nc > 1) threads += ((int64_t)hkv * v[i].pr * team + WAVE - 1) / WAVE * WAVE;
      }
      cargs.tab.first[hi - lo] = (int32_t)std::min<int64_t>(threads, INT32_MAX);
      return threads;
    };
    int64_t threads = plan_combine(true);
    if (threads > INT32_MAX) threads = plan_combine(false);
    for (int i = lo; i < hi; ++i) {
      // the few-rows kernel writes every (row, chunk) partial; the lse kernel
      // only the chunks a row reaches
      if (v[i].mode != Mode::WIDE) cargs.tab.kc[i - lo] = 0;
    }
    if (threads > 0) {
      hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                         stream, cargs);
      if (launched() != WAITS_OK) return WAITS_EDEVICE;
    }
  }
  return WAITS_OK;
}

int run_colsum(const waits_shape* s, const void* q, const void* k, const float* lse,
               const float* a, const int32_t* b, float* scores, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  const std::vector<Seq> v = plan_seqs(s, a, b, 2);
  // only the key-block kernel addresses a group's Q rows from one buffer base
  for (const Seq& sq : v)
    if (sq.mode == Mode::BIG && !sq.p2rb && group_span(s) > SPAN_BYTES / 2) return WAITS_EUNSUPPORTED;
  const size_t need = colsum_ws_bytes(s, v);
  if (ws_bytes < need || (need > 0 && (!ws || !is_aligned(ws, 4)))) return WAITS_EWORKSPACE;
  const int G = s->n_q_heads / s->n_kv_heads;
  const int hkv = s->n_kv_heads;
  float* cpart = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + kb_part_bytes(s, v));
  for (int lo = 0; lo < s->batch; lo += MAXB) {
    const int hi = std::min(s->batch, lo + MAXB);
    SeqTable tab;
    fill_table(tab, v, lo, hi, hkv);
    // row-block partials of this launch group, sequence by sequence
    SeqTable rbtab = tab;
    int64_t rb_off = 0;
    for (int i = lo; i < hi; ++i) {
      rbtab.ws0[i - lo] = rb_off;
      if (v[i].mode == Mode::BIG && v[i].p2rb) rb_off += (int64_t)v[i].nrb * hkv * v[i].n;
    }

    // few-rows sequences, and the row blocks of longer ones, on every workgroup shape
    {
      FrArgs f = fr_args(s, q, k);
      f.lse = const_cast<float*>(lse);
      f.scores = scores;
      f.cpart = cpart;
      f.tab = rbtab;
      int items[FR_NSHAPES] = {};
      int32_t firsts[FR_NSHAPES][MAXB + 1] = {};
      for (int shape = 0; shape < FR_NSHAPES; ++shape) {
        for (int i = lo; i < hi; ++i) {
          firsts[shape][i - lo] = items[shape];
          if (v[i].frs != shape) continue;
          if (v[i].mode == Mode::FR) items[shape] += hkv * v[i].nc;
          else if (v[i].mode == Mode::BIG && v[i].p2rb) items[shape] += hkv * v[i].nrb * v[i].nc;
        }
        firsts[shape][hi - lo] = items[shape];
      }
      if (launch_fr_shapes<true>(s, f, items, firsts, row_block_shape(s, 2), stream) != WAITS_OK)
        return WAITS_EDEVICE;
    }
    {
      RowBlockReduceArgs ra;
      ra.cpart = cpart;
      ra.scores = scores;
      ra.T = s->cu_seqlens[s->batch];
      ra.hkv = hkv;
      ra.G = G;
      ra.rows = FR_ROWS;
      ra.tab = rbtab;
      int items = 0;
      for (int i = lo; i < hi; ++i) {
        ra.tab.first[i - lo] = items;
        if (v[i].mode == Mode::BIG && v[i].p2rb) items += hkv * v[i].n;
      }
      ra.tab.first[hi - lo] = items;
      if (items > 0) {
        hipLaunchKernelGGL(rowblock_reduce_kernel, dim3((items + 255) / 256), dim3(256), 0, stream, ra);
        if (launched() != WAITS_OK) return WAITS_EDEVICE;
      }
    }

    // key blocks of the longer sequences
    BlockArgs kbargs;
    kbargs.q = q;
    kbargs.k = k;
    kbargs.lse = lse;
    kbargs.scores = scores;
    kbargs.part = static_cast<float*>(ws);
    kbargs.st = strides_of(s);
    kbargs.T = s->cu_seqlens[s->batch];
    kbargs.G = G;
    kbargs.hkv = hkv;
    kbargs.scale_log2 = s->scale * LOG2E;
    kbargs.tab = tab;
    ReduceArgs rargs;
    rargs.part = static_cast<const float*>(ws);
    rargs.scores = scores;
    rargs.T = kbargs.T;
    rargs.hkv = hkv;
    rargs.tab = tab;
    int kb_items = 0, red_items = 0;
    for (int i = lo; i < hi; ++i) {
      kbargs.tab.first[i - lo] = kb_items;
      kbargs.tab.nc[i - lo] = v[i].nrc;
      rargs.tab.first[i - lo] = red_items;
      rargs.tab.nc[i - lo] = v[i].nrc;
      if (v[i].mode == Mode::BIG && !v[i].p2rb) {
        kb_items += hkv * v[i].nkb * v[i].nrc;
        if (v[i].nrc > 1) red_items += hkv * v[i].n;
      }
    }
    kbargs.tab.first[hi - lo] = kb_items;
    rargs.tab.first[hi - lo] = red_items;
    if (kb_items > 0) {
      if (s->dtype == WAITS_BF16) {
        if (s->head_dim == 64)
          hipLaunchKernelGGL((key_block_kernel<bf16_t, 64>), dim3(kb_items), dim3(KB_THREADS), 0, stream, kbargs);
        else
          hipLaunchKernelGGL((key_block_kernel<bf16_t, 128>), dim3(kb_items), dim3(KB_THREADS), 0, stream, kbargs);
      } else {  // fp32 only at head_dim 64 (see plan_seqs)
        hipLaunchKernelGGL((key_block_kernel<float, 64>), dim3(kb_items), dim3(KB_THREADS), 0, stream, kbargs);
      }
      if (launched() != WAITS_OK) return WAITS_EDEVICE;
    }
    if (red_items > 0) {
      hipLaunchKernelGGL(colsum_reduce_kernel, dim3((red_items + 255) / 256), dim3(256), 0, stream, rargs);
      if (launched() != WAITS_OK) return WAITS_EDEVICE;
    }

    // fp32 rows of head_dim 128
    ColsumArgs args;
    args.q = q;
    args.k = k;
    args.lse = lse;
    args.scores = scores;
    args.st = strides_of(s);
    args.T = s->cu_seqlens[s->batch];
    args.G = G;
    args.hkv = hkv;
    args.scale_log2 = s->scale * LOG2E;
    args.tab = tab;
    int items = 0;
    for (int i = lo; i < hi; ++i) {
      args.tab.first[i - lo] = items;
      if (v[i].mode == Mode::WIDE) items += hkv * ((v[i].n + WGKEYS2 - 1) / WGKEYS2);
    }
    args.tab.first[hi - lo] = items;
    if (items > 0) {
      launch_colsum<float, 128>(args, items, stream);
      if (launched() != WAITS_OK) return WAITS_EDEVICE;
    }
  }
  return WAITS_OK;
}

// The fields waits_select reads: batch, cu_seqlens, n_kv_heads; and the budget.
int check_select_shape(const waits_shape* s, int32_t budget) {
  if (!s || !s->cu_seqlens || s->batch < 1 || s->n_kv_heads < 1 || s->cu_seqlens[0] != 0)
    return WAITS_EINVAL;
  for (int i = 0; i < s->batch; ++i) {
    const int64_t n = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    if (n < 0 || n > MAX_SEQ_LEN) return WAITS_EINVAL;
  }
  return budget < 1 ? WAITS_EINVAL : WAITS_OK;
}

int check_select(const waits_shape* s, const float* scores, int32_t budget, const int32_t* idx) {
  const int rc = check_select_shape(s, budget);
  if (rc != WAITS_OK) return rc;
  if (!idx || !is_aligned(idx, 4)) return WAITS_EINVAL;
  if (s->cu_seqlens[s->batch] > 0 && (!scores || !is_aligned(scores, 4))) return WAITS_EINVAL;
  return WAITS_OK;
}

int check_gather(const waits_shape* s, const void* k, const void* v, const int32_t* idx,
                 int32_t budget, const void* k_out, const void* v_out) {
  if (budget < 1 || !idx || !k_out || !v_out || !is_aligned(idx, 4) || !is_aligned(k_out, 16) ||
      !is_aligned(v_out, 16))
    return WAITS_EINVAL;
  if (s->cu_seqlens[s->batch] > 0 && (!k || !v || !is_aligned(k, 16) || !is_aligned(v, 16)))
    return WAITS_EINVAL;
  return WAITS_OK;
}

int run_compact(const waits_shape* s, const void* k, const void* v, const int32_t* idx,
                int32_t budget, void* k_out, void* v_out, hipStream_t stream);

int seq_len(const waits_shape* s, int i) { return (int)(s->cu_seqlens[i + 1] - s->cu_seqlens[i]); }

// Table of sequences [lo, hi) for the select and compact kernels, which read
// only the lengths and token offsets.
void fill_len_table(SeqTable& t, const waits_shape* s, int lo, int hi) {
  std::memset(&t, 0, sizeof(t));
  t.nb = hi - lo;
  for (int i = lo; i < hi; ++i) {
    t.n[i - lo] = seq_len(s, i);
    t.tok0[i - lo] = s->cu_seqlens[i];
  }
}

// Workspace of the several-workgroup select for sequences [lo, hi): one
// record per chunk (WIDE_REC_BYTES: its bin offsets and its order keys in
// bin order).  0 when every sequence is short enough for one workgroup.
struct WideWs {
  int items = 0;
  size_t total() const { return (size_t)items * WIDE_REC_BYTES; }
};
WideWs wide_ws(const waits_shape* s, int lo, int hi) {
  WideWs w;
  int gmax = 0;
  for (int i = lo; i < hi; ++i) gmax = std::max(gmax, seq_len(s, i));
  if (gmax <= SEL_WIDE_MIN) return w;
  for (int i = lo; i < hi; ++i) w.items += s->n_kv_heads * wide_chunks(seq_len(s, i));
  return w;
}
static_assert(wide_chunks(MAX_SEQ_LEN) <= WIDE_MAX_CHUNKS, "the longest head fits the place kernel's tables");

size_t select_ws_bytes(const waits_shape* s) {
  size_t mx = 0;
  for (int lo = 0; lo < s->batch; lo += MAXB) mx = std::max(mx, wide_ws(s, lo, std::min(s->batch, lo + MAXB)).total());
  return mx;
}

// The gather of sequences [lo, hi) from their kept positions.
int launch_compact(const waits_shape* s, const void* k, const void* v, const int32_t* idx, int32_t budget,
                   void* k_out, void* v_out, int lo, int hi, hipStream_t stream) {
  const int e = elt_bytes(s->dtype);
  const int row_bytes = s->head_dim * e;
  const int rows_per_block = 256 / (row_bytes / 16);
  const int64_t first_row = (int64_t)lo * s->n_kv_heads * budget;
  CompactArgs args;
  args.k = static_cast<const unsigned char*>(k);
  args.v = static_cast<const unsigned char*>(v);
  args.idx = idx + first_row;
  args.k_out = static_cast<unsigned char*>(k_out) + first_row * row_bytes;
  args.v_out = static_cast<unsigned char*>(v_out) + first_row * row_bytes;
  args.st = strides_of(s);
  args.rows = (int64_t)(hi - lo) * s->n_kv_heads * budget;
  args.hkv = s->n_kv_heads;
  args.budget = budget;
  args.elt = e;
  fill_len_table(args.tab, s, lo, hi);
  const int64_t blocks = (args.rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, args, row_bytes);
  return launched();
}

// Select (and, with FUSE, the gather) per launch group of up to MAXB
// sequences.  Plans from cu_seqlens alone: no host allocation.
template <bool FUSE>
int run_select(const waits_shape* s, const float* scores, int32_t budget, int32_t* idx,
               const void* k, const void* vv, void* k_out, void* v_out, void* ws, size_t ws_bytes,
               hipStream_t stream) {
  const size_t need = select_ws_bytes(s);
  if (ws_bytes < need || (need > 0 && (!ws || !is_aligned(ws, 16)))) return WAITS_EWORKSPACE;
  const int e = FUSE ? elt_bytes(s->dtype) : 0;
  const int row_bytes = FUSE ? s->head_dim * e : 0;
  for (int lo = 0; lo < s->batch; lo += MAXB) {
    const int hi = std::min(s->batch, lo + MAXB);
    const int64_t first_row = (int64_t)lo * s->n_kv_heads * budget;
    int gmax = 0;
    for (int i = lo; i < hi; ++i) gmax = std::max(gmax, seq_len(s, i));
    if (gmax > SEL_WIDE_MIN) {
      WideArgs args;
      std::memset(&args, 0, sizeof(args));
      args.scores = scores;
      args.idx = idx + first_row;
      args.rec = static_cast<unsigned char*>(ws);
      args.T = s->cu_seqlens[s->batch];
      args.hkv = s->n_kv_heads;
      args.budget = budget;
      args.k = static_cast<const unsigned char*>(k);
      args.v = static_cast<const unsigned char*>(vv);
      args.k_out = FUSE ? static_cast<unsigned char*>(k_out) + first_row * row_bytes : nullptr;
      args.v_out = FUSE ? static_cast<unsigned char*>(v_out) + first_row * row_bytes : nullptr;
      args.st = strides_of(s);
      args.elt = e;
      args.row_shift = FUSE ? __builtin_ctz(row_bytes / 16) : 0;
      fill_len_table(args.tab, s, lo, hi);
      int items = 0;
      for (int i = lo; i < hi; ++i) {
        args.tab.first[i - lo] = items;
        items += s->n_kv_heads * wide_chunks(seq_len(s, i));
      }
      args.tab.first[hi - lo] = items;
      if (items > 0) {
        hipLaunchKernelGGL(wide_sort_kernel, dim3(items), dim3(SEL_THREADS), 0, stream, args);
        if (launched() != WAITS_OK) return WAITS_EDEVICE;
        hipLaunchKernelGGL((wide_place_kernel<FUSE>), dim3(items), dim3(SEL_THREADS), 0, stream, args);
        if (launched() != WAITS_OK) return WAITS_EDEVICE;
      }
      continue;
    }
    SelectArgs args;
    args.scores = scores;
    args.idx = idx + first_row;
    args.T = s->cu_seqlens[s->batch];
    args.hkv = s->n_kv_heads;
    args.budget = budget;
    args.k = static_cast<const unsigned char*>(k);
    args.v = static_cast<const unsigned char*>(vv);
    args.k_out = FUSE ? static_cast<unsigned char*>(k_out) + first_row * row_bytes : nullptr;
    args.v_out = FUSE ? static_cast<unsigned char*>(v_out) + first_row * row_bytes : nullptr;
    args.st = strides_of(s);
    args.elt = e;
    args.row_shift = FUSE ? __builtin_ctz(row_bytes / 16) : 0;
    fill_len_table(args.tab, s, lo, hi);
    const dim3 grid((hi - lo) * s->n_kv_heads);
    static_assert(SEL_WIDE_MIN == SEL_THREADS * 32, "one workgroup holds at most 32 keys per lane");
    // slots per lane: the fewest that hold the launch group's longest head
    if (gmax <= SEL_THREADS * 4)
      hipLaunchKernelGGL((select_kernel<4, FUSE>), grid, dim3(SEL_THREADS), 0, stream, args);
    else if (gmax <= SEL_THREADS * 8)
      hipLaunchKernelGGL((select_kernel<8, FUSE>), grid, dim3(SEL_THREADS), 0, stream, args);
    else if (gmax <= SEL_THREADS * 16)
      hipLaunchKernelGGL((select_kernel<16, FUSE>), grid, dim3(SEL_THREADS), 0, stream, args);
    else
      hipLaunchKernelGGL((select_kernel<32, FUSE>), grid, dim3(SEL_THREADS), 0, stream, args);
    if (launched() != WAITS_OK) return WAITS_EDEVICE;
  }
  return WAITS_OK;
}

// The static scratch's address on the device `stream` belongs to (the
// current device for the null stream), looked up on the first call for that
// device, with the device current, and kept.
constexpr int SCRATCH_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_DEVICES];
void* scratch_ptr[SCRATCH_DEVICES];
hipError_t scratch_rc[SCRATCH_DEVICES];

int device_scratch(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return WAITS_EDEVICE;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return WAITS_EDEVICE;
    dev = sd;
  }
  if (dev < 0 || dev >= SCRATCH_DEVICES) return WAITS_EUNSUPPORTED;
  std::call_once(scratch_once[dev], [dev, cur] {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) {
      scratch_rc[dev] = hipErrorInvalidDevice;
      return;
    }
    void* ptr = nullptr;
    scratch_rc[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = ptr;
    if (dev != cur) (void)hipSetDevice(cur);
  });
  if (scratch_rc[dev] != hipSuccess || !scratch_ptr[dev]) return WAITS_EDEVICE;
  *out = scratch_ptr[dev];
  return WAITS_OK;
}

int check_select_compact(const waits_shape* s, const float* scores, const void* k, const void* v,
                         int32_t budget, int32_t* idx, void* k_out, void* v_out) {
  int rc = check_shape(s, false);
  if (rc == WAITS_OK) rc = check_select(s, scores, budget, idx);
  if (rc == WAITS_OK) rc = check_gather(s, k, v, idx, budget, k_out, v_out);
  return rc;
}

int run_select_compact(const waits_shape* s, const float* scores, const void* k, const void* v,
                       int32_t budget, int32_t* idx, void* k_out, void* v_out, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  if (budget > SEL_FUSE_MAX) {
    const int rc = run_select<false>(s, scores, budget, idx, nullptr, nullptr, nullptr, nullptr, ws,
                                     ws_bytes, stream);
    if (rc != WAITS_OK) return rc;
    return run_compact(s, k, v, idx, budget, k_out, v_out, stream);
  }
  return run_select<true>(s, scores, budget, idx, k, v, k_out, v_out, ws, ws_bytes, stream);
}

// Prefill attention forward: one item per (sequence, KV head, block of
// AT_ROWS packed rows), the blocks with the longest key ranges first.
int run_attention(const waits_shape* s, const void* q, const void* k, const void* v, void* out,
                  float* lse, hipStream_t stream) {
  const int G = s->n_q_heads / s->n_kv_heads;
  const int hkv = s->n_kv_heads;
  const int64_t row_bytes = s->kv_stride_tok * elt_bytes(s->dtype);
  for (int i = 0; i < s->batch; ++i) {
    const int64_t n = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    // buffer loads address a sequence's K/V rows with 32-bit offsets
    // (the last stage may reach AT_STAGE rows past the sequence end)
    if ((n + AT_STAGE) * row_bytes > 0x7FFFFFFF || (int64_t)G * n > INT32_MAX / 2) return WAITS_EUNSUPPORTED;
  }
  for (int lo = 0; lo < s->batch; lo += MAXB) {
    const int hi = std::min(s->batch, lo + MAXB);
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = static_cast<bf16_t*>(out);
    a.lse = lse;
    a.st = strides_of(s);
    a.ntok = s->cu_seqlens[s->batch];
    a.G = G;
    a.hkv = hkv;
    a.hq = s->n_q_heads;
    a.scale_log2 = s->scale * LOG2E;
    SeqTable& t = a.tab;
    t.nb = hi - lo;
    int items = 0;
    for (int i = lo; i < hi; ++i) {
      const int n = (int)(s->cu_seqlens[i + 1] - s->cu_seqlens[i]);
      const int j = i - lo;
      t.n[j] = n;
      t.tok0[j] = s->cu_seqlens[i];
      t.nrb[j] = (int)ceil_div((int64_t)G * n, AT_ROWS);
      t.first[j] = items;
      items += hkv * t.nrb[j];
    }
    t.first[hi - lo] = items;
    if (items == 0) continue;
    if (s->head_dim == 64)
      hipLaunchKernelGGL(attn_fwd_kernel<64>, dim3(items), dim3(AT_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_fwd_kernel<128>, dim3(items), dim3(AT_THREADS), 0, stream, a);
    if (launched() != WAITS_OK) return WAITS_EDEVICE;
  }
  return WAITS_OK;
}

int run_compact(const waits_shape* s, const void* k, const void* v, const int32_t* idx,
                int32_t budget, void* k_out, void* v_out, hipStream_t stream) {
  for (int lo = 0; lo < s->batch; lo += MAXB) {
    const int hi = std::min(s->batch, lo + MAXB);
    if (launch_compact(s, k, v, idx, budget, k_out, v_out, lo, hi, stream) != WAITS_OK) return WAITS_EDEVICE;
  }
  return WAITS_OK;
}

}  // namespace
}  // namespace waits

using namespace waits;

extern "C" {

int waits_first_rows(const waits_shape* s, const float* a, const int32_t* b, int32_t* first_row) {
  if (!s || !s->cu_seqlens || s->batch < 1 || s->cu_seqlens[0] != 0 || !first_row)
    return WAITS_EINVAL;
  for (int i = 0; i < s->batch; ++i) {
    const int64_t n = s->cu_seqlens[i + 1] - s->cu_seqlens[i];
    if (n < 0 || n > MAX_SEQ_LEN) return WAITS_EINVAL;
  }
  const int rc = check_curves(s, a, b);
  if (rc != WAITS_OK) return rc;
  for (int i = 0; i < s->batch; ++i)
    first_row[i] = first_live_row((int)(s->cu_seqlens[i + 1] - s->cu_seqlens[i]), a[i], b[i]);
  return WAITS_OK;
}

int waits_lse_workspace_bytes(const waits_shape* s, const float* a, const int32_t* b,
                              size_t* bytes) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc == WAITS_OK && !bytes) rc = WAITS_EINVAL;
  if (rc != WAITS_OK) return rc;
  *bytes = lse_ws_bytes(s, plan_seqs(s, a, b, 1));
  return WAITS_OK;
}

int waits_colsum_workspace_bytes(const waits_shape* s, const float* a, const int32_t* b,
                                 size_t* bytes) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc == WAITS_OK && !bytes) rc = WAITS_EINVAL;
  if (rc != WAITS_OK) return rc;
  *bytes = colsum_ws_bytes(s, plan_seqs(s, a, b, 2));
  return WAITS_OK;
}

int waits_score_workspace_bytes(const waits_shape* s, const float* a, const int32_t* b,
                                size_t* bytes) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc == WAITS_OK && !bytes) rc = WAITS_EINVAL;
  if (rc != WAITS_OK) return rc;
  *bytes = lse_buffer_bytes(s) +
           std::max(lse_ws_bytes(s, plan_seqs(s, a, b, 1)), colsum_ws_bytes(s, plan_seqs(s, a, b, 2)));
  return WAITS_OK;
}

int waits_lse(const waits_shape* s, const void* q, const void* k, const float* a,
              const int32_t* b, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc != WAITS_OK) return rc;
  if (s->cu_seqlens[s->batch] == 0) return WAITS_OK;
  if (!q || !k || !lse || !is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(lse, 4))
    return WAITS_EINVAL;
  return run_lse(s, q, k, a, b, lse, ws, ws_bytes, stream);
}

int waits_colsum(const waits_shape* s, const void* q, const void* k, const float* lse,
                 const float* a, const int32_t* b, float* scores, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc != WAITS_OK) return rc;
  if (s->cu_seqlens[s->batch] == 0) return WAITS_OK;
  if (!q || !k || !lse || !scores || !is_aligned(q, 16) || !is_aligned(k, 16) ||
      !is_aligned(lse, 4) || !is_aligned(scores, 4))
    return WAITS_EINVAL;
  return run_colsum(s, q, k, lse, a, b, scores, ws, ws_bytes, stream);
}

int waits_score(const waits_shape* s, const void* q, const void* k, const float* a,
                const int32_t* b, float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(s, true);
  if (rc == WAITS_OK) rc = check_curves(s, a, b);
  if (rc != WAITS_OK) return rc;
  if (s->cu_seqlens[s->batch] == 0) return WAITS_OK;
  if (!q || !k || !scores || !is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(scores, 4))
    return WAITS_EINVAL;
  const size_t lse_bytes = lse_buffer_bytes(s);
  const size_t need =
      lse_bytes + std::max(lse_ws_bytes(s, plan_seqs(s, a, b, 1)), colsum_ws_bytes(s, plan_seqs(s, a, b, 2)));
  if (!ws || ws_bytes < need || !is_aligned(ws, 256)) return WAITS_EWORKSPACE;
  float* lse = static_cast<float*>(ws);
  void* part = static_cast<unsigned char*>(ws) + lse_bytes;  // pass-1 partials, then pass-2 partials
  rc = run_lse(s, q, k, a, b, lse, part, ws_bytes - lse_bytes, stream);
  if (rc != WAITS_OK) return rc;
  return run_colsum(s, q, k, lse, a, b, scores, part, ws_bytes - lse_bytes, stream);
}

int waits_select_workspace_bytes(const waits_shape* s, int32_t budget, size_t* bytes) {
  const int rc = check_select_shape(s, budget);
  if (rc != WAITS_OK) return rc;
  if (!bytes) return WAITS_EINVAL;
  *bytes = select_ws_bytes(s);
  return WAITS_OK;
}

int waits_select(const waits_shape* s, const float* scores, int32_t budget, int32_t* idx,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  const int rc = check_select(s, scores, budget, idx);
  if (rc != WAITS_OK) return rc;
  return run_select<false>(s, scores, budget, idx, nullptr, nullptr, nullptr, nullptr, ws,
                           ws_bytes, stream);
}

int waits_compact(const waits_shape* s, const void* k, const void* v, const int32_t* idx,
                  int32_t budget, void* k_out, void* v_out, hipStream_t stream) {
  int rc = check_shape(s, false);
  if (rc == WAITS_OK) rc = check_gather(s, k, v, idx, budget, k_out, v_out);
  if (rc != WAITS_OK) return rc;
  return run_compact(s, k, v, idx, budget, k_out, v_out, stream);
}

int waits_select_compact(const waits_shape* s, const float* scores, const void* k, const void* v,
                         int32_t budget, int32_t* idx, void* k_out, void* v_out, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  const int rc = check_select_compact(s, scores, k, v, budget, idx, k_out, v_out);
  if (rc != WAITS_OK) return rc;
  return run_select_compact(s, scores, k, v, budget, idx, k_out, v_out, ws, ws_bytes, stream);
}

int waits_select_compact_noalloc(const waits_shape* s, const float* scores, const void* k,
                                 const void* v, int32_t budget, int32_t* idx, void* k_out,
                                 void* v_out, hipStream_t stream) {
  int rc = check_select_compact(s, scores, k, v, budget, idx, k_out, v_out);
  if (rc != WAITS_OK) return rc;
  const size_t need = select_ws_bytes(s);
  if (need > STATIC_SCRATCH_BYTES) return WAITS_ESCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    rc = device_scratch(stream, &ws);
    if (rc != WAITS_OK) return rc;
  }
  return run_select_compact(s, scores, k, v, budget, idx, k_out, v_out, ws, need, stream);
}

const char* waits_strerror(int code) {
  switch (code) {
    case WAITS_OK: return "ok";
    case WAITS_EINVAL: return "invalid argument";
    case WAITS_EUNSUPPORTED: return "unsupported configuration (head_dim must be 64 or 128)";
    case WAITS_EWORKSPACE: return "workspace missing or too small";
    case WAITS_EDEVICE: return "HIP runtime refused a kernel launch";
    case WAITS_ESCRATCH:
      return "batch needs more scratch than the no-allocation call's static 16 MiB (use the workspace call)";
    default: return "unknown WAITS status";
  }
}

int waits_attention(const waits_shape* s, const void* q, const void* k, const void* v, void* out,
                    float* lse, hipStream_t stream) {
  const int rc = check_shape(s, true);
  if (rc != WAITS_OK) return rc;
  if (s->dtype != WAITS_BF16) return WAITS_EUNSUPPORTED;
  if (s->cu_seqlens[s->batch] == 0) return WAITS_OK;
  if (!q || !k || !v || !out || !is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) ||
      !is_aligned(out, 16) || (lse && !is_aligned(lse, 4)))
    return WAITS_EINVAL;
  return run_attention(s, q, k, v, out, lse, stream);
}

}  // extern "C"
