// Host side of waits_decode (include/waits.h, "Decode attention over the
// compacted cache"): argument checks, the work plan and kernel launches on
// the caller's stream.  Nothing here allocates, synchronises or keeps state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>

#include "waits.h"
#include "decode.hpp"

namespace waits {
namespace {

constexpr int DEC_NUM_CU = 256;
constexpr int DEC_MIN_KS = 256;                      // shortest key split (shorter caches: one)
constexpr int DEC_MAX_CAP = DEC_MAX_KS * DEC_MAX_SPLITS;

struct DecPlan {
  int gc = 1, ngc = 1, ks = DEC_MIN_KS, nsplit = 1;
  size_t ml_bytes = 0, ws_bytes = 0;                 // partials: (max, sum), then o
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t cdiv(int64_t x, int64_t y) { return (x + y - 1) / y; }

int check_decode_shape(const waits_decode_shape* s) {
  if (!s) return WAITS_EINVAL;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->capacity < 1) return WAITS_EINVAL;
  if (s->n_q_heads % s->n_kv_heads) return WAITS_EINVAL;
  if (s->dtype != WAITS_BF16 && s->dtype != WAITS_F32) return WAITS_EINVAL;
  if (!(std::isfinite(s->scale) && s->scale > 0.f)) return WAITS_EINVAL;
  if (s->head_dim != 64 && s->head_dim != 128) return WAITS_EUNSUPPORTED;
  if (s->capacity > DEC_MAX_CAP) return WAITS_EUNSUPPORTED;
  return WAITS_OK;
}

// Query heads per item: the group (rounded up to a power of two) while it
// fits 8, so every K/V row is read once per split; larger groups in chunks
// of 8.  Key splits: about 4 items per CU over the batch, 256..1024 keys each
// (a shorter cache is one split: its combine launch would cost more than the
// parallelism it buys).
DecPlan plan_decode(const waits_decode_shape* s) {
  DecPlan p;
  const int G = s->n_q_heads / s->n_kv_heads;
  p.gc = G > 4 ? 8 : G > 2 ? 4 : G;
  p.ngc = (G + p.gc - 1) / p.gc;
  const int64_t rows = (int64_t)s->batch * s->n_kv_heads * p.ngc * s->capacity;
  int64_t ks = cdiv(rows, 4 * DEC_NUM_CU);
  ks = cdiv(ks, 16) * 16;
  ks = std::max<int64_t>(ks, cdiv(s->capacity, DEC_MAX_SPLITS));
  const int64_t min_ks = std::min<int64_t>(DEC_MIN_KS, cdiv(s->capacity, 16) * 16);
  p.ks = (int)std::min<int64_t>(std::max<int64_t>(ks, min_ks), DEC_MAX_KS);
  p.nsplit = (int)cdiv(s->capacity, p.ks);
  if (p.nsplit > 1) {
    const size_t slots = (size_t)s->batch * s->n_q_heads * p.nsplit;
    p.ml_bytes = (slots * sizeof(float2) + 255) / 256 * 256;
    p.ws_bytes = p.ml_bytes + slots * s->head_dim * sizeof(float);
  }
  return p;
}

template <typename T, int D>
void launch_decode_gc(const DecodeArgs& a, int gc, unsigned grid, hipStream_t st) {
  switch (gc) {
    case 1: hipLaunchKernelGGL((decode_kernel<T, D, 1>), dim3(grid), dim3(DEC_THREADS), 0, st, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<T, D, 2>), dim3(grid), dim3(DEC_THREADS), 0, st, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<T, D, 4>), dim3(grid), dim3(DEC_THREADS), 0, st, a); break;
    default: hipLaunchKernelGGL((decode_kernel<T, D, 8>), dim3(grid), dim3(DEC_THREADS), 0, st, a); break;
  }
}

void launch_decode(const waits_decode_shape* s, const DecodeArgs& a, int gc, unsigned grid,
                   hipStream_t st) {
  if (s->dtype == WAITS_BF16) {
    if (s->head_dim == 64) launch_decode_gc<bf16_t, 64>(a, gc, grid, st);
    else launch_decode_gc<bf16_t, 128>(a, gc, grid, st);
  } else {
    if (s->head_dim == 64) launch_decode_gc<float, 64>(a, gc, grid, st);
    else launch_decode_gc<float, 128>(a, gc, grid, st);
  }
}

}  // namespace
}  // namespace waits

using namespace waits;

extern "C" {

int waits_decode_workspace_bytes(const waits_decode_shape* s, size_t* bytes) {
  const int rc = check_decode_shape(s);
  if (rc != WAITS_OK) return rc;
  if (!bytes) return WAITS_EINVAL;
  *bytes = plan_decode(s).ws_bytes;
  return WAITS_OK;
}

int waits_decode(const waits_decode_shape* s, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* lens, float* out, float* lse,
                 void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_decode_shape(s);
  if (rc != WAITS_OK) return rc;
  if (!q || !k_cache || !v_cache || !lens || !out) return WAITS_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(lens, 4) ||
      !aligned(out, 4) || (lse && !aligned(lse, 4)))
    return WAITS_EINVAL;
  const DecPlan p = plan_decode(s);
  if (ws_bytes < p.ws_bytes || (p.ws_bytes > 0 && (!ws || !aligned(ws, 16)))) return WAITS_EWORKSPACE;
  const int64_t grid = (int64_t)s->batch * s->n_kv_heads * p.nsplit * p.ngc;
  if (grid > INT_MAX) return WAITS_EUNSUPPORTED;

  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.lens = lens;
  a.out = out;
  a.lse = lse;
  a.part_ml = p.nsplit > 1 ? static_cast<float2*>(ws) : nullptr;
  a.part_o = p.nsplit > 1 ? reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + p.ml_bytes)
                          : nullptr;
  a.B = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.G = s->n_q_heads / s->n_kv_heads;
  a.D = s->head_dim;
  a.cap = s->capacity;
  a.ks = p.ks;
  a.nsplit = p.nsplit;
  a.ngc = p.ngc;
  a.scale_log2 = s->scale * LOG2E;

  launch_decode(s, a, p.gc, (unsigned)grid, stream);
  if (hipGetLastError() != hipSuccess) return WAITS_EDEVICE;
  if (p.nsplit > 1) {
    const int64_t heads = (int64_t)s->batch * s->n_q_heads;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((unsigned)cdiv(heads, DEC_WAVES)), dim3(DEC_THREADS),
                       0, stream, a);
    if (hipGetLastError() != hipSuccess) return WAITS_EDEVICE;
  }
  return WAITS_OK;
}

}  // extern "C"
