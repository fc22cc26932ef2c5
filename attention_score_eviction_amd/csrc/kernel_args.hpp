// Kernel argument blocks.  Per-sequence tables travel by value in the kernel
// argument segment, so a launch needs no host-to-device copy and no device
// work list: a workgroup finds its sequence by scanning `first`.
#pragma once

#include <stdint.h>

#include "device_common.hpp"

namespace waits {

struct SeqTable {
  int32_t nb;                 // sequences in this launch (<= MAXB)
  int32_t n[MAXB];            // sequence length N
  int32_t q0[MAXB];           // first processed query row
  int32_t first[MAXB + 1];    // first work item of each sequence; first[nb] = total
  int32_t rg[MAXB];           // pass 1 (fp32 wide rows): row groups per KV head
  int32_t nrb[MAXB];          // pass 1 (few-rows kernel): row blocks per KV head
  int32_t nc[MAXB];           // pass 1: key chunks per row group
  int32_t kc[MAXB];           // keys per chunk (multiple of 32); 0 in the combine: every chunk
  int32_t prow[MAXB];         // pass 1: packed-row pitch per KV head of the partials
  float a[MAXB];              // forgetting-curve slope
  float c[MAXB];              // N - b - 0.5 (exact in fp32)
  int64_t tok0[MAXB];         // first token of the sequence in the packed batch
  int64_t ws0[MAXB];          // pass 1: first partial slot (float2 units)
};

struct Strides {
  int64_t q_tok, q_head;      // elements
  int64_t kv_tok, kv_head;    // elements
};

struct LseArgs {
  const void* q;
  const void* k;
  float* lse;                 // [Hq, T]
  float2* part;               // pass-1 partials (split over keys)
  Strides st;
  int64_t T;
  int32_t G;
  int32_t hkv;
  float scale;                // softmax scale
  float scale_log2;           // scale * log2(e)
  SeqTable tab;
};

struct CombineArgs {
  float* lse;
  const float2* part;
  int64_t T;
  int32_t G;
  int32_t hkv;
  int32_t team[MAXB];         // lanes per row of each sequence (power of two dividing 64)
  SeqTable tab;               // first[]: first thread of each sequence (multiples of 64)
};

struct ColsumArgs {
  const void* q;
  const void* k;
  const float* lse;           // [Hq, T]
  float* scores;              // [Hkv, T]
  Strides st;
  int64_t T;
  int32_t G;
  int32_t hkv;
  float scale_log2;
  SeqTable tab;
};

struct SelectArgs {
  const float* scores;        // [Hkv, T]
  int32_t* idx;               // [nb, Hkv, budget] (this launch's slice)
  int64_t T;
  int32_t hkv;
  int32_t budget;
  // Gather fused into the select launch (select_kernel<..., true> only):
  // rows of K and V at the kept positions, zero rows past the kept count.
  const unsigned char* k;
  const unsigned char* v;
  unsigned char* k_out;       // [nb, Hkv, budget, d] (this launch's slice)
  unsigned char* v_out;
  Strides st;                 // kv_* used
  int32_t elt;                // bytes per element
  int32_t row_shift;          // log2 of the 16-byte vectors per row
  SeqTable tab;
};

struct CompactArgs {
  const unsigned char* k;
  const unsigned char* v;
  const int32_t* idx;         // this launch's slice
  unsigned char* k_out;
  unsigned char* v_out;
  Strides st;                 // kv_* used
  int64_t rows;               // nb * Hkv * budget rows in this launch
  int32_t hkv;
  int32_t budget;
  int32_t elt;                // bytes per element
  SeqTable tab;               // tok0 used
};

}  // namespace waits
