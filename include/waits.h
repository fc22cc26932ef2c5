/*
 * waits.h -- C ABI of the WAITS prefill KV-selection path on AMD MI355X
 * (gfx950): score every prompt key, keep the top keys per KV head, gather
 * the kept K/V rows into a compacted cache.
 *
 * Method (WAITS README, page "Dirac-Notation/A2SF", introduction): a prompt
 * key's score is the causal softmax attention it receives, summed over all
 * query rows of the prompt with the sigmoid forgetting-curve weight
 *     w[q] = 1 / (1 + exp(-a (q - (N - b - 0.5)))),   q = 0 .. N-1,
 * and the cache keeps the highest-scoring keys.  a = 0 is H2O, a = +inf with
 * b = 1 is TOVA, a = +inf with b = window is SnapKV.  The README's
 * "Quickstart" names the knobs: sigmoid_a (a), recent_budget (b) and
 * select_budget (keys kept per KV head); "Repository layout" names the top-k
 * selector.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - A batch is `batch` independent sequences (prompts, or layers of one
 *   prompt) packed along a token axis of T = cu_seqlens[batch] tokens.
 *   Positions q, k restart at 0 in every sequence.
 * - Q is [T, n_q_heads, head_dim], K and V are [T, n_kv_heads, head_dim],
 *   addressed with element strides (q_stride_tok, q_stride_head) and
 *   (kv_stride_tok, kv_stride_head); the head_dim axis is contiguous.  K and
 *   V share strides.  Every row must start on a 16-byte boundary.
 * - Query head g reads KV head g / G, G = n_q_heads / n_kv_heads; a KV
 *   head's score sums its G query heads.
 * - dtype WAITS_BF16: bf16 inputs, bf16 x bf16 products accumulated in
 *   fp32; WAITS_F32: fp32 inputs and fp32 arithmetic.  Softmax, weights and
 *   scores are fp32.
 * - Ownership: the caller allocates every buffer (device memory unless the
 *   argument says host).  The library allocates nothing, frees nothing,
 *   keeps no state between calls and never synchronises: it enqueues
 *   kernels on `stream` and returns.  Results are ready when the stream is.
 * - Errors: every argument is checked on the host before anything is
 *   enqueued; a failed check returns a nonzero WAITS_E* code and enqueues
 *   nothing.  WAITS_EDEVICE reports a launch the HIP runtime refused; faults
 *   inside kernels surface at the caller's next synchronisation.
 * - Per-sequence limits: 0 <= N < 2^22 and 1 <= b <= 2^22 (so N - b - 0.5
 *   and q - (N - b - 0.5) are exact in fp32); larger values are rejected.
 */
#ifndef WAITS_H
#define WAITS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  WAITS_OK = 0,
  WAITS_EINVAL = 1,       /* malformed argument (null, negative, NaN, ...) */
  WAITS_EUNSUPPORTED = 2, /* well-formed but not built (head_dim, dtype)   */
  WAITS_EWORKSPACE = 3,   /* workspace missing or smaller than required    */
  WAITS_EDEVICE = 4,      /* the HIP runtime refused a launch              */
  WAITS_ESCRATCH = 5      /* the no-allocation call's static scratch is too
                             small for this batch                          */
};

enum { WAITS_BF16 = 0, WAITS_F32 = 1 };

/*
 * Pass-2 plan for sequences with more than 512 packed query rows (G x
 * processed rows) per KV head; shorter ones always keep every row of a KV
 * head in one workgroup.
 * WAITS_PASS2_AUTO: pass 2 reuses pass 1's row blocks (512 packed rows
 *   each), every block writing its column sums to the workspace as
 *   [row block][n_kv_heads][N] fp32 per sequence, added per key in block
 *   order; sequences whose partials would pass 6 GiB (6 GiB over a launch of
 *   up to 32 sequences) take the key-block plan instead.
 * WAITS_PASS2_KEY_BLOCKS: every such sequence runs pass 2 on blocks of 512
 *   keys, each streaming the rows that can see it; a block's rows may be
 *   cut into chunks whose partial sums take [chunk][n_kv_heads][T] fp32 of
 *   workspace, added in chunk order.  Same definition, different summation
 *   order (agreement to fp32 rounding, not bit for bit).
 */
enum { WAITS_PASS2_AUTO = 0, WAITS_PASS2_KEY_BLOCKS = 1 };

typedef struct waits_shape {
  int32_t batch;              /* number of sequences, >= 1                     */
  const int64_t* cu_seqlens;  /* HOST array [batch + 1], cu[0] = 0, ascending */
  int32_t n_q_heads;          /* >= 1, multiple of n_kv_heads                  */
  int32_t n_kv_heads;         /* >= 1                                          */
  int32_t head_dim;           /* 64 or 128                                     */
  int32_t dtype;              /* WAITS_BF16 or WAITS_F32                       */
  int64_t q_stride_tok, q_stride_head;   /* element strides of Q          */
  int64_t kv_stride_tok, kv_stride_head; /* element strides of K and V    */
  float scale;                /* softmax scale, finite > 0 (1/sqrt(head_dim)) */
  int32_t pass2;              /* WAITS_PASS2_AUTO (0) or WAITS_PASS2_KEY_BLOCKS;
                                 checked by every call that takes Q (any other
                                 value: WAITS_EINVAL)                          */
} waits_shape;

/*
 * a[i], b[i] (HOST arrays [batch]): the forgetting curve of sequence i.
 * a in [0, +inf] (NaN and negative values are rejected); 1 <= b <= 2^22
 * (b > N is allowed and weights every row).  a = +inf is evaluated with IEEE
 * arithmetic: N - b - 0.5 is a half-integer, so w is exactly 0 or 1.
 *
 * Only query rows whose fp32 weight is nonzero can change a score; the
 * library processes every row from the first one whose fp32 weight can be
 * nonzero to the end of the sequence and skips the rows before it, whose
 * fp32 weight is exactly 0.
 */

/*
 * Host-only planning query (enqueues nothing, touches no device): for every
 * sequence i, first_row[i] receives the first query row the library
 * processes.  Every row q < first_row[i] has fp32 a * (c - q) > 89 with
 * c = N - b - 0.5, so expf overflows and its fp32 weight is exactly 0.
 * first_row: HOST int32 [batch].
 */
int waits_first_rows(const waits_shape* shape, const float* a, const int32_t* b,
                     int32_t* first_row);

/* Bytes of device workspace waits_lse needs for this batch (0 is possible). */
int waits_lse_workspace_bytes(const waits_shape* shape, const float* a,
                              const int32_t* b, size_t* bytes);

/*
 * Pass 1, per-row log-sum-exp (README introduction: the softmax normaliser
 * of each weighted query row):
 *   lse[g * T + t] = ln sum_{k <= q} exp(scale * <Q[t, g], K[t0 + k, g / G]>)
 * for every processed row q (t = t0 + q, t0 = cu_seqlens[i]).
 * lse: device fp32 [n_q_heads, T], written only at processed rows; other
 * entries are left untouched.  workspace: device, 8-byte aligned,
 * >= waits_lse_workspace_bytes (per-chunk (max, sum) pairs of rows whose keys
 * are split over several workgroups; WAITS_EWORKSPACE if missing, short or
 * misaligned).
 */
int waits_lse(const waits_shape* shape, const void* q, const void* k,
              const float* a, const int32_t* b, float* lse, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace waits_colsum needs for this batch (0 is possible). */
int waits_colsum_workspace_bytes(const waits_shape* shape, const float* a,
                                 const int32_t* b, size_t* bytes);

/*
 * Pass 2, weighted column sums (README introduction: accumulative attention
 * score under the forgetting curve):
 *   scores[h * T + t0 + k] = sum_{g in group h} sum_{q >= k}
 *                            w[q] * exp(scale <Q[t0+q, g], K[t0+k, h]> - lse[g*T+t0+q])
 * for every key k of every sequence.  lse: as written by waits_lse.
 * scores: device fp32 [n_kv_heads, T], fully written.  workspace: device,
 * 4-byte aligned, >= waits_colsum_workspace_bytes (partial sums of keys
 * whose rows are split over several workgroups; they are added in a fixed
 * order, so scores are bitwise reproducible).
 */
int waits_colsum(const waits_shape* shape, const void* q, const void* k,
                 const float* lse, const float* a, const int32_t* b,
                 float* scores, void* workspace, size_t workspace_bytes,
                 hipStream_t stream);

/* Bytes of device workspace waits_score needs: the lse buffer, then room
 * for the larger of the pass-1 and pass-2 workspaces. */
int waits_score_workspace_bytes(const waits_shape* shape, const float* a,
                                const int32_t* b, size_t* bytes);

/* waits_lse followed by waits_colsum, with lse kept in the workspace. */
int waits_score(const waits_shape* shape, const void* q, const void* k,
                const float* a, const int32_t* b, float* scores,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Prefill attention forward with the row log-sum-exp.  README "Quickstart":
 * the method runs inside the model's attention call; introduction: the
 * score is built from the causal softmax of every prompt row.  The attention
 * forward computes each row's normaliser anyway, so it writes it out: for
 * every query row q (t = t0 + q, t0 = cu_seqlens[i]) and query head g,
 *   out[(t * n_q_heads + g) * head_dim + e]
 *       = sum_{k <= q} softmax_k(scale <Q[t, g], K[t0 + k, g / G]>) V[t0 + k, g / G, e]
 *   lse[g * T + t] = ln sum_{k <= q} exp(scale <Q[t, g], K[t0 + k, g / G]>)
 * lse equals what waits_lse writes at every row, so waits_colsum can take it
 * directly and the WAITS scores then need no pass 1 of their own.
 * out: device bf16, dense [T, n_q_heads, head_dim], 16-byte aligned.  lse:
 * device fp32 [n_q_heads, T], or NULL.  V shares K's strides.  dtype must be
 * WAITS_BF16 (WAITS_F32: WAITS_EUNSUPPORTED); a sequence's K/V rows must span
 * less than 2^31 bytes (else WAITS_EUNSUPPORTED).  Softmax sums and out
 * accumulate in fp32; P is rounded to bf16 for the P V product.
 */
int waits_attention(const waits_shape* shape, const void* q, const void* k, const void* v,
                    void* out, float* lse, hipStream_t stream);

/*
 * Top-k selection (README "Repository layout": top-k selector): for every
 * sequence i and KV head h, the min(N_i, select_budget) keys with the
 * largest score, ties to the lower position, written in ascending position
 * order to idx[(i * n_kv_heads + h) * select_budget + j] (device int32,
 * sequence-relative positions); slots j >= N_i hold -1.
 * scores: device fp32 [n_kv_heads, T], every value >= +0 (as waits_score
 * writes them).  select_budget >= 1.  Only shape->batch, cu_seqlens and
 * n_kv_heads are read from `shape`.
 */
int waits_select(const waits_shape* shape, const float* scores,
                 int32_t select_budget, int32_t* idx, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace waits_select and waits_select_compact need for
 * this batch: 0 unless a sequence has more than 32768 keys, whose selection
 * is split over workgroups of 4096 keys that meet in the workspace (each
 * chunk's counting sort by the top 12 bits of its scores: bin offsets and
 * the scores' order keys, 24864 bytes per chunk).  The select writes every word of it
 * that it reads, so its contents between calls do not matter.
 * workspace: device, 16-byte aligned.
 */
int waits_select_workspace_bytes(const waits_shape* shape, int32_t select_budget,
                                 size_t* bytes);

/*
 * Compaction (README introduction: the retained key-value pairs): copies
 * the selected rows bit for bit,
 *   k_out[((i * n_kv_heads + h) * select_budget + j) * head_dim + e]
 *     = K[cu_seqlens[i] + idx[(i * n_kv_heads + h) * select_budget + j], h, e]
 * and the same for V; slots whose idx is -1 are zero-filled.  k_out, v_out:
 * device, dtype of K/V, dense [batch, n_kv_heads, select_budget, head_dim].
 * idx entries must be -1 or in [0, N_i) (as waits_select writes them).
 */
int waits_compact(const waits_shape* shape, const void* k, const void* v,
                  const int32_t* idx, int32_t select_budget, void* k_out,
                  void* v_out, hipStream_t stream);

/*
 * Selection and compaction fused: the outputs of waits_select (idx)
 * followed by waits_compact (k_out, v_out), with the same arguments,
 * layouts and error codes as those two calls, bit for bit.  The workgroup
 * that places a key also copies its K/V rows while the position is at hand,
 * so the gather needs no launch of its own and no re-read of idx.  For
 * select_budget > 8192 it runs the select and compact kernels one after
 * the other on `stream`.  workspace: as for waits_select.
 */
int waits_select_compact(const waits_shape* shape, const float* scores,
                         const void* k, const void* v, int32_t select_budget,
                         int32_t* idx, void* k_out, void* v_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * waits_select_compact for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument, and the same outputs, layouts and
 * error codes as waits_select_compact, bit for bit.  The select of heads of
 * more than 32768 keys needs scratch (per-chunk counting-sort records: the
 * bytes waits_select_workspace_bytes reports); this call takes it from a
 * static device array of WAITS_STATIC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends, and returns WAITS_ESCRATCH
 * for a batch that needs more: a launch group (32 sequences) with such a
 * head needs 24864 bytes per 4096 keys (rounded up) of each of its KV heads,
 * e.g. 6.1 MiB for one sequence of 8 KV heads x 131072 keys; 16 MiB holds
 * 674 such chunks.
 * - The scratch of a GPU is the copy on the device `stream` belongs to (the
 *   current device for the null stream); the first call for a device looks
 *   its address up (hipGetSymbolAddress) and keeps it.
 * - Every call on a GPU shares that GPU's array and leaves its contents
 *   behind; each call writes every word it reads before reading it.  Calls that overlap
 *   on one GPU (several streams or host threads at once) race on the array
 *   and give undefined results: serialise them.
 * - No device or host memory is allocated by this call.
 */
#define WAITS_STATIC_SCRATCH_BYTES (16u << 20)
int waits_select_compact_noalloc(const waits_shape* shape, const float* scores,
                                 const void* k, const void* v, int32_t select_budget,
                                 int32_t* idx, void* k_out, void* v_out, hipStream_t stream);

/*
 * Decode attention over the compacted cache
 * -----------------------------------------
 * README "Quickstart": after init_cache compresses the prompt's cache,
 * generation runs on it, so every decoding step attends over the kept rows
 * (and the rows generation appends after them).  The attention is ordinary
 * scaled dot-product attention of the step's one query per query head:
 *   out[i, g, :] = sum_{j < len[i]} softmax_j(scale <q[i, g], K[i, h, j]>) V[i, h, j]
 *   lse[i, g]    = ln sum_{j < len[i]} exp(scale <q[i, g], K[i, h, j]>),   h = g / G
 * with no mask inside the cache and no position change (cached keys carry
 * their own).  An empty cache (len = 0) gives out = 0 and lse = -inf.
 *
 * Layouts (all dense, device, 16-byte-aligned base pointers for q and the
 * caches):
 *   q        [batch, n_q_heads, head_dim]              (dtype)
 *   k_cache  [batch, n_kv_heads, capacity, head_dim]   (dtype; the layout
 *   v_cache   waits_compact writes, with capacity = select_budget, or a
 *             larger capacity whose rows past the kept ones hold new tokens)
 *   lens     int32 [batch]: rows attended per sequence; values outside
 *            [0, capacity] are clamped to it
 *   out      fp32 [batch, n_q_heads, head_dim]
 *   lse      fp32 [batch, n_q_heads], or NULL
 * dtype WAITS_BF16: bf16 q and caches, products accumulated in fp32, the
 * probabilities and the weighted sum of V in fp32; WAITS_F32: fp32
 * throughout.  Ownership, stream and error rules are those of the rest of
 * this header.
 */
typedef struct waits_decode_shape {
  int32_t batch;       /* number of sequences, >= 1                        */
  int32_t n_q_heads;   /* >= 1, multiple of n_kv_heads                     */
  int32_t n_kv_heads;  /* >= 1                                             */
  int32_t head_dim;    /* 64 or 128                                        */
  int32_t dtype;       /* WAITS_BF16 or WAITS_F32                          */
  int32_t capacity;    /* cache rows per (sequence, KV head), 1 .. 2^20    */
  float scale;         /* softmax scale, finite > 0 (1/sqrt(head_dim))     */
} waits_decode_shape;

/* Bytes of device workspace waits_decode needs (0 when every (sequence,
 * KV head) runs as one work item; otherwise room for per-split partials). */
int waits_decode_workspace_bytes(const waits_decode_shape* shape, size_t* bytes);

/* One decoding step's attention for a batch, as defined above.  workspace:
 * device, 16-byte aligned, >= waits_decode_workspace_bytes (NULL if 0). */
int waits_decode(const waits_decode_shape* shape, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* lens, float* out, float* lse,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a WAITS_E* code. */
const char* waits_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* WAITS_H */
