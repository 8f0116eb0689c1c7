/*
 * misa.h - C ABI of the MI355X (gfx950) lightning-indexer library.
 *
 * The library computes, on one GPU, the token selection that a DeepSeek
 * sparse-attention indexer hands to sparse attention, in the three forms the
 * MISA and HISA write-ups describe:
 *
 *   misa_route      block-mean router: pick A of the H indexer heads per query
 *                   (MISA technical summary, "Metodologia: MISA", first stage).
 *   misa_score_topk routed heads score every visible key, then top-k
 *                   (same section, second stage "sparse token scoring").
 *   misa_hier_topk  routed pass keeps k' candidates, all H heads rescore them,
 *                   then top-k (MISA technical summary, "Variante Jerarquica").
 *   hisa_topk       top-m key blocks by their mean-pooled representative, then
 *                   the full indexer on the tokens of those blocks, then top-k
 *                   (HISA write-up, section 3, Stage 1 and Stage 2).
 *   hisa_maxpool_topk  HISA with max-pooled block representatives (HISA
 *                   write-up, limitations).
 *   misa_hisa_topk  HISA with the routed heads in both stages: the head axis
 *                   of MISA and the token axis of HISA combined.
 *   misa_block_means  the query-independent block means the router pools.
 *
 * Definitions (the pages give the structure; the exact formulas are fixed here):
 *   z(t,h,s)  = q[t,h,:] . k[s,:]
 *   I_S(t,s)  = sum_{h in S} w[t,h] * max(0, z(t,h,s))        (no renormalisation)
 *   visible   : key s is visible to query t iff s <= pos[t]; n_t = pos[t]+1
 *   blocks    : M_t = ceil(n_t/B); block b = [b*B, min((b+1)*B, n_t)); its
 *               representative Kbar_{t,b} is the mean of those keys (so the
 *               last block of a query may be partial)
 *   router    : r(t,h) = w[t,h] * max_b max(0, q[t,h] . Kbar_{t,b}); keep the
 *               first A heads under (-r, h)
 *   HISA block score: beta(t,b) = sum_h w[t,h] * max(0, q[t,h] . Kbar_{t,b})
 *   selection : the first min(k, count) items under (-score, index); -0.0 == +0.0
 *
 * Conventions shared by every entry point:
 *   - Every array argument is caller-owned, contiguous, row-major DEVICE memory;
 *     the struct misa_problem itself lives in host memory. The library never
 *     allocates or frees device memory: scratch comes from the caller's
 *     workspace `ws` of `ws_bytes` bytes (size it with misa_workspace_bytes;
 *     256-byte alignment is required).
 *   - `stream` is a hipStream_t (NULL = the legacy default stream). Calls only
 *     enqueue work and return; they never synchronise the host.
 *   - Argument errors are reported synchronously, before anything is enqueued,
 *     and leave every output untouched. MISA_ERR_HIP reports a failed launch.
 *   - Outputs: idx[T,k] int32 and scores[T,k] float32. Row t holds its
 *     k_t = min(k, count) selected keys in ascending key order, followed by
 *     k - k_t padding entries (idx = -1, score = -inf).
 *   - pos values outside [0, L) are clamped: pos < 0 gives a row with no
 *     visible key (all padding), pos >= L behaves as pos = L-1.
 *   - Supported on the GPU: d = 128; 1 <= H <= 64; 1 <= A <= H; B >= 1;
 *     q bf16, or OCP E4M3FN codes with a per-(query, head) fp32 scale;
 *     K bf16 or OCP E4M3FN with a per-token fp32 scale (any finite scale
 *     value; the sign of a negative scale is honoured).
 *   - fp8 queries (q_dtype MISA_Q_FP8_E4M3FN) need fp8 keys (the contraction
 *     runs on fp8 x fp8 matrix cores) and decode-shaped batches wherever heads
 *     are routed or keys are scored over the whole prefix (misa_route,
 *     misa_score_topk, misa_hier_topk, misa_hisa_topk: T * A' <= 256 with A'
 *     = A rounded up to a power of two >= 4, and the few-query router);
 *     hisa_topk and hisa_maxpool_topk take any T. Otherwise
 *     MISA_ERR_UNSUPPORTED.
 *   - Calls that share a workspace must be ordered on one stream; otherwise the
 *     library is stateless and reentrant.
 */
#ifndef MISA_H
#define MISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum misa_status {
  MISA_OK = 0,
  MISA_ERR_INVALID_ARG = -1, /* null pointer, negative size, A > H, k' < k ... */
  MISA_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels support (d != 128, H > 64) */
  MISA_ERR_WORKSPACE = -3,   /* ws too small or misaligned */
  MISA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} misa_status;

typedef enum misa_kdtype {
  MISA_K_BF16 = 0,        /* K[L,d] as bf16 bit patterns (uint16) */
  MISA_K_FP8_E4M3FN = 1   /* K[L,d] as OCP E4M3FN bytes; value = code * k_scale[s] */
} misa_kdtype;

typedef enum misa_qdtype {
  MISA_Q_BF16 = 0,        /* q[T,H,d] as bf16 bit patterns (uint16) */
  MISA_Q_FP8_E4M3FN = 1   /* q[T,H,d] as OCP E4M3FN bytes; value = code * q_scale[t,h] */
} misa_qdtype;

typedef enum misa_op {
  MISA_OP_ROUTE = 0,
  MISA_OP_SCORE_TOPK = 1,
  MISA_OP_HIER_TOPK = 2,
  MISA_OP_HISA_TOPK = 3,
  MISA_OP_BLOCK_MEANS = 4,
  MISA_OP_MISA_HISA_TOPK = 5,
  MISA_OP_BLOCK_SCORES = 6
} misa_op;

/* One indexer problem. All pointers are device pointers. */
typedef struct misa_problem {
  int32_t T;               /* queries (>= 0; T == 0 is a no-op) */
  int32_t H;               /* indexer heads per query */
  int32_t d;               /* head dim (128) */
  int32_t L;               /* keys (>= 1) */
  int32_t B;               /* block size of the router / HISA blocks (>= 1) */
  int32_t k_dtype;         /* misa_kdtype */
  const void* q;           /* [T,H,d] bf16 bits, or E4M3FN bytes (q_dtype) */
  const float* w;          /* [T,H]   per-query head weights */
  const void* K;           /* [L,d]   shared indexer keys (bf16 bits or e4m3fn bytes) */
  const float* k_scale;    /* [L]     per-token scale, required iff k_dtype is fp8, else NULL */
  const int32_t* pos;      /* [T]     causal position of each query */
  const float* kbar;       /* [ceil(L/B),d] cached block means, or NULL (see below) */
  int32_t q_dtype;         /* misa_qdtype (MISA_Q_BF16 for bf16 queries) */
  const float* q_scale;    /* [T,H]   per-(query, head) scale, required iff q_dtype is fp8, else NULL */
} misa_problem;

/* Cached block means (kbar). When p->kbar is NULL every call pools the keys
 * itself. When it is set, row b of kbar stands for the mean of block b
 * wherever block b is a complete block before a query's own last block
 * (b < M_t - 1); each query's last block is always pooled from K, since it
 * depends on pos[t]. The library trusts the values: results are those of the
 * definitions evaluated with these means, which is what misa_block_means
 * writes. Pointer must be 16-byte aligned. Used by misa_route,
 * misa_score_topk, misa_hier_topk, hisa_topk and misa_hisa_topk; misa_block_means
 * ignores it. */

/* Bytes of workspace entry point `op` needs for this problem and these
 * parameters (unused parameters are ignored). Returns 0 for an invalid request;
 * a valid request always needs at least 256 bytes. */
size_t misa_workspace_bytes(const misa_problem* p, int32_t op, int32_t A, int32_t kprime,
                            int32_t k, int32_t m);

/* Full-block means of the whole key array (MISA summary, "Metodologia: MISA":
 * the router pools keys block by block; HISA Stage 1 pools each block by its mean).
 * kbar[ceil(L/B), d] float32: row b is the mean of keys [b*B, min((b+1)*B, L)),
 * accumulated in float64 and rounded once. q, w and pos are not read. */
misa_status misa_block_means(const misa_problem* p, float* kbar, void* ws, size_t ws_bytes,
                             void* stream);

/* Incremental form of misa_block_means for a growing key array (the cached
 * block statistics the MISA summary's "Metodologia: MISA" presumes when it
 * calls the router's cost negligible): with p->L the new length, rows
 * first_block .. ceil(L/B) - 1 of kbar are recomputed exactly as
 * misa_block_means computes them, and only those blocks' keys are read; the
 * rows before first_block are left as they are. After keys [L_old, L) were
 * appended, first_block = L_old / B brings kbar up to date. first_block must
 * lie in [0, ceil(L/B)] (MISA_ERR_INVALID_ARG otherwise; ceil(L/B) is a no-op);
 * the workspace is that of misa_block_means. */
misa_status misa_block_means_update(const misa_problem* p, int32_t first_block, float* kbar, void* ws,
                                    size_t ws_bytes, void* stream);

/* Router (MISA summary, "Metodologia: MISA", block-pooled router): heads[T,A]
 * int32 receives the routed heads of each query in ascending order; r[T,H]
 * float32 (may be NULL) receives r(t,h). The selection is taken in float64
 * from exact block sums, so it matches an exact evaluation except where two
 * heads' scores agree to float64 rounding. */
misa_status misa_route(const misa_problem* p, int32_t A, int32_t* heads, float* r, void* ws,
                       size_t ws_bytes, void* stream);

/* MISA selection (MISA summary, "Metodologia: MISA", sparse token scoring):
 * the A routed heads of each query score every visible key with I_R; the
 * top-k keys are returned. `heads` [T,A] may supply the routed heads (any
 * distinct values in [0,H)); NULL routes inside the call. A == H with
 * heads == NULL is the dense DSA indexer. scores[] hold I_R. */
misa_status misa_score_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t k,
                            int32_t* idx, float* scores, void* ws, size_t ws_bytes, void* stream);

/* MISA-dagger (MISA summary, "Variante Jerarquica"): the routed pass keeps the
 * top-kprime keys by I_R, all H heads rescore those candidates with I_all and
 * the top-k of them are returned (scores hold I_all). Requires kprime >= k. */
misa_status misa_hier_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t kprime,
                           int32_t k, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                           void* stream);

/* Size in bytes of the library's static device scratch (see
 * misa_hier_topk_noalloc). */
#define MISA_STATIC_SCRATCH_BYTES (32u << 20)

/* misa_hier_topk for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, and harnesses that forbid
 * hipMalloc. Same arguments, results, validation and errors as
 * misa_hier_topk, except that there is no workspace argument: the scratch is
 * a static device array of MISA_STATIC_SCRATCH_BYTES bytes inside the library
 * (one copy per GPU, held from the library's first use on that GPU until the
 * process ends). The call allocates and frees nothing.
 *   - A problem whose scratch need (misa_workspace_bytes(p, MISA_OP_HIER_TOPK,
 *     A, kprime, k, 1)) exceeds MISA_STATIC_SCRATCH_BYTES is rejected with
 *     MISA_ERR_WORKSPACE before anything is enqueued (decode batches up to
 *     T = 16 queries over 131,072 keys fit).
 *   - Every call on one GPU shares that GPU's scratch and leaves its own
 *     contents there. Calls ordered on one stream are safe; calls that may
 *     overlap on one GPU (different streams, or threads enqueuing
 *     concurrently) race on the scratch and give undefined results.
 *   - The device is the calling thread's current device. */
misa_status misa_hier_topk_noalloc(const misa_problem* p, int32_t A, const int32_t* heads, int32_t kprime,
                                   int32_t k, int32_t* idx, float* scores, void* stream);

/* HISA (HISA write-up, section 3, Stage 1 and Stage 2): keep the top-m blocks
 * of each query by beta (ties to the lower block), score the visible tokens of
 * those blocks with all H heads (I_all) and return the top-k. */
misa_status hisa_topk(const misa_problem* p, int32_t m, int32_t k, int32_t* idx, float* scores,
                      void* ws, size_t ws_bytes, void* stream);

/* HISA Stage 1 block scores on their own (HISA write-up, section 3, Stage 1:
 * the query is scored against the block representatives only):
 *   beta[t * beta_ld + b] = sum_h w[t,h] * max(0, q[t,h] . Kbar_{t,b})
 * for every visible block b < M_t of query t, formed in float64 and rounded
 * once to float32; entries b >= M_t are not written. These are the values
 * hisa_topk ranks for its top-m blocks (same kernel, same bits). beta is
 * device memory [T, beta_ld] float32 with beta_ld >= ceil(L/B).
 * Workspace: misa_workspace_bytes(p, MISA_OP_BLOCK_SCORES, ...). Cached means
 * (p->kbar) are used as in hisa_topk. */
misa_status hisa_block_scores(const misa_problem* p, float* beta, int64_t beta_ld, void* ws,
                              size_t ws_bytes, void* stream);

/* HISA with max-pooled block representatives (HISA write-up, limitations:
 * max pooling in place of mean pooling, listed as a possible improvement).
 * As hisa_topk, except that the representative of block b of query t is, per
 * dimension, the largest of its visible keys' values (dequantised keys; the
 * tail block over [b*B, n_t) only), so that one key standing out in a block is
 * not averaged away. Workspace: misa_workspace_bytes(p, MISA_OP_HISA_TOPK, ., .,
 * k, m). p->kbar must be NULL (cached means do not apply); otherwise errors,
 * arguments and outputs as hisa_topk. */
misa_status hisa_maxpool_topk(const misa_problem* p, int32_t m, int32_t k, int32_t* idx, float* scores,
                              void* ws, size_t ws_bytes, void* stream);

/* MISA inside HISA. The MISA technical summary presents head routing as an
 * efficiency axis complementary to token-axis hierarchies such as HISA and
 * combinable with them ("Contribuciones Clave", "Significado y Afirmaciones");
 * the plain reading used here puts the A routed heads R_t (as misa_route picks
 * them) in place of all H heads in both HISA stages:
 *   beta_R(t,b) = sum_{h in R_t} w[t,h] * max(0, q[t,h] . Kbar_{t,b}),
 * the top-m blocks by beta_R (ties to the lower block), I_R on the visible
 * tokens of those blocks, and the top-k of those (scores hold I_R).
 * `heads` [T,A] may supply the routed heads (distinct values in [0,H)); NULL
 * routes inside the call. A == H with heads == NULL is hisa_topk. Errors as
 * for misa_score_topk and hisa_topk. */
misa_status misa_hisa_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t m, int32_t k,
                           int32_t* idx, float* scores, void* ws, size_t ws_bytes, void* stream);

/* Short static text for a status code. */
const char* misa_status_str(int32_t status);

/* Detail of the most recent error reported on the calling host thread
 * ("" if none). The pointer stays valid until the thread's next call. */
const char* misa_last_error(void);

/* Kernel timing instrumentation. While enabled, every kernel the library
 * enqueues is bracketed by a pair of HIP events on the same stream; this adds
 * a little launch overhead, so time whole calls with it disabled.
 * misa_profile_read synchronises the recorded events and returns, for kernels
 * whose name contains `name_substr`, the summed duration in milliseconds and
 * the launch count; misa_profile_reset drops all records. */
misa_status misa_profile_enable(int32_t on);
misa_status misa_profile_read(const char* name_substr, double* total_ms, int64_t* launches);
misa_status misa_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MISA_H */
