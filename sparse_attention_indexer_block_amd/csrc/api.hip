// C ABI of the indexer library: argument checks, workspace layout, and the
// four pipelines (route; MISA score + top-k; MISA-dagger; HISA), each a short
// sequence of asynchronous launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/misa.h"
#include "launch.h"

namespace misa {

// ---------------------------------------------------------------- errors

static thread_local std::string g_last_error;

static misa_status fail(misa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

static misa_status hip_fail(hipError_t e, const char* where) {
  return fail(MISA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---------------------------------------------------------------- profiling

struct ProfRec {
  std::string name;
  hipEvent_t start = nullptr, stop = nullptr;
};

static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<ProfRec> g_prof;

bool prof_events(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (!g_prof_on) return false;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  ProfRec r;
  r.name = name;
  if (hipEventCreate(&r.start) != hipSuccess) return false;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return false;
  }
  g_prof.push_back(r);
  *start = r.start;
  *stop = r.stop;
  return true;
}

// ---------------------------------------------------------------- workspace

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  }
};

struct Plan {
  size_t ksum = 0, tsum = 0, pmax = 0, kb16 = 0, part = 0, heads = 0, beta = 0, qr = 0, wr = 0;
  size_t S = 0;
  size_t rmm = 0, ghist = 0, rec = 0, gcnt = 0, bcnt = 0, bkeys = 0;
  size_t cand = 0, ncand = 0, S2 = 0, blocks = 0, nblocks = 0;
  long long S_ld = 0, cand_ld = 0, S2_ld = 0, beta_ld = 0;
  long long zero_words = 0;  // ghist, cleared by the first kernel that needs it
  int Mmax = 0, mm = 0;
  size_t total = 0;
};

static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Long-row selection scratch for `rows` rows of up to `max_n` items.
static void plan_long(Bump& bp, Plan& pl, int rows, int max_n) {
  if (max_n <= topk_lds_cap()) return;
  const size_t nch = (size_t)topk_long_chunks(max_n);
  const size_t rld = nch * (size_t)topk_long_chunk();
  const size_t nmm = nch > (size_t)score_max_splits() ? nch : (size_t)score_max_splits();
  // one set of scratch serves every selection of a call (they run in order)
  pl.rmm = bp.take(nmm * rows * 2 * 4);
  pl.zero_words = (long long)rows * topk_coarse_bins();
  pl.ghist = bp.take((size_t)pl.zero_words * 4);
  pl.rec = bp.take((size_t)rows * topk_long_rec_bytes());
  pl.gcnt = bp.take((size_t)rows * nch * 4);
  pl.bcnt = bp.take((size_t)rows * nch * 4);
  pl.bkeys = bp.take((size_t)rows * rld * 4);
}

static void plan_route(Bump& bp, Plan& pl, const misa_problem* p) {
  const int M = ceil_div(p->L, p->B);
  pl.ksum = bp.take((size_t)M * 128 * 8);
  pl.tsum = bp.take((size_t)p->T * 128 * 8);
  // router: per-tile head maxima, then the last blocks' values
  pl.pmax = bp.take((size_t)p->T * (route_chunks(p->L, p->B) + 1) * 64 * 8);
  if (route_fast_wins(p->L, p->B, p->T)) {
    pl.kb16 = bp.take((size_t)M * 2 * 128 * 2);
    pl.part = bp.take((size_t)p->T * route_fast_parts(p->L, p->B, p->T) * 64 * route_part_bytes());
  }
}

static Plan make_plan(const misa_problem* p, int op, int A, int kprime, int k, int m) {
  Bump bp;
  Plan pl;
  const int T = p->T, L = p->L;
  bp.take(256);  // keep offset 0 unused so 0 can mean "absent"
  switch (op) {
    case MISA_OP_BLOCK_MEANS:
      pl.ksum = bp.take((size_t)ceil_div(L, p->B) * 128 * 8);
      break;
    case MISA_OP_ROUTE:
    case MISA_OP_BLOCK_SCORES:
      plan_route(bp, pl, p);
      break;
    case MISA_OP_SCORE_TOPK:
      plan_route(bp, pl, p);
      pl.heads = bp.take((size_t)T * A * 4);
      pl.qr = bp.take((size_t)T * A * 128 * 2);
      pl.wr = bp.take((size_t)T * A * 4);
      pl.S_ld = padded_ld(L);
      pl.S = bp.take((size_t)(T + 1) * pl.S_ld * 4);  // + the scoring kernel's dump row
      plan_long(bp, pl, T, L);
      break;
    case MISA_OP_HIER_TOPK: {
      plan_route(bp, pl, p);
      pl.heads = bp.take((size_t)T * A * 4);
      pl.qr = bp.take((size_t)T * A * 128 * 2);
      pl.wr = bp.take((size_t)T * A * 4);
      pl.S_ld = padded_ld(L);
      pl.S = bp.take((size_t)(T + 1) * pl.S_ld * 4);  // + the scoring kernel's dump row
      pl.cand_ld = padded_ld(kprime < L ? kprime : L);
      pl.cand = bp.take((size_t)T * pl.cand_ld * 4);
      pl.ncand = bp.take((size_t)T * 4);
      pl.S2_ld = pl.cand_ld;
      pl.S2 = bp.take((size_t)(T + 1) * pl.S2_ld * 4);  // + the scoring kernel's dump row
      plan_long(bp, pl, T, L);  // covers the k' stage and the final stage (k' <= L)
      break;
    }
    case MISA_OP_HISA_TOPK:
    case MISA_OP_MISA_HISA_TOPK: {
      plan_route(bp, pl, p);
      if (op == MISA_OP_MISA_HISA_TOPK) {  // the routed heads' packed rows
        pl.heads = bp.take((size_t)T * A * 4);
        pl.qr = bp.take((size_t)T * A * 128 * 2);
        pl.wr = bp.take((size_t)T * A * 4);
      }
      pl.Mmax = ceil_div(L, p->B);
      pl.mm = m < pl.Mmax ? m : pl.Mmax;
      pl.beta_ld = padded_ld(pl.Mmax);
      pl.beta = bp.take((size_t)T * pl.beta_ld * 4);
      pl.blocks = bp.take((size_t)T * pl.mm * 4);
      pl.nblocks = bp.take((size_t)T * 4);
      const long long mb = (long long)pl.mm * p->B;
      pl.cand_ld = padded_ld(mb < L ? mb : L);
      pl.cand = bp.take((size_t)T * pl.cand_ld * 4);
      pl.ncand = bp.take((size_t)T * 4);
      pl.S2_ld = pl.cand_ld;
      pl.S2 = bp.take((size_t)(T + 1) * pl.S2_ld * 4);  // + the scoring kernel's dump row
      const int mx = pl.Mmax > (int)pl.cand_ld ? pl.Mmax : (int)pl.cand_ld;
      plan_long(bp, pl, T, mx);
      break;
    }
    default:
      break;
  }
  pl.total = bp.off;
  return pl;
}

template <typename Tp>
static Tp* at(void* ws, size_t off) {
  return off ? reinterpret_cast<Tp*>(static_cast<char*>(ws) + off) : nullptr;
}

// ---------------------------------------------------------------- validation

static bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

static misa_status check_problem(const misa_problem* p, bool need_queries) {
  if (!p) return fail(MISA_ERR_INVALID_ARG, "problem is NULL");
  if (p->T < 0) return fail(MISA_ERR_INVALID_ARG, "T = %d is negative", p->T);
  if (p->d < 1 || p->H < 1) return fail(MISA_ERR_INVALID_ARG, "H = %d and d = %d must be >= 1", p->H, p->d);
  if (p->L < 1) return fail(MISA_ERR_INVALID_ARG, "L = %d must be >= 1", p->L);
  if (p->B < 1) return fail(MISA_ERR_INVALID_ARG, "B = %d must be >= 1", p->B);
  if (p->k_dtype != MISA_K_BF16 && p->k_dtype != MISA_K_FP8_E4M3FN)
    return fail(MISA_ERR_INVALID_ARG, "k_dtype = %d is not a misa_kdtype", p->k_dtype);
  if (p->d != kHeadDimHost) return fail(MISA_ERR_UNSUPPORTED, "d = %d (only d = 128 is supported)", p->d);
  if (p->H > 64) return fail(MISA_ERR_UNSUPPORTED, "H = %d (at most 64 heads are supported)", p->H);
  if (p->L > (1 << 23)) return fail(MISA_ERR_UNSUPPORTED, "L = %d exceeds 2^23 keys", p->L);
  if (p->T > (1 << 24)) return fail(MISA_ERR_UNSUPPORTED, "T = %d exceeds 2^24 queries", p->T);
  if (!p->K) return fail(MISA_ERR_INVALID_ARG, "K is NULL");
  if (!aligned(p->K, 16)) return fail(MISA_ERR_INVALID_ARG, "K must be 16-byte aligned");
  const bool fp8 = p->k_dtype == MISA_K_FP8_E4M3FN;
  if (fp8 && !p->k_scale) return fail(MISA_ERR_INVALID_ARG, "k_scale is required for fp8 keys");
  if (!fp8 && p->k_scale) return fail(MISA_ERR_INVALID_ARG, "k_scale must be NULL for bf16 keys");
  if (p->k_scale && !aligned(p->k_scale, 4)) return fail(MISA_ERR_INVALID_ARG, "k_scale must be 4-byte aligned");
  if (p->kbar && !aligned(p->kbar, 16)) return fail(MISA_ERR_INVALID_ARG, "kbar must be 16-byte aligned");
  if (p->q_dtype != MISA_Q_BF16 && p->q_dtype != MISA_Q_FP8_E4M3FN)
    return fail(MISA_ERR_INVALID_ARG, "q_dtype = %d is not a misa_qdtype", p->q_dtype);
  if (need_queries && p->T > 0) {
    const bool qf8 = p->q_dtype == MISA_Q_FP8_E4M3FN;
    if (qf8 && !p->q_scale) return fail(MISA_ERR_INVALID_ARG, "q_scale is required for fp8 queries");
    if (!qf8 && p->q_scale) return fail(MISA_ERR_INVALID_ARG, "q_scale must be NULL for bf16 queries");
    if (qf8 && !aligned(p->q_scale, 4)) return fail(MISA_ERR_INVALID_ARG, "q_scale must be 4-byte aligned");
    if (qf8 && !fp8)
      return fail(MISA_ERR_UNSUPPORTED, "fp8 queries need fp8 keys (fp8 x fp8 matrix products)");
    if (!p->q || !p->w || !p->pos) return fail(MISA_ERR_INVALID_ARG, "q, w and pos must be non-NULL");
    if (!aligned(p->q, 16)) return fail(MISA_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if (!aligned(p->w, 4) || !aligned(p->pos, 4)) return fail(MISA_ERR_INVALID_ARG, "w and pos must be 4-byte aligned");
  }
  return MISA_OK;
}

static misa_status check_ws(const Plan& pl, void* ws, size_t ws_bytes) {
  if (ws_bytes < pl.total)
    return fail(MISA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", ws_bytes, pl.total);
  if (!ws) return fail(MISA_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MISA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return MISA_OK;
}

static misa_status check_out(const void* ptr, const char* name) {
  if (!ptr) return fail(MISA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(ptr, 4)) return fail(MISA_ERR_INVALID_ARG, "%s must be 4-byte aligned", name);
  return MISA_OK;
}

#define MISA_TRY(expr)                   \
  do {                                   \
    misa_status _st = (expr);            \
    if (_st != MISA_OK) return _st;      \
  } while (0)

#define HIP_TRY(expr, where)                     \
  do {                                           \
    hipError_t _e = (expr);                      \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// ---------------------------------------------------------------- pipelines

// sums_ready: the block sums (ksum, or only the query tails with cached means)
// and tsum are already in the workspace from an earlier router pass of this call.
// keep_sums: leave ksum and the query tails tsum in the workspace for a later
// block-score pass of the same call (the float64 head ranking alone pools each
// query's last block itself and reads no tails).
static misa_status run_route(const LaunchCtx& cx, const misa_problem* p, const Plan& pl, void* ws,
                             int A, int32_t* heads, float* r, float* beta, int beta_ld,
                             uint16_t* qr = nullptr, float* wr = nullptr, bool sums_ready = false,
                             bool max_pool = false, bool keep_sums = false) {
  const bool fp8 = p->k_dtype == MISA_K_FP8_E4M3FN;
  double* ksum = at<double>(ws, pl.ksum);
  double* tsum = at<double>(ws, pl.tsum);
  // many queries: a bf16 MFMA pass over hi/lo block means, settled in float64 where it is
  // ambiguous; few queries: every block's rho in float64 directly
  const bool fast = !beta && route_fast_wins(p->L, p->B, p->T);
  uint16_t* kb16 = fast ? at<uint16_t>(ws, pl.kb16) : nullptr;
  // float64 head ranking: per-tile maxima of the complete blocks (plain stores)
  double* part = (!fast && !beta) ? at<double>(ws, pl.pmax) : nullptr;
  const bool qf8 = p->q_dtype == MISA_Q_FP8_E4M3FN;
  if (qf8 && fast)
    return fail(MISA_ERR_UNSUPPORTED, "fp8 queries: T = %d queries over %d blocks need the many-query router",
                p->T, ceil_div(p->L, p->B));
  if (part && max_pool) return fail(MISA_ERR_HIP, "internal: max pooling ranks no heads");
  // query tails: pooled by the block-sum pass whenever it runs (with cached
  // means, where no such pass runs, the router launch pools them itself)
  const bool tails = !part || keep_sums || p->kbar == nullptr;
  // with cached block means only the query tails are pooled here (nothing is
  // launched when no tails are needed either)
  if (!sums_ready)
    HIP_TRY(launch_block_sums(cx, p->K, p->k_scale, fp8, p->L, p->B, ksum, nullptr, p->T, p->pos,
                              tails ? tsum : nullptr, p->kbar != nullptr, kb16, 0, max_pool),
            "block sums");
  if (!fast) {
    HIP_TRY(launch_route(cx, p->q, qf8, p->q_scale, p->w, p->pos, p->T, p->H, p->L, p->B, A, ksum, p->kbar,
                         tails ? tsum : nullptr, p->K, p->k_scale, fp8, part, heads, r, beta, beta_ld, qr, wr,
                         max_pool),
            "router");
  } else {
    HIP_TRY(launch_route_heads(cx, static_cast<const uint16_t*>(p->q), p->w, p->pos, p->T, p->H, p->L, p->B, A, ksum, kb16, p->kbar,
                               tsum, at<void>(ws, pl.part), heads, r, qr, wr),
            "router");
  }
  return MISA_OK;
}

static TopkLongWs long_ws(const Plan& pl, void* ws, int nmm) {
  TopkLongWs lw;
  lw.rmm = at<uint32_t>(ws, pl.rmm);
  lw.nmm = nmm;
  lw.ghist = at<uint32_t>(ws, pl.ghist);
  lw.rec = at<void>(ws, pl.rec);
  lw.gcnt = at<int32_t>(ws, pl.gcnt);
  lw.bcnt = at<int32_t>(ws, pl.bcnt);
  lw.bkeys = at<uint32_t>(ws, pl.bkeys);
  return lw;
}

// Top-k of rows of up to max_n items. Long rows need each row's key range:
// `nmm` > 0 means the scoring kernel already wrote it (and cleared the
// selection counters); otherwise a range pass runs first.
static misa_status run_topk(const LaunchCtx& cx, const TopkArgs& a, const Plan& pl, void* ws,
                            int max_n, int nmm = 0, const RerankArgs* rr = nullptr) {
  if (max_n <= topk_lds_cap()) {
    if (rr) return fail(MISA_ERR_HIP, "internal: the rerank form needs long rows");
    HIP_TRY(launch_topk_rows(cx, a, max_n), "top-k");
    return MISA_OK;
  }
  if (nmm == 0) {
    HIP_TRY(launch_topk_range(cx, a, at<uint32_t>(ws, pl.rmm), at<uint32_t>(ws, pl.ghist),
                              pl.zero_words, max_n),
            "top-k range");
    nmm = topk_long_chunks(max_n);
  }
  HIP_TRY(launch_topk_long(cx, a, long_ws(pl, ws, nmm), max_n, rr), "top-k (long rows)");
  return MISA_OK;
}

static ScoreArgs score_args(const misa_problem* p) {
  ScoreArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = p->q;
  a.q_fp8 = p->q_dtype == MISA_Q_FP8_E4M3FN;
  a.qscale = p->q_scale;  // null for rows that already carry their scales
  a.w = p->w;
  a.H = p->H;
  a.T = p->T;
  a.K = p->K;
  a.kscale = p->k_scale;
  a.L = p->L;
  a.pos = p->pos;
  return a;
}

static TopkArgs topk_args(const misa_problem* p) {
  TopkArgs a;
  std::memset(&a, 0, sizeof(a));
  a.pos = p->pos;
  a.L = p->L;
  a.n_div = 1;
  a.rows = p->T;
  return a;
}

// Routed scores of every visible key into S[T, S_ld]. Returns in *nmm the
// number of per-split key ranges written for long-row selection (0 if none).
static misa_status run_routed_scores(const LaunchCtx& cx, const misa_problem* p, const Plan& pl,
                                     void* ws, int A, const int32_t* heads, int* nmm) {
  ScoreArgs sa = score_args(p);
  uint16_t* qr = at<uint16_t>(ws, pl.qr);
  float* wr = at<float>(ws, pl.wr);
  if (heads) {
    // caller-chosen heads: pack their q rows and weights
    HIP_TRY(launch_gather_heads(cx, p->q, sa.q_fp8, p->q_scale, p->w, heads, p->T, p->H, A, qr, wr),
            "head gather");
  } else if (A < p->H) {
    // routing packs the q rows and weights of the chosen heads as it selects them
    MISA_TRY(run_route(cx, p, pl, ws, A, at<int32_t>(ws, pl.heads), nullptr, nullptr, 0, qr, wr));
  }
  if (heads || A < p->H) {
    sa.q = qr;
    sa.w = wr;
    sa.H = A;
    sa.qscale = nullptr;  // packed fp8 rows carry their scales (sign in the codes, |scale| in w)
  }  // else dense: all H heads in their own order
  sa.A = A;
  sa.S = at<float>(ws, pl.S);
  sa.S_ld = pl.S_ld;
  const bool long_rows = p->L > topk_lds_cap();
  if (long_rows) {
    sa.rmm = at<uint32_t>(ws, pl.rmm);
    sa.zero = at<uint32_t>(ws, pl.ghist);
    sa.zero_n = pl.zero_words;
  }
  int nsplit = 0;
  HIP_TRY(launch_score_keys(cx, sa, p->k_dtype == MISA_K_FP8_E4M3FN, &nsplit), "routed scoring");
  *nmm = long_rows ? nsplit : 0;
  return MISA_OK;
}

// HISA Stage 1 and Stage 2 (HISA write-up, section 3) with the heads of p:
// block scores of every visible block, the top-m blocks, the indexer on their
// tokens, top-k. sums_ready: the block sums are already in the workspace.
static misa_status run_hisa(const LaunchCtx& cx, const misa_problem* p, const Plan& pl, void* ws, int k,
                            int32_t* idx, float* scores, bool sums_ready, bool max_pool = false) {
  float* beta = at<float>(ws, pl.beta);
  MISA_TRY(run_route(cx, p, pl, ws, 1, nullptr, nullptr, beta, (int)pl.beta_ld, nullptr, nullptr,
                     sums_ready, max_pool));
  int32_t* blocks = at<int32_t>(ws, pl.blocks);
  int32_t* nblocks = at<int32_t>(ws, pl.nblocks);
  TopkArgs tb = topk_args(p);
  tb.S = beta;
  tb.S_ld = pl.beta_ld;
  tb.n_div = p->B;
  tb.k = pl.mm;
  tb.out_idx = blocks;
  tb.out_ld = pl.mm;
  tb.out_count = nblocks;
  MISA_TRY(run_topk(cx, tb, pl, ws, pl.Mmax));
  int32_t* cand = at<int32_t>(ws, pl.cand);
  int32_t* ncand = at<int32_t>(ws, pl.ncand);
  const int ncmax = (long long)pl.mm * p->B < p->L ? pl.mm * p->B : p->L;  // candidate bound
  // the refine pass forms the candidate list (indices and counts) from the blocks
  ScoreArgs sa = score_args(p);
  sa.blocks = blocks;
  sa.blocks_ld = pl.mm;
  sa.nblocks = nblocks;
  sa.B = p->B;
  sa.cand_out = cand;
  sa.ncand_out = ncand;
  sa.cand_ld = pl.cand_ld;
  sa.cand_max = ncmax;
  sa.S = at<float>(ws, pl.S2);
  sa.S_ld = pl.S2_ld;
  HIP_TRY(launch_score_gather(cx, sa, p->k_dtype == MISA_K_FP8_E4M3FN), "refine scoring");
  TopkArgs tf = topk_args(p);
  tf.S = at<float>(ws, pl.S2);
  tf.S_ld = pl.S2_ld;
  tf.row_n = ncand;
  tf.row_idx = cand;
  tf.idx_ld = pl.cand_ld;
  tf.k = k;
  tf.out_idx = idx;
  tf.out_score = scores;
  tf.out_ld = k;
  return run_topk(cx, tf, pl, ws, ncmax);
}

static misa_status check_hier_args(const misa_problem* p, int A, const int32_t* heads, int kprime, int k,
                                   int32_t* idx, float* scores) {
  MISA_TRY(check_problem(p, true));
  if (A < 1 || A > p->H) return fail(MISA_ERR_INVALID_ARG, "A = %d must lie in [1, H = %d]", A, p->H);
  if (k < 1) return fail(MISA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (kprime < k) return fail(MISA_ERR_INVALID_ARG, "kprime = %d must be >= k = %d", kprime, k);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(idx, "idx"));
  MISA_TRY(check_out(scores, "scores"));
  if (heads && !aligned(heads, 4)) return fail(MISA_ERR_INVALID_ARG, "heads must be 4-byte aligned");
  if (p->q_dtype == MISA_Q_FP8_E4M3FN && !score_fp8q_supported(p->T, A))
    return fail(MISA_ERR_UNSUPPORTED, "fp8 queries: T = %d with A = %d exceeds the decode-shaped batches", p->T, A);
  return MISA_OK;
}

// MISA-dagger (MISA technical summary, "Variante Jerarquica"): routed scores,
// top-k' candidates, all-head rescoring of the candidates, top-k.
static misa_status run_hier(const LaunchCtx& cx, const misa_problem* p, const Plan& pl, void* ws, int A,
                            const int32_t* heads, int kprime, int k, int32_t* idx, float* scores) {
  int nmm = 0;
  MISA_TRY(run_routed_scores(cx, p, pl, ws, A, heads, &nmm));
  int32_t* cand = at<int32_t>(ws, pl.cand);
  int32_t* ncand = at<int32_t>(ws, pl.ncand);
  const int kc = kprime < p->L ? kprime : p->L;  // candidates kept per query
  // coarse stage: top-k' of the routed scores (indices only)
  TopkArgs ta = topk_args(p);
  ta.S = at<float>(ws, pl.S);
  ta.S_ld = pl.S_ld;
  ta.k = kc;
  ta.out_idx = cand;
  ta.out_ld = pl.cand_ld;
  ta.out_count = ncand;
  // fine stage: all H heads rescore the candidates, then top-k. Long rows
  // rescore each chunk's kept candidates inside the emission pass; otherwise
  // the gather form of the scoring kernel rescores the list.
  const bool fp8k = p->k_dtype == MISA_K_FP8_E4M3FN;
  if (p->L > topk_lds_cap()) {
    RerankArgs rr;
    rr.q = p->q;
    rr.q_fp8 = p->q_dtype == MISA_Q_FP8_E4M3FN;
    rr.qscale = p->q_scale;
    rr.w = p->w;
    rr.H = p->H;
    rr.K = p->K;
    rr.kscale = p->k_scale;
    rr.fp8 = fp8k;
    rr.S = at<float>(ws, pl.S2);
    rr.S_ld = pl.S2_ld;
    MISA_TRY(run_topk(cx, ta, pl, ws, p->L, nmm, &rr));
  } else {
    MISA_TRY(run_topk(cx, ta, pl, ws, p->L, nmm));
    ScoreArgs sa = score_args(p);
    sa.cand = cand;
    sa.cand_ld = pl.cand_ld;
    sa.cand_max = kc;
    sa.ncand = ncand;
    sa.S = at<float>(ws, pl.S2);
    sa.S_ld = pl.S2_ld;
    HIP_TRY(launch_score_gather(cx, sa, fp8k), "rerank scoring");
  }
  TopkArgs tb = topk_args(p);
  tb.S = at<float>(ws, pl.S2);
  tb.S_ld = pl.S2_ld;
  tb.row_n = ncand;
  tb.row_idx = cand;
  tb.idx_ld = pl.cand_ld;
  tb.k = k;
  tb.out_idx = idx;
  tb.out_score = scores;
  tb.out_ld = k;
  return run_topk(cx, tb, pl, ws, kc);
}

// ---------------------------------------------------------------- static scratch

// Device memory for misa_hier_topk_noalloc, which takes no workspace: one copy
// of this array lives on every GPU the library runs on, from the code
// object's load until the process ends. Host code never uses the array's name
// as an address (on the host it is only a stand-in); the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kStaticScratchBytes = MISA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
static misa_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MISA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256)) return fail(MISA_ERR_HIP, "static scratch has no usable device address");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MISA_OK;
}

}  // namespace misa

using namespace misa;

// ---------------------------------------------------------------- C ABI

extern "C" {

size_t misa_workspace_bytes(const misa_problem* p, int32_t op, int32_t A, int32_t kprime, int32_t k,
                            int32_t m) {
  if (check_problem(p, false) != MISA_OK) return 0;
  switch (op) {
    case MISA_OP_ROUTE:
    case MISA_OP_SCORE_TOPK:
      if (A < 1 || A > p->H) return 0;
      if (op == MISA_OP_SCORE_TOPK && k < 1) return 0;
      break;
    case MISA_OP_HIER_TOPK:
      if (A < 1 || A > p->H || k < 1 || kprime < k) return 0;
      break;
    case MISA_OP_HISA_TOPK:
      if (m < 1 || k < 1) return 0;
      break;
    case MISA_OP_MISA_HISA_TOPK:
      if (A < 1 || A > p->H || m < 1 || k < 1) return 0;
      break;
    case MISA_OP_BLOCK_MEANS:
    case MISA_OP_BLOCK_SCORES:
      break;
    default:
      return 0;
  }
  return make_plan(p, op, A, kprime, k, m).total;
}

misa_status misa_block_means(const misa_problem* p, float* kbar, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, false));
  MISA_TRY(check_out(kbar, "kbar"));
  const Plan pl = make_plan(p, MISA_OP_BLOCK_MEANS, 1, 1, 1, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  HIP_TRY(launch_block_sums(cx, p->K, p->k_scale, p->k_dtype == MISA_K_FP8_E4M3FN, p->L, p->B,
                            at<double>(ws, pl.ksum), kbar, 0, nullptr, nullptr),
          "block means");
  return MISA_OK;
}

misa_status misa_block_means_update(const misa_problem* p, int32_t first_block, float* kbar, void* ws,
                                    size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, false));
  MISA_TRY(check_out(kbar, "kbar"));
  const int M = (int)(((long long)p->L + p->B - 1) / p->B);
  if (first_block < 0 || first_block > M)
    return fail(MISA_ERR_INVALID_ARG, "first_block = %d must lie in [0, ceil(L/B) = %d]", first_block, M);
  if (first_block == M) return MISA_OK;
  const Plan pl = make_plan(p, MISA_OP_BLOCK_MEANS, 1, 1, 1, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  HIP_TRY(launch_block_sums(cx, p->K, p->k_scale, p->k_dtype == MISA_K_FP8_E4M3FN, p->L, p->B,
                            at<double>(ws, pl.ksum), kbar, 0, nullptr, nullptr, false, nullptr, first_block),
          "block means update");
  return MISA_OK;
}

misa_status misa_route(const misa_problem* p, int32_t A, int32_t* heads, float* r, void* ws,
                       size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  if (A < 1 || A > p->H) return fail(MISA_ERR_INVALID_ARG, "A = %d must lie in [1, H = %d]", A, p->H);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(heads, "heads"));
  if (r && !aligned(r, 4)) return fail(MISA_ERR_INVALID_ARG, "r must be 4-byte aligned");
  const Plan pl = make_plan(p, MISA_OP_ROUTE, A, 1, 1, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  return run_route(cx, p, pl, ws, A, heads, r, nullptr, 0);
}

misa_status misa_score_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t k,
                            int32_t* idx, float* scores, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  if (A < 1 || A > p->H) return fail(MISA_ERR_INVALID_ARG, "A = %d must lie in [1, H = %d]", A, p->H);
  if (k < 1) return fail(MISA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(idx, "idx"));
  MISA_TRY(check_out(scores, "scores"));
  if (heads && !aligned(heads, 4)) return fail(MISA_ERR_INVALID_ARG, "heads must be 4-byte aligned");
  if (p->q_dtype == MISA_Q_FP8_E4M3FN && !score_fp8q_supported(p->T, A))
    return fail(MISA_ERR_UNSUPPORTED, "fp8 queries: T = %d with A = %d exceeds the decode-shaped batches", p->T, A);
  const Plan pl = make_plan(p, MISA_OP_SCORE_TOPK, A, 1, k, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  int nmm = 0;
  MISA_TRY(run_routed_scores(cx, p, pl, ws, A, heads, &nmm));
  TopkArgs ta = topk_args(p);
  ta.S = at<float>(ws, pl.S);
  ta.S_ld = pl.S_ld;
  ta.k = k;
  ta.out_idx = idx;
  ta.out_score = scores;
  ta.out_ld = k;
  return run_topk(cx, ta, pl, ws, p->L, nmm);
}

misa_status misa_hier_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t kprime,
                           int32_t k, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                           void* stream) {
  MISA_TRY(check_hier_args(p, A, heads, kprime, k, idx, scores));
  if (p->T == 0) return MISA_OK;
  const Plan pl = make_plan(p, MISA_OP_HIER_TOPK, A, kprime, k, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  return run_hier(LaunchCtx{static_cast<hipStream_t>(stream)}, p, pl, ws, A, heads, kprime, k, idx, scores);
}

misa_status misa_hier_topk_noalloc(const misa_problem* p, int32_t A, const int32_t* heads, int32_t kprime,
                                   int32_t k, int32_t* idx, float* scores, void* stream) {
  MISA_TRY(check_hier_args(p, A, heads, kprime, k, idx, scores));
  if (p->T == 0) return MISA_OK;
  const Plan pl = make_plan(p, MISA_OP_HIER_TOPK, A, kprime, k, 1);
  if (pl.total > kStaticScratchBytes)
    return fail(MISA_ERR_WORKSPACE,
                "this problem needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use misa_hier_topk with a caller workspace)", pl.total, (size_t)kStaticScratchBytes);
  void* ws = nullptr;
  MISA_TRY(static_scratch(&ws));
  return run_hier(LaunchCtx{static_cast<hipStream_t>(stream)}, p, pl, ws, A, heads, kprime, k, idx, scores);
}

misa_status hisa_topk(const misa_problem* p, int32_t m, int32_t k, int32_t* idx, float* scores,
                      void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  if (m < 1) return fail(MISA_ERR_INVALID_ARG, "m = %d must be >= 1", m);
  if (k < 1) return fail(MISA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(idx, "idx"));
  MISA_TRY(check_out(scores, "scores"));
  const Plan pl = make_plan(p, MISA_OP_HISA_TOPK, 1, 1, k, m);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  return run_hisa(cx, p, pl, ws, k, idx, scores, false);
}

misa_status hisa_block_scores(const misa_problem* p, float* beta, int64_t beta_ld, void* ws,
                              size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  const long long M = ((long long)p->L + p->B - 1) / p->B;
  if (beta_ld < M || beta_ld > (1ll << 30))
    return fail(MISA_ERR_INVALID_ARG, "beta_ld = %lld must lie in [ceil(L/B) = %lld, 2^30]", (long long)beta_ld, M);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(beta, "beta"));
  const Plan pl = make_plan(p, MISA_OP_BLOCK_SCORES, 1, 1, 1, 1);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  return run_route(cx, p, pl, ws, 1, nullptr, nullptr, beta, (int)beta_ld);
}

misa_status hisa_maxpool_topk(const misa_problem* p, int32_t m, int32_t k, int32_t* idx, float* scores,
                              void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  if (p->kbar) return fail(MISA_ERR_INVALID_ARG, "kbar must be NULL: cached means do not apply to max pooling");
  if (m < 1) return fail(MISA_ERR_INVALID_ARG, "m = %d must be >= 1", m);
  if (k < 1) return fail(MISA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(idx, "idx"));
  MISA_TRY(check_out(scores, "scores"));
  const Plan pl = make_plan(p, MISA_OP_HISA_TOPK, 1, 1, k, m);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  return run_hisa(cx, p, pl, ws, k, idx, scores, false, true);
}

misa_status misa_hisa_topk(const misa_problem* p, int32_t A, const int32_t* heads, int32_t m, int32_t k,
                           int32_t* idx, float* scores, void* ws, size_t ws_bytes, void* stream) {
  MISA_TRY(check_problem(p, true));
  if (A < 1 || A > p->H) return fail(MISA_ERR_INVALID_ARG, "A = %d must lie in [1, H = %d]", A, p->H);
  if (m < 1) return fail(MISA_ERR_INVALID_ARG, "m = %d must be >= 1", m);
  if (k < 1) return fail(MISA_ERR_INVALID_ARG, "k = %d must be >= 1", k);
  if (p->T == 0) return MISA_OK;
  MISA_TRY(check_out(idx, "idx"));
  MISA_TRY(check_out(scores, "scores"));
  if (heads && !aligned(heads, 4)) return fail(MISA_ERR_INVALID_ARG, "heads must be 4-byte aligned");
  const Plan pl = make_plan(p, MISA_OP_MISA_HISA_TOPK, A, 1, k, m);
  MISA_TRY(check_ws(pl, ws, ws_bytes));
  const LaunchCtx cx{static_cast<hipStream_t>(stream)};
  if (!heads && A == p->H)  // every head is routed: HISA itself
    return run_hisa(cx, p, pl, ws, k, idx, scores, false);
  uint16_t* qr = at<uint16_t>(ws, pl.qr);
  float* wr = at<float>(ws, pl.wr);
  if (heads)
    HIP_TRY(launch_gather_heads(cx, p->q, p->q_dtype == MISA_Q_FP8_E4M3FN, p->q_scale, p->w, heads, p->T, p->H, A,
                                qr, wr),
            "head gather");
  else  // the block sums and query tails stay for the block filter
    MISA_TRY(run_route(cx, p, pl, ws, A, at<int32_t>(ws, pl.heads), nullptr, nullptr, 0, qr, wr, false, false,
                       true));
  // both HISA stages with the routed heads: their packed rows stand in for q and w
  // (packed fp8 rows carry their scales: scale 1 from here on)
  misa_problem pr = *p;
  pr.q = qr;
  pr.w = wr;
  pr.H = A;
  pr.q_scale = nullptr;
  return run_hisa(cx, &pr, pl, ws, k, idx, scores, heads == nullptr);
}

const char* misa_status_str(int32_t status) {
  switch (status) {
    case MISA_OK: return "MISA_OK";
    case MISA_ERR_INVALID_ARG: return "MISA_ERR_INVALID_ARG";
    case MISA_ERR_UNSUPPORTED: return "MISA_ERR_UNSUPPORTED";
    case MISA_ERR_WORKSPACE: return "MISA_ERR_WORKSPACE";
    case MISA_ERR_HIP: return "MISA_ERR_HIP";
    default: return "unknown misa_status";
  }
}

const char* misa_last_error(void) { return g_last_error.c_str(); }

misa_status misa_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return MISA_OK;
}

misa_status misa_profile_read(const char* name_substr, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(MISA_ERR_INVALID_ARG, "total_ms and launches must be non-NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double sum = 0.0;
  int64_t n = 0;
  for (auto& r : g_prof) {
    if (name_substr && !strstr(r.name.c_str(), name_substr)) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return fail(MISA_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return fail(MISA_ERR_HIP, "event elapsed failed");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return MISA_OK;
}

misa_status misa_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_prof) {
    if (r.start) (void)hipEventDestroy(r.start);
    if (r.stop) (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  return MISA_OK;
}

}  // extern "C"
