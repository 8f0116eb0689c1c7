// Per-query top-k selection (MISA technical summary, "Metodologia: MISA":
// the final tokens are the top-k of the reduced scores; the same selection
// keeps MISA-dagger's k' candidates and HISA's m blocks).
//
// Rule: keep the first min(k, n) items under (-score, index); -0.0 == +0.0.
// Scores become order-preserving 32-bit keys; a three-digit (11/11/10-bit)
// radix pass over LDS histograms finds the exact k-th key tau and how many
// items equal to tau are still needed; a wave-ballot compaction then emits the
// chosen items in ascending index order, so ties go to the lower index and the
// output is deterministic.
//
// Rows that fit in LDS are handled by one workgroup each. Longer rows first go
// through a many-workgroup 12-bit histogram and an ordered prefilter that keeps
// only the items at or above the threshold bin, then the per-row selection runs
// on those candidates.
#include "device_common.h"
#include "launch.h"

namespace misa {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kLdsCap = 16384;       // items per row selected inside LDS
constexpr int kLongChunk = 8192;     // items per workgroup in the long-row prefilter
constexpr int kCoarseBins = 4096;    // prefilter histogram: top 12 key bits

struct TopkShared {
  uint32_t hist[2048];
  int wave_tot[kTopkWaves];
  int wgt[kTopkWaves];
  int weq[kTopkWaves];
  int digit;
  int rem;
};

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int row_length(const TopkArgs& a, int row) {
  if (a.row_n) return a.row_n[row];
  return ceil_div_i(visible_len(a.pos[row], a.L), a.n_div);
}

// Block-wide inclusive scan (256 threads); *total receives the block sum.
__device__ __forceinline__ int block_scan(int v, int* wave_tot, int* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) wave_tot[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const int x = wave_tot[i];
    off += i < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return inc + off;
}

// Exact k-th largest key of items [0, n) (requires 1 <= k < n). On return
// tau is that key and need_eq the number of items equal to tau that belong to
// the selection (the lowest-index ones).
template <typename KeyAt>
__device__ void radix_threshold(KeyAt key_at, int n, int k, TopkShared& sm, uint32_t& tau,
                                int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int rem = k;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbits = pass == 2 ? 10 : 11;
    const int nb = 1 << nbits;
    for (int b = tid; b < 2048; b += kTopkThreads) sm.hist[b] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = key_at(i);
      if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> sh) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    const int per = nb / kTopkThreads;
    int local = 0;
    for (int j = 0; j < per; ++j) local += (int)sm.hist[tid * per + j];
    int tot;
    const int inc = block_scan(local, sm.wave_tot, &tot);
    const int above = tot - inc;
    if (above < rem && rem <= above + local) {
      int cum = above;
      for (int j = per - 1; j >= 0; --j) {
        const int c = (int)sm.hist[tid * per + j];
        if (cum + c >= rem) {
          sm.digit = tid * per + j;
          sm.rem = rem - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sm.digit << sh;
    mask |= (uint32_t)(nb - 1) << sh;
    rem = sm.rem;
    __syncthreads();
  }
  tau = prefix;
  need_eq = rem;
}

// Emit the selection in ascending item order: items with key > tau, plus the
// first need_eq items with key == tau (all items when take_all). Each wave
// owns a contiguous segment; a count pass and a write pass keep the order.
template <typename KeyAt, typename IdxAt>
__device__ void emit_ordered(KeyAt key_at, IdxAt idx_at, int n, uint32_t tau, int need_eq,
                             bool take_all, TopkShared& sm, int32_t* out_idx, float* out_score) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = ceil_div_i(ceil_div_i(n, kTopkWaves), kWave) * kWave;
  const int s0 = min(n, w * seg), s1 = min(n, s0 + seg);
  int gt = 0, eq = 0;
  if (take_all) {
    gt = s1 - s0;
  } else {
    for (int base = s0; base < s1; base += kWave) {
      const int i = base + lane;
      const bool in = i < s1;
      const uint32_t u = in ? key_at(i) : 0u;
      gt += __popcll(wave_ballot(in && u > tau));
      eq += __popcll(wave_ballot(in && u == tau));
    }
  }
  if (lane == 0) {
    sm.wgt[w] = gt;
    sm.weq[w] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
  for (int i = 0; i < w; ++i) {
    gt_before += sm.wgt[i];
    eq_before += sm.weq[i];
  }
  int out = gt_before + min(eq_before, need_eq);
  int eq_run = eq_before;
  for (int base = s0; base < s1; base += kWave) {
    const int i = base + lane;
    const bool in = i < s1;
    const uint32_t u = in ? key_at(i) : 0u;
    bool sel;
    if (take_all) {
      sel = in;
    } else {
      const bool iseq = in && u == tau;
      const uint64_t em = wave_ballot(iseq);
      sel = (in && u > tau) || (iseq && eq_run + lanes_below(em) < need_eq);
      eq_run += __popcll(em);
    }
    const uint64_t smask = wave_ballot(sel);
    if (sel) {
      const int p = out + lanes_below(smask);
      out_idx[p] = idx_at(i);
      if (out_score) out_score[p] = key_score(u);
    }
    out += __popcll(smask);
  }
  __syncthreads();
}

template <typename KeyAt, typename IdxAt>
__device__ void select_row(KeyAt key_at, IdxAt idx_at, int n, int k, TopkShared& sm,
                           int32_t* out_idx, float* out_score, int32_t* out_count) {
  const bool take_all = k >= n;
  uint32_t tau = 0u;
  int need_eq = 0;
  if (!take_all) radix_threshold(key_at, n, k, sm, tau, need_eq);
  emit_ordered(key_at, idx_at, n, tau, need_eq, take_all, sm, out_idx, out_score);
  const int nsel = take_all ? n : k;
  for (int p = nsel + (int)threadIdx.x; p < k; p += kTopkThreads) {
    out_idx[p] = -1;
    if (out_score) out_score[p] = -__builtin_huge_valf();
  }
  if (out_count && threadIdx.x == 0) *out_count = nsel;
}

// One workgroup per row; the row's keys (and indices) are staged in LDS.
__global__ __launch_bounds__(kTopkThreads) void k_topk_rows(TopkArgs a, int cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ TopkShared sm;
  const int row = blockIdx.x;
  const int n = min(row_length(a, row), cap);
  uint32_t* keys = dyn;
  int32_t* idx = reinterpret_cast<int32_t*>(dyn + cap);
  const float* src = a.S + (size_t)row * a.S_ld;
  for (int i = threadIdx.x; i < n; i += kTopkThreads) keys[i] = score_key(src[i]);
  if (a.row_idx) {
    const int32_t* isrc = a.row_idx + (size_t)row * a.idx_ld;
    for (int i = threadIdx.x; i < n; i += kTopkThreads) idx[i] = isrc[i];
  }
  __syncthreads();
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  int32_t* oc = a.out_count ? a.out_count + row : nullptr;
  auto key_at = [&](int i) { return keys[i]; };
  if (a.row_idx) {
    auto idx_at = [&](int i) { return idx[i]; };
    select_row(key_at, idx_at, n, a.k, sm, oi, os, oc);
  } else {
    auto idx_at = [&](int i) { return i; };
    select_row(key_at, idx_at, n, a.k, sm, oi, os, oc);
  }
}

// ---------------------------------------------------------------------------
// Long rows.

// grid (nchunk, rows): coarse 12-bit histogram of each row, summed in ghist.
__global__ __launch_bounds__(kTopkThreads) void k_topk_hist(TopkArgs a, uint32_t* ghist) {
  __shared__ uint32_t lh[kCoarseBins];
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int n = row_length(a, row);
  const int s0 = chunk * kLongChunk, s1 = min(n, s0 + kLongChunk);
  if (s0 >= s1) return;
  for (int b = threadIdx.x; b < kCoarseBins; b += kTopkThreads) lh[b] = 0u;
  __syncthreads();
  const float* src = a.S + (size_t)row * a.S_ld;
  for (int i = s0 + threadIdx.x; i < s1; i += kTopkThreads) atomicAdd(&lh[score_key(src[i]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (size_t)row * kCoarseBins;
  for (int b = threadIdx.x; b < kCoarseBins; b += kTopkThreads)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// grid (nchunk, rows): keep, in index order, the items of this chunk whose
// coarse bin is at or above the row's threshold bin (the bin holding the k-th
// largest key); everything is kept when k >= n.
__global__ __launch_bounds__(kTopkThreads) void k_topk_filter(TopkArgs a, const uint32_t* ghist,
                                                             uint32_t* rkeys, int32_t* ridx,
                                                             int32_t* rcnt, int nchunk,
                                                             long long rld) {
  __shared__ TopkShared sm;
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int n = row_length(a, row);
  const int tid = threadIdx.x;
  uint32_t bstar = 0u;
  if (a.k < n) {
    constexpr int per = kCoarseBins / kTopkThreads;
    const uint32_t* gh = ghist + (size_t)row * kCoarseBins;
    int local = 0;
    for (int j = 0; j < per; ++j) local += (int)gh[tid * per + j];
    int tot;
    const int inc = block_scan(local, sm.wave_tot, &tot);
    const int above = tot - inc;
    if (above < a.k && a.k <= above + local) {
      int cum = above;
      for (int j = per - 1; j >= 0; --j) {
        const int c = (int)gh[tid * per + j];
        if (cum + c >= a.k) {
          sm.digit = tid * per + j;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    bstar = (uint32_t)sm.digit;
  }
  const int s0 = chunk * kLongChunk, s1 = min(n, s0 + kLongChunk);
  int32_t* cnt_out = rcnt + (size_t)row * nchunk + chunk;
  if (s0 >= s1) {
    if (tid == 0) *cnt_out = 0;
    return;
  }
  const float* src = a.S + (size_t)row * a.S_ld;
  uint32_t* kd = rkeys + (size_t)row * rld + s0;
  int32_t* id = ridx + (size_t)row * rld + s0;
  const int w = tid >> 6, lane = tid & 63;
  const int len = s1 - s0;
  const int seg = ceil_div_i(ceil_div_i(len, kTopkWaves), kWave) * kWave;
  const int w0 = s0 + min(len, w * seg), w1 = s0 + min(len, w * seg + seg);
  int cnt = 0;
  for (int base = w0; base < w1; base += kWave) {
    const int i = base + lane;
    const bool keep = i < w1 && (score_key(src[i]) >> 20) >= bstar;
    cnt += __popcll(wave_ballot(keep));
  }
  if (lane == 0) sm.wgt[w] = cnt;
  __syncthreads();
  int out = 0, total = 0;
  for (int i = 0; i < kTopkWaves; ++i) {
    out += i < w ? sm.wgt[i] : 0;
    total += sm.wgt[i];
  }
  for (int base = w0; base < w1; base += kWave) {
    const int i = base + lane;
    uint32_t u = 0u;
    bool keep = false;
    if (i < w1) {
      u = score_key(src[i]);
      keep = (u >> 20) >= bstar;
    }
    const uint64_t m = wave_ballot(keep);
    if (keep) {
      const int p = out + lanes_below(m);
      kd[p] = u;
      id[p] = i;
    }
    out += __popcll(m);
  }
  if (tid == 0) *cnt_out = total;
}

// One workgroup per row: gather the prefiltered candidates in index order
// (into LDS when they fit, else into a contiguous global copy) and select.
__global__ __launch_bounds__(kTopkThreads) void k_topk_select(TopkArgs a, const uint32_t* rkeys,
                                                             const int32_t* ridx,
                                                             const int32_t* rcnt, int nchunk,
                                                             long long rld, uint32_t* gkeys,
                                                             int32_t* gidx, int cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ TopkShared sm;
  const int row = blockIdx.x;
  const int32_t* cnts = rcnt + (size_t)row * nchunk;
  int C = 0;
  for (int c = 0; c < nchunk; ++c) C += cnts[c];
  const bool in_lds = C <= cap;
  uint32_t* keys = in_lds ? dyn : gkeys + (size_t)row * rld;
  int32_t* idx = in_lds ? reinterpret_cast<int32_t*>(dyn + cap) : gidx + (size_t)row * rld;
  int off = 0;
  for (int c = 0; c < nchunk; ++c) {
    const int cc = cnts[c];
    const uint32_t* ks = rkeys + (size_t)row * rld + (size_t)c * kLongChunk;
    const int32_t* is = ridx + (size_t)row * rld + (size_t)c * kLongChunk;
    for (int j = threadIdx.x; j < cc; j += kTopkThreads) {
      keys[off + j] = ks[j];
      idx[off + j] = is[j];
    }
    off += cc;
  }
  __syncthreads();
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  int32_t* oc = a.out_count ? a.out_count + row : nullptr;
  auto key_at = [&](int i) { return keys[i]; };
  auto idx_at = [&](int i) { return idx[i]; };
  select_row(key_at, idx_at, C, a.k, sm, oi, os, oc);
}

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// HISA Stage 2 candidate list: the visible tokens of the chosen blocks, in
// ascending order (blocks arrive ascending).
__global__ __launch_bounds__(256) void k_expand_blocks(const int32_t* blocks, const int32_t* nblocks,
                                                       int m, const int32_t* pos, int L, int B,
                                                       int32_t* cand, long long cand_ld,
                                                       int32_t* ncand) {
  const int t = blockIdx.x;
  const int n = visible_len(pos[t], L);
  const int nb = nblocks[t];
  int off = 0;
  for (int j = 0; j < nb; ++j) {
    const int b = blocks[(size_t)t * m + j];
    const long long s0 = (long long)b * B;
    const int sz = (int)(n - s0 < B ? n - s0 : B);
    for (int u = threadIdx.x; u < sz; u += 256) cand[(size_t)t * cand_ld + off + u] = (int32_t)(s0 + u);
    off += sz;
  }
  if (threadIdx.x == 0) ncand[t] = off;
}

// ---------------------------------------------------------------------------
// Host launchers.

int topk_lds_cap() { return kLdsCap; }
int topk_long_chunk() { return kLongChunk; }
int topk_coarse_bins() { return kCoarseBins; }

int topk_long_chunks(int max_n) { return max_n <= 0 ? 1 : (max_n + kLongChunk - 1) / kLongChunk; }

static size_t rows_lds_bytes(int cap, bool with_idx) {
  return (size_t)cap * 4u * (with_idx ? 2u : 1u);
}

hipError_t launch_topk_rows(const LaunchCtx& cx, const TopkArgs& a, int max_n) {
  if (a.rows == 0) return hipSuccess;
  int cap = max_n < 64 ? 64 : ((max_n + 63) / 64) * 64;
  if (cap > kLdsCap) cap = kLdsCap;
  const size_t shmem = rows_lds_bytes(cap, true);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_rows),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  return cx.launch("topk_rows", k_topk_rows, dim3(a.rows), dim3(kTopkThreads), shmem, a, cap);
}

hipError_t launch_topk_long(const LaunchCtx& cx, const TopkArgs& a, const TopkLongWs& ws,
                            int max_n) {
  if (a.rows == 0) return hipSuccess;
  const int nch = topk_long_chunks(max_n);
  const long long rld = (long long)nch * kLongChunk;
  hipError_t e = launch_fill_u32(cx, ws.ghist, (size_t)a.rows * kCoarseBins, 0u);
  if (e != hipSuccess) return e;
  e = cx.launch("topk_hist", k_topk_hist, dim3(nch, a.rows), dim3(kTopkThreads), 0, a, ws.ghist);
  if (e != hipSuccess) return e;
  e = cx.launch("topk_filter", k_topk_filter, dim3(nch, a.rows), dim3(kTopkThreads), 0, a,
                (const uint32_t*)ws.ghist, ws.rkeys, ws.ridx, ws.rcnt, nch, rld);
  if (e != hipSuccess) return e;
  const size_t shmem = rows_lds_bytes(kLdsCap, true);
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_select),
                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
  return cx.launch("topk_select", k_topk_select, dim3(a.rows), dim3(kTopkThreads), shmem, a,
                   (const uint32_t*)ws.rkeys, (const int32_t*)ws.ridx, (const int32_t*)ws.rcnt, nch,
                   rld, ws.gkeys, ws.gidx, kLdsCap);
}

hipError_t launch_fill_u32(const LaunchCtx& cx, uint32_t* p, size_t n, uint32_t v) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  return cx.launch("fill", k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, p, n, v);
}

hipError_t launch_expand_blocks(const LaunchCtx& cx, const int32_t* blocks, const int32_t* nblocks,
                                int m, const int32_t* pos, int L, int B, int T, int32_t* cand,
                                long long cand_ld, int32_t* ncand) {
  if (T == 0) return hipSuccess;
  return cx.launch("expand_blocks", k_expand_blocks, dim3(T), dim3(256), 0, blocks, nblocks, m, pos,
                   L, B, cand, cand_ld, ncand);
}

}  // namespace misa
