// Per-query top-k selection (MISA technical summary, "Metodologia: MISA":
// the final tokens are the top-k of the reduced scores; the same selection
// keeps MISA-dagger's k' candidates and HISA's m blocks).
//
// Rule: keep the first min(k, n) items under (-score, index); -0.0 == +0.0.
// Scores become order-preserving 32-bit keys. A radix select over LDS
// histograms finds the exact k-th key tau and how many items equal to tau are
// still needed; it starts at the highest bit in which the row's keys differ, so
// the first histogram spreads the row over all bins. A wave-ballot compaction
// then emits the chosen items in ascending index order, so ties go to the lower
// index and the output is deterministic.
//
// Rows that fit in LDS are handled by one workgroup each. Longer rows are split
// over many workgroups: a histogram pass (bins spread between the row's
// smallest and largest key, which the scoring kernel reports), then a pass
// that keeps each chunk's items at or above the threshold bin in index order;
// the last workgroup of a row to finish gathers the survivors and selects.
#include "device_common.h"
#include "launch.h"

namespace misa {

constexpr int kLdsCap = 16384;     // items per row selected inside LDS
constexpr int kLongChunk = 8192;   // items per workgroup in the long-row passes
constexpr int kCoarseBits = 12;
constexpr int kCoarseBins = 1 << kCoarseBits;
constexpr int kListCap = 4096;     // survivors of the first radix digit kept in LDS
constexpr int kRankCap = 128;      // lists this short are ranked pairwise instead of by digits

template <int NT>
struct TopkShared {
  static constexpr int NW = NT / kWave;
  uint32_t hist[2048];
  int wave_tot[NW];
  int wgt[NW];
  int weq[NW];
  uint32_t wmin[NW];
  uint32_t wmax[NW];
  uint32_t umin, umax;
  int digit, rem;
  int flag;
  int nlist;
  uint32_t tau;
  int need;
  uint32_t list[kListCap];
};

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

__device__ __forceinline__ int row_length(const TopkArgs a, int row) {
  if (a.row_n) return a.row_n[row];
  return ceil_div_i(visible_len(a.pos[row], a.L), a.n_div);
}

// Block-wide inclusive scan; *total receives the block sum.
template <int NT>
__device__ __forceinline__ int block_scan(int v, TopkShared<NT>& sm, int* total) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) sm.wave_tot[w] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TopkShared<NT>::NW; ++i) {
    const int x = sm.wave_tot[i];
    off += i < w ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return inc + off;
}

template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, TopkShared<NT>& sm) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t a = __shfl_xor(lo, off, kWave), b = __shfl_xor(hi, off, kWave);
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
  }
  if (lane == 0) {
    sm.wmin[w] = lo;
    sm.wmax[w] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = sm.wmin[0], b = sm.wmax[0];
    for (int i = 1; i < TopkShared<NT>::NW; ++i) {
      a = sm.wmin[i] < a ? sm.wmin[i] : a;
      b = sm.wmax[i] > b ? sm.wmax[i] : b;
    }
    sm.umin = a;
    sm.umax = b;
  }
  __syncthreads();
}

// Locate the bin holding the rem-th largest item of hist[0, nb) (nb a power of
// two <= 4096, 1 <= rem <= total): sm.digit receives the bin and sm.rem the rank
// inside it. Each thread reads its (at most 16) bins with vector loads, one
// block scan orders the thread sums, and the owning thread finishes from
// registers.
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int rem, TopkShared<NT>& sm) {
  const int tid = threadIdx.x;
  const int per = nb >= NT ? nb / NT : 1;
  const bool act = tid < (nb >= NT ? NT : nb);
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) h[i] = 0u;
  if (act) {
    if (per >= 4) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * v < per) {
          const u32x4 x = reinterpret_cast<const u32x4*>(hist + tid * per)[v];
          h[4 * v] = x[0];
          h[4 * v + 1] = x[1];
          h[4 * v + 2] = x[2];
          h[4 * v + 3] = x[3];
        }
    } else if (per == 2) {
      const u32x2 x = reinterpret_cast<const u32x2*>(hist)[tid];
      h[0] = x[0];
      h[1] = x[1];
    } else {
      h[0] = hist[tid];
    }
  }
  int local = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) local += (int)h[i];
  int tot;
  const int inc = block_scan<NT>(local, sm, &tot);
  const int above = tot - inc;
  if (act && above < rem && rem <= above + local) {
    int cum = above;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      const int c = (int)h[i];
      if (i < per && cum < rem && cum + c >= rem) {
        sm.digit = tid * per + i;
        sm.rem = rem - cum;
      }
      cum += i < per ? c : 0;
    }
  }
  __syncthreads();
}

// tau = the rem-th largest of the c keys in sm.list (all-pairs count; c <=
// kRankCap) and need_eq = rem - #{keys > tau}.
template <int NT>
__device__ __forceinline__ void rank_in_list(int c, int rem, TopkShared<NT>& sm, uint32_t& tau,
                                             int& need_eq) {
  const int c4 = c & ~3;
  for (int e = threadIdx.x; e < c; e += NT) {
    const uint32_t ue = sm.list[e];
    int gt = 0, ge = 0;
    for (int f = 0; f < c4; f += 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&sm.list[f]);
      gt += (v[0] > ue) + (v[1] > ue) + (v[2] > ue) + (v[3] > ue);
      ge += (v[0] >= ue) + (v[1] >= ue) + (v[2] >= ue) + (v[3] >= ue);
    }
    for (int f = c4; f < c; ++f) {
      gt += sm.list[f] > ue;
      ge += sm.list[f] >= ue;
    }
    if (gt < rem && rem <= ge) {  // every such item has the same key
      sm.tau = ue;
      sm.need = rem - gt;
    }
  }
  __syncthreads();
  tau = sm.tau;
  need_eq = sm.need;
  __syncthreads();
}

// Exact k-th largest key of items [0, n) whose keys lie in [umin, umax]
// (requires 1 <= k < n). Returns tau and the number need_eq of items equal to
// tau that belong to the selection (the lowest-index ones).
// Digits are taken of the offset key v = u - umin, so the first 2048-bin pass
// spreads over the row's actual range. The chosen bin's items go to an LDS list;
// a short list is finished by pairwise ranking, a longer one by further digits.
template <int NT, typename KeyAt>
__device__ __forceinline__ void radix_threshold(KeyAt key_at, int n, int k, uint32_t umin, uint32_t umax,
                                                TopkShared<NT>& sm, uint32_t& tau, int& need_eq) {
  const int tid = threadIdx.x;
  const uint32_t span = umax - umin;
  int hi = span ? 32 - __clz(span) : 0;  // bits of the offset key in use
  uint32_t mask = hi >= 32 ? 0u : ~((1u << hi) - 1u);
  uint32_t prefix = 0u;  // of the offset key
  int rem = k;
  bool listed = false;
  int nl = 0;
  while (hi > 0) {
    const int w = hi < 11 ? hi : 11;
    const int sh = hi - w;
    const int nb = 1 << w;
    for (int b = tid; b < nb; b += NT) sm.hist[b] = 0u;
    if (tid == 0) sm.nlist = 0;
    __syncthreads();
    if (listed) {
      for (int i = tid; i < nl; i += NT) {
        const uint32_t v = sm.list[i] - umin;
        if ((v & mask) == prefix) atomicAdd(&sm.hist[(v >> sh) & (uint32_t)(nb - 1)], 1u);
      }
    } else {
      constexpr int U = 8;
      for (int base = 0; base < n; base += NT * U) {
        uint32_t v[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const int i = base + j * NT + tid;
          v[j] = i < n ? key_at(i) - umin : 0u;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          const int i = base + j * NT + tid;
          if (i < n && (v[j] & mask) == prefix) atomicAdd(&sm.hist[(v[j] >> sh) & (uint32_t)(nb - 1)], 1u);
        }
      }
    }
    __syncthreads();
    find_bin<NT>(sm.hist, nb, rem, sm);
    const uint32_t digit = (uint32_t)sm.digit;
    const int bin_count = (int)sm.hist[digit];
    prefix |= digit << sh;
    mask |= (uint32_t)(nb - 1) << sh;
    rem = sm.rem;
    hi = sh;
    __syncthreads();  // everyone has read the histogram
    if (hi > 0) {
      if (!listed && bin_count <= kListCap) {
        // keep only the chosen bin's items (as keys) for the remaining digits
        constexpr int U = 8;
        for (int base = 0; base < n; base += NT * U) {
          uint32_t u[U];
#pragma unroll
          for (int j = 0; j < U; ++j) {
            const int i = base + j * NT + tid;
            u[j] = i < n ? key_at(i) : 0u;
          }
#pragma unroll
          for (int j = 0; j < U; ++j) {
            const int i = base + j * NT + tid;
            const bool keep = i < n && ((u[j] - umin) & mask) == prefix;
            const uint64_t m = wave_ballot(keep);
            int at = 0;
            if ((threadIdx.x & 63) == 0 && m) at = atomicAdd(&sm.nlist, __popcll(m));
            at = __shfl(at, 0, kWave);
            if (keep) sm.list[at + lanes_below(m)] = u[j];
          }
        }
        __syncthreads();
        nl = bin_count;
        listed = true;
      } else if (listed && bin_count <= kRankCap) {
        // shrink the list to the items still matching (staged through hist)
        for (int i = tid; i < nl; i += NT) {
          const uint32_t u = sm.list[i];
          const bool keep = ((u - umin) & mask) == prefix;
          const uint64_t m = wave_ballot(keep);
          int at = 0;
          if ((threadIdx.x & 63) == 0 && m) at = atomicAdd(&sm.nlist, __popcll(m));
          at = __shfl(at, 0, kWave);
          if (keep) sm.hist[at + lanes_below(m)] = u;
        }
        __syncthreads();
        for (int i = tid; i < bin_count; i += NT) sm.list[i] = sm.hist[i];
        __syncthreads();
        nl = bin_count;
      }
      if (listed && nl <= kRankCap) {
        rank_in_list<NT>(nl, rem, sm, tau, need_eq);
        return;
      }
    }
  }
  tau = prefix + umin;
  need_eq = rem;
}

// Emit the selection in ascending item order: items with key > tau plus the
// first need_eq items equal to tau (every item when take_all). Each wave owns a
// contiguous segment; a count pass and a write pass keep the order.
template <int NT, bool TAKE_ALL, bool WITH_SCORE, typename KeyAt, typename IdxAt>
__device__ __forceinline__ void emit_ordered(KeyAt key_at, IdxAt idx_at, int n, uint32_t tau, int need_eq,
                                             TopkShared<NT>& sm, int32_t* out_idx, float* out_score) {
  constexpr int NW = TopkShared<NT>::NW;
  constexpr int U = 4;  // 64-item groups loaded before use
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = ceil_div_i(ceil_div_i(n, NW), kWave * U) * kWave * U;
  const int s0 = min(n, w * seg), s1 = min(n, s0 + seg);
  int gt = 0, eq = 0;
  if (TAKE_ALL) {
    gt = s1 - s0;
  } else {
    for (int base = s0; base < s1; base += kWave * U) {
      uint32_t u[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int i = base + j * kWave + lane;
        u[j] = i < s1 ? key_at(i) : 0u;
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const bool in = base + j * kWave + lane < s1;
        gt += __popcll(wave_ballot(in && u[j] > tau));
        eq += __popcll(wave_ballot(in && u[j] == tau));
      }
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
  for (int base = s0; base < s1; base += kWave * U) {
    uint32_t u[U];
    int32_t ix[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = base + j * kWave + lane;
      const bool in = i < s1;
      u[j] = in ? key_at(i) : 0u;
      ix[j] = in ? idx_at(i) : 0;
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const bool in = base + j * kWave + lane < s1;
      bool sel;
      if (TAKE_ALL) {
        sel = in;
      } else {
        const bool iseq = in && u[j] == tau;
        const uint64_t em = wave_ballot(iseq);
        sel = (in && u[j] > tau) || (iseq && eq_run + lanes_below(em) < need_eq);
        eq_run += __popcll(em);
      }
      const uint64_t smask = wave_ballot(sel);
      if (sel) {
        const int p = out + lanes_below(smask);
        out_idx[p] = ix[j];
        if (WITH_SCORE) out_score[p] = key_score(u[j]);
      }
      out += __popcll(smask);
    }
  }
  __syncthreads();
}

template <int NT, typename KeyAt, typename IdxAt>
__device__ __forceinline__ void select_row(KeyAt key_at, IdxAt idx_at, int n, int k, uint32_t umin,
                                           uint32_t umax, TopkShared<NT>& sm, int32_t* out_idx,
                                           float* out_score, int32_t* out_count) {
  const bool take_all = k >= n;
  uint32_t tau = 0u;
  int need_eq = 0;
  if (!take_all) radix_threshold<NT>(key_at, n, k, umin, umax, sm, tau, need_eq);
  if (take_all) {
    if (out_score) emit_ordered<NT, true, true>(key_at, idx_at, n, tau, need_eq, sm, out_idx, out_score);
    else emit_ordered<NT, true, false>(key_at, idx_at, n, tau, need_eq, sm, out_idx, out_score);
  } else {
    if (out_score) emit_ordered<NT, false, true>(key_at, idx_at, n, tau, need_eq, sm, out_idx, out_score);
    else emit_ordered<NT, false, false>(key_at, idx_at, n, tau, need_eq, sm, out_idx, out_score);
  }
  const int nsel = take_all ? n : k;
  for (int p = nsel + (int)threadIdx.x; p < k; p += NT) {
    out_idx[p] = -1;
    if (out_score) out_score[p] = -__builtin_huge_valf();
  }
  if (out_count && threadIdx.x == 0) *out_count = nsel;
}

// Load n scores (row start 16-byte aligned) as keys into LDS, tracking the
// smallest and largest key. Loads are issued U per thread before use.
template <int NT, int U>
__device__ __forceinline__ void load_keys(const float* src, int n, uint32_t* keys, uint32_t& lo,
                                          uint32_t& hi) {
  const int tid = threadIdx.x;
  const int n4 = n >> 2;
  const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
  for (int base = 0; base < n4; base += NT * U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      if (j < n4) v[u] = s4[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      if (j < n4) {
        const uint32_t a = score_key(v[u][0]), b = score_key(v[u][1]), c = score_key(v[u][2]),
                       d = score_key(v[u][3]);
        *reinterpret_cast<u32x4*>(&keys[4 * j]) = u32x4{a, b, c, d};
        lo = min(lo, min(min(a, b), min(c, d)));
        hi = max(hi, max(max(a, b), max(c, d)));
      }
    }
  }
  for (int i = 4 * n4 + tid; i < n; i += NT) {
    const uint32_t a = score_key(src[i]);
    keys[i] = a;
    lo = min(lo, a);
    hi = max(hi, a);
  }
}

template <int NT, int U>
__device__ __forceinline__ void load_ints(const int32_t* src, int n, int32_t* dst) {
  const int tid = threadIdx.x;
  const int n4 = n >> 2;
  const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
  for (int base = 0; base < n4; base += NT * U) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      if (j < n4) v[u] = s4[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NT + tid;
      if (j < n4) *reinterpret_cast<i32x4*>(&dst[4 * j]) = v[u];
    }
  }
  for (int i = 4 * n4 + tid; i < n; i += NT) dst[i] = src[i];
}

// One workgroup per row; the row's keys (and indices) are staged in LDS.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_rows(TopkArgs a, int cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.x;
  const int n = min(row_length(a, row), cap);
  uint32_t* keys = dyn;
  int32_t* idx = reinterpret_cast<int32_t*>(dyn + cap);
  uint32_t lo = 0xffffffffu, hi = 0u;
  load_keys<NT, 4>(a.S + (size_t)row * a.S_ld, n, keys, lo, hi);
  if (a.row_idx) load_ints<NT, 4>(a.row_idx + (size_t)row * a.idx_ld, n, idx);
  block_minmax<NT>(lo, hi, sm);
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  int32_t* oc = a.out_count ? a.out_count + row : nullptr;
  auto key_at = [=](int i) { return keys[i]; };
  if (a.row_idx) {
    auto idx_at = [=](int i) { return idx[i]; };
    select_row<NT>(key_at, idx_at, n, a.k, sm.umin, sm.umax, sm, oi, os, oc);
  } else {
    auto idx_at = [=](int i) { return i; };
    select_row<NT>(key_at, idx_at, n, a.k, sm.umin, sm.umax, sm, oi, os, oc);
  }
}

// ---------------------------------------------------------------------------
// Long rows.

// Row key range from the scoring kernel's per-split partial ranges
// (layout [nmm][rows][2] = {min, max}).
template <int NT>
__device__ __forceinline__ void row_range(const uint32_t* rmm, int nmm, int rows, int row,
                                          TopkShared<NT>& sm) {
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < nmm; i += NT) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(rmm + ((size_t)i * rows + row) * 2);
    lo = min(lo, v[0]);
    hi = max(hi, v[1]);
  }
  block_minmax<NT>(lo, hi, sm);
}

__device__ __forceinline__ int range_shift(uint32_t umin, uint32_t umax) {
  const uint32_t span = umax - umin;
  const int bits = span ? 32 - __clz(span) : 0;
  return bits > kCoarseBits ? bits - kCoarseBits : 0;
}

// grid (nchunk, rows): histogram of (key - umin) >> shift, summed in ghist.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_hist(TopkArgs a, const uint32_t* rmm, int nmm,
                                                  uint32_t* ghist) {
  __shared__ uint32_t lh[kCoarseBins];
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int n = row_length(a, row);
  const int s0 = chunk * kLongChunk, s1 = min(n, s0 + kLongChunk);
  if (s0 >= s1) return;
  row_range<NT>(rmm, nmm, a.rows, row, sm);
  const uint32_t umin = sm.umin;
  const int sh = range_shift(umin, sm.umax);
  for (int b = threadIdx.x; b < kCoarseBins; b += NT) lh[b] = 0u;
  __syncthreads();
  constexpr int U = kLongChunk / 4 / NT;
  const f32x4* s4 = reinterpret_cast<const f32x4*>(a.S + (size_t)row * a.S_ld + s0);
  const int m4 = (s1 - s0) >> 2;
  f32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = u * NT + threadIdx.x;
    if (j < m4) v[u] = s4[j];
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = u * NT + threadIdx.x;
    if (j < m4) {
      atomicAdd(&lh[(score_key(v[u][0]) - umin) >> sh], 1u);
      atomicAdd(&lh[(score_key(v[u][1]) - umin) >> sh], 1u);
      atomicAdd(&lh[(score_key(v[u][2]) - umin) >> sh], 1u);
      atomicAdd(&lh[(score_key(v[u][3]) - umin) >> sh], 1u);
    }
  }
  const float* src = a.S + (size_t)row * a.S_ld;
  for (int i = s0 + 4 * m4 + threadIdx.x; i < s1; i += NT) atomicAdd(&lh[(score_key(src[i]) - umin) >> sh], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (size_t)row * kCoarseBins;
  for (int b = threadIdx.x; b < kCoarseBins; b += NT)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// grid (nchunk, rows): keep, in index order, this chunk's items whose bin is
// at or above the row's threshold bin (everything when k >= n); the last
// workgroup of the row to finish gathers all survivors in chunk order and
// selects the top-k.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_filter_select(TopkArgs a, const uint32_t* rmm, int nmm,
                                                          const uint32_t* ghist, uint32_t* rkeys,
                                                          int32_t* ridx, int32_t* rcnt,
                                                          uint32_t* done, int nchunk, long long rld,
                                                          uint32_t* gkeys, int32_t* gidx, int cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ TopkShared<NT> sm;
  __shared__ int coff[1025];
  constexpr int NW = TopkShared<NT>::NW;
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = row_length(a, row);
  row_range<NT>(rmm, nmm, a.rows, row, sm);
  const uint32_t umin = sm.umin, umax = sm.umax;
  const int sh = range_shift(umin, umax);
  uint32_t bstar = 0u;
  if (a.k < n) {
    // the row histogram, staged in LDS after the chunk area
    uint32_t* gh = dyn + kLongChunk;
    const u32x4* src = reinterpret_cast<const u32x4*>(ghist + (size_t)row * kCoarseBins);
    for (int i = tid; i < kCoarseBins / 4; i += NT) reinterpret_cast<u32x4*>(gh)[i] = src[i];
    __syncthreads();
    find_bin<NT>(gh, kCoarseBins, a.k, sm);
    bstar = (uint32_t)sm.digit;
  }
  const int s0 = chunk * kLongChunk, s1 = min(n, s0 + kLongChunk);
  int total = 0;
  if (s0 < s1) {
    // stage the chunk's keys in LDS, then count and write survivors in order
    uint32_t* ck = dyn;
    uint32_t lo = 0u, hi = 0u;
    const int len = s1 - s0;
    load_keys<NT, kLongChunk / 4 / NT>(a.S + (size_t)row * a.S_ld + s0, len, ck, lo, hi);
    __syncthreads();
    const int seg = ceil_div_i(ceil_div_i(len, NW), kWave) * kWave;
    const int w0 = min(len, w * seg), w1 = min(len, w0 + seg);
    int cnt = 0;
    for (int base = w0; base < w1; base += kWave) {
      const int i = base + lane;
      cnt += __popcll(wave_ballot(i < w1 && ((ck[i] - umin) >> sh) >= bstar));
    }
    if (lane == 0) sm.wgt[w] = cnt;
    __syncthreads();
    int out = 0;
    for (int i = 0; i < NW; ++i) {
      out += i < w ? sm.wgt[i] : 0;
      total += sm.wgt[i];
    }
    uint32_t* kd = rkeys + (size_t)row * rld + s0;
    int32_t* id = ridx + (size_t)row * rld + s0;
    for (int base = w0; base < w1; base += kWave) {
      const int i = base + lane;
      const uint32_t u = i < w1 ? ck[i] : 0u;
      const bool keep = i < w1 && ((u - umin) >> sh) >= bstar;
      const uint64_t m = wave_ballot(keep);
      if (keep) {
        const int p = out + lanes_below(m);
        kd[p] = u;
        id[p] = s0 + i;
      }
      out += __popcll(m);
    }
  }
  // publish this chunk and find out whether it is the row's last one
  __syncthreads();
  if (tid == 0) {
    rcnt[(size_t)row * nchunk + chunk] = total;
    __threadfence();
    const uint32_t prev = atomicAdd(&done[row], 1u);
    sm.flag = prev == (uint32_t)(nchunk - 1);
  }
  __syncthreads();
  if (!sm.flag) return;
  __threadfence();
  // last workgroup of the row: offsets of every chunk's survivors
  for (int c = tid; c < nchunk; c += NT)
    coff[c + 1] = __hip_atomic_load(&rcnt[(size_t)row * nchunk + c], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) {
    coff[0] = 0;
    done[row] = 0u;  // ready for the next call
  }
  __syncthreads();
  if (tid == 0)
    for (int c = 0; c < nchunk; ++c) coff[c + 1] += coff[c];
  __syncthreads();
  const int C = coff[nchunk];
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  int32_t* oc = a.out_count ? a.out_count + row : nullptr;
  // copy every chunk's survivors, in chunk order, to keys[0, C) / idx[0, C)
  auto gather = [&](uint32_t* keys, int32_t* idx) {
    uint32_t lo = 0xffffffffu, hi = 0u;
    constexpr int U = 4;
    for (int base = 0; base < C; base += NT * U) {
      uint32_t kv[U];
      int32_t iv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * NT + tid;
        if (j < C) {
          int lo_c = 0, hi_c = nchunk - 1;  // chunk c with coff[c] <= j < coff[c+1]
          while (lo_c < hi_c) {
            const int mid = (lo_c + hi_c + 1) >> 1;
            if (coff[mid] <= j) lo_c = mid; else hi_c = mid - 1;
          }
          const size_t at = (size_t)row * rld + (size_t)lo_c * kLongChunk + (j - coff[lo_c]);
          kv[u] = rkeys[at];
          iv[u] = ridx[at];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = base + u * NT + tid;
        if (j < C) {
          keys[j] = kv[u];
          idx[j] = iv[u];
          lo = min(lo, kv[u]);
          hi = max(hi, kv[u]);
        }
      }
    }
    block_minmax<NT>(lo, hi, sm);
  };
  if (C <= cap) {
    uint32_t* keys = dyn;
    int32_t* idx = reinterpret_cast<int32_t*>(dyn + cap);
    gather(keys, idx);
    auto key_at = [=](int i) { return keys[i]; };
    auto idx_at = [=](int i) { return idx[i]; };
    select_row<NT>(key_at, idx_at, C, a.k, sm.umin, sm.umax, sm, oi, os, oc);
  } else {
    // more survivors than LDS holds (heavy ties): select from a global copy
    uint32_t* keys = gkeys + (size_t)row * rld;
    int32_t* idx = gidx + (size_t)row * rld;
    gather(keys, idx);
    __threadfence_block();
    __syncthreads();
    auto key_at = [=](int i) { return keys[i]; };
    auto idx_at = [=](int i) { return idx[i]; };
    select_row<NT>(key_at, idx_at, C, a.k, sm.umin, sm.umax, sm, oi, os, oc);
  }
}

// grid (nchunk, rows): {min, max} score key of each chunk into rmm[chunk, row];
// workgroup (0, 0) also clears `zero`.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_range(TopkArgs a, uint32_t* rmm, uint32_t* zero,
                                                   long long zero_n) {
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.y, chunk = blockIdx.x;
  if (zero && row == 0 && chunk == 0)
    for (long long i = threadIdx.x; i < zero_n; i += NT) zero[i] = 0u;
  const int n = row_length(a, row);
  const int s0 = chunk * kLongChunk, s1 = min(n, s0 + kLongChunk);
  uint32_t lo = 0xffffffffu, hi = 0u;
  const float* src = a.S + (size_t)row * a.S_ld;
  for (int i = s0 + threadIdx.x; i < s1; i += NT) {
    const uint32_t u = score_key(src[i]);
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_minmax<NT>(lo, hi, sm);
  if (threadIdx.x == 0) {
    rmm[((size_t)chunk * a.rows + row) * 2] = sm.umin;
    rmm[((size_t)chunk * a.rows + row) * 2 + 1] = sm.umax;
  }
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
  __shared__ int offs[1025];
  const int t = blockIdx.x;
  const int n = visible_len(pos[t], L);
  const int nb = min(nblocks[t], 1024);
  const int32_t* bl = blocks + (size_t)t * m;
  auto size_of = [&](int j) {
    const long long s0 = (long long)bl[j] * B;
    return (int)(n - s0 < B ? n - s0 : B);
  };
  if (threadIdx.x == 0) {
    int off = 0;
    for (int j = 0; j < nb; ++j) {
      offs[j] = off;
      off += size_of(j);
    }
    offs[nb] = off;
    ncand[t] = off;
  }
  __syncthreads();
  const int total = offs[nb];
  for (int i = threadIdx.x; i < total; i += 256) {
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offs[mid] <= i) lo = mid; else hi = mid - 1;
    }
    cand[(size_t)t * cand_ld + i] = (int32_t)((long long)bl[lo] * B + (i - offs[lo]));
  }
}

// ---------------------------------------------------------------------------
// Host launchers.

int topk_lds_cap() { return kLdsCap; }
int topk_long_chunk() { return kLongChunk; }
int topk_coarse_bins() { return kCoarseBins; }
int topk_long_chunks(int max_n) { return max_n <= 0 ? 1 : (max_n + kLongChunk - 1) / kLongChunk; }

template <int NT>
static hipError_t rows_launch(const LaunchCtx& cx, const TopkArgs& a, int cap) {
  const size_t shmem = (size_t)cap * 4u * (a.row_idx ? 2u : 1u);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_rows<NT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kLdsCap * 8));
    attr_set = true;
  }
  return cx.launch("topk_rows", k_topk_rows<NT>, dim3(a.rows), dim3(NT), shmem, a, cap);
}

hipError_t launch_topk_rows(const LaunchCtx& cx, const TopkArgs& a, int max_n) {
  if (a.rows == 0) return hipSuccess;
  int cap = max_n < 64 ? 64 : ((max_n + 63) / 64) * 64;
  if (cap > kLdsCap) cap = kLdsCap;
  // few rows: wide workgroups; many rows (prefill): several workgroups per CU
  if (a.rows <= 1024) return rows_launch<1024>(cx, a, cap);
  return rows_launch<256>(cx, a, cap);
}

hipError_t launch_topk_long(const LaunchCtx& cx, const TopkArgs& a, const TopkLongWs& ws, int max_n) {
  if (a.rows == 0) return hipSuccess;
  const int nch = topk_long_chunks(max_n);
  if (nch > 1024) return hipErrorInvalidValue;
  const long long rld = (long long)nch * kLongChunk;
  hipError_t e = cx.launch("topk_hist", k_topk_hist<256>, dim3(nch, a.rows), dim3(256), 0, a,
                           (const uint32_t*)ws.rmm, ws.nmm, ws.ghist);
  if (e != hipSuccess) return e;
  const size_t shmem = (size_t)kLdsCap * 8;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_filter_select<1024>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    attr_set = true;
  }
  return cx.launch("topk_filter_select", k_topk_filter_select<1024>, dim3(nch, a.rows), dim3(1024),
                   shmem, a, (const uint32_t*)ws.rmm, ws.nmm, (const uint32_t*)ws.ghist, ws.rkeys,
                   ws.ridx, ws.rcnt, ws.done, nch, rld, ws.gkeys, ws.gidx, kLdsCap);
}

hipError_t launch_topk_range(const LaunchCtx& cx, const TopkArgs& a, uint32_t* rmm_out,
                             uint32_t* zero, long long zero_n, int max_n) {
  if (a.rows == 0) return hipSuccess;
  const int nch = topk_long_chunks(max_n);
  return cx.launch("topk_range", k_topk_range<256>, dim3(nch, a.rows), dim3(256), 0, a, rmm_out,
                   zero, zero_n);
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
  if (m > 1024) return hipErrorInvalidValue;
  return cx.launch("expand_blocks", k_expand_blocks, dim3(T), dim3(256), 0, blocks, nblocks, m, pos,
                   L, B, cand, cand_ld, ncand);
}

}  // namespace misa
