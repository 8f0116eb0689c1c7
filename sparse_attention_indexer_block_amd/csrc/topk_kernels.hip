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
// over many workgroups: a coarse histogram (bins spread between the row's
// smallest and largest key, which the scoring kernel reports) locates the
// threshold bin; only that bin's items are ranked exactly; every chunk then
// writes its kept items at an offset from a per-chunk prefix count.
#include "device_common.h"
#include "launch.h"

namespace misa {

constexpr int kLdsCap = 16384;     // items per row selected inside LDS
constexpr int kChunk = 2048;       // items per workgroup in the long-row passes
constexpr int kMaxChunks = 4096;   // chunks per long row (rows up to 2^23 items)
constexpr int kBoundaryCap = 4096; // boundary-bin items resolved inside LDS
constexpr int kCoarseBits = 10;
constexpr int kCoarseBins = 1 << kCoarseBits;  // long rows: bins of the first pass
constexpr int kFineBins = 2048;                  // rows in one workgroup
constexpr int kListCap = 4096;     // survivors of the first radix digit kept in LDS
constexpr int kRankCap = 128;      // lists this short are ranked pairwise instead of by digits
constexpr int kPairCap = 64;       // threshold bins this short are ranked pairwise directly

template <int NT>
struct RegShared {
  static constexpr int NW = NT / kWave;
  uint32_t red[NW][8];
  uint32_t wmin[NW], wmax[NW];
  int wgt[NW], weq[NW];
  uint32_t umin, umax;
  uint32_t base;
  int rem;
};

template <int NT>
struct alignas(16) TopkShared {
  static constexpr int NW = NT / kWave;
  alignas(16) uint32_t hist[2048];
  int wave_tot[NW];
  int wgt[NW];
  int weq[NW];
  uint32_t wmin[NW];
  uint32_t wmax[NW];
  uint32_t umin, umax;
  int digit, rem;
  int flag;
  int nlist;
  int ncand;            // keys of the threshold bin gathered so far
  uint32_t cmin, cmax;  // and their extremes
  uint32_t tau;
  int need;
  alignas(16) uint32_t list[kListCap];
  RegShared<NT> reg;
};

__device__ __forceinline__ int ceil_div_i(int a, int b) { return (a + b - 1) / b; }

// First-pass bins are linear in the score between the row's smallest and
// largest values (monotone in the score, so a bin holds a contiguous range of
// keys); a zero or non-finite span puts everything in bin 0.
__device__ __forceinline__ float lin_scale(float lo, float hi, int nb) {
  const float span = hi - lo;
  return (span > 0.f && span < __builtin_huge_valf()) ? (float)nb / span : 0.f;
}
__device__ __forceinline__ uint32_t lin_bin(uint32_t key, float lo, float scale, int nb) {
  const float f = (key_score(key) - lo) * scale;
  return (uint32_t)fminf(fmaxf(f, 0.f), (float)(nb - 1));
}

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
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    sm.wmin[w] = lo;
    sm.wmax[w] = hi;
  }
  __syncthreads();
  // every thread folds the per-wave extremes itself and stores the same values
  // (a thread reads back its own store: no second barrier; the next writer of
  // wmin / umin is always behind another barrier)
  uint32_t a = sm.wmin[0], b = sm.wmax[0];
#pragma unroll
  for (int i = 1; i < TopkShared<NT>::NW; ++i) {
    a = sm.wmin[i] < a ? sm.wmin[i] : a;
    b = sm.wmax[i] > b ? sm.wmax[i] : b;
  }
  sm.umin = a;
  sm.umax = b;
}

// Locate the bin holding the rem-th largest item of hist[0, nb) (nb a power of
// two <= 4096, 1 <= rem <= total): sm.digit receives the bin and sm.rem the rank
// inside it. Each thread reads its (at most 16) bins with vector loads, one
// block scan orders the thread sums, and the owning thread finishes from
// registers.
// This thread's bins of hist[0, nb) for find_bin_in (h[i], i < nb / NT).
template <int NT>
__device__ __forceinline__ void load_bins(const uint32_t* hist, int nb, uint32_t (&h)[16]) {
  const int tid = threadIdx.x;
  const int per = nb >= NT ? nb / NT : 1;
  const bool act = tid < (nb >= NT ? NT : nb);
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
}

// find_bin over bins already loaded by load_bins.
template <int NT>
__device__ __forceinline__ void find_bin_in(const uint32_t (&h)[16], int nb, int rem, TopkShared<NT>& sm) {
  const int tid = threadIdx.x;
  const int per = nb >= NT ? nb / NT : 1;
  const bool act = tid < (nb >= NT ? NT : nb);
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

template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* hist, int nb, int rem, TopkShared<NT>& sm) {
  uint32_t h[16];
  load_bins<NT>(hist, nb, h);
  find_bin_in<NT>(h, nb, rem, sm);
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

// Threshold of the c keys key_at(0..c) (1 <= rem < c, extremes umin, umax):
// tau = the rem-th largest and need_eq = rem - #{keys > tau}. A short list is
// ranked pairwise. A longer one takes one pass of kSubBins bins linear in the
// score over [umin, umax]; the bin of a key never decreases as the key grows,
// so keys of higher bins all exceed, and keys of lower bins all fall below,
// every key of the bin holding the rem-th largest. That bin's keys (a few,
// unless many keys tie) are then ranked pairwise; a crowded bin falls back to
// radix digits over the whole list. Work is linear in c, not quadratic.
template <int NT, typename KeyAt>
__device__ __forceinline__ void list_threshold(KeyAt key_at, int c, int rem, uint32_t umin, uint32_t umax,
                                               TopkShared<NT>& sm, uint32_t& tau, int& need_eq) {
  constexpr int kSubBins = 1024;
  const int tid = threadIdx.x;
  if (c <= kPairCap) {
    for (int i = tid; i < c; i += NT) sm.list[i] = key_at(i);
    __syncthreads();
    rank_in_list<NT>(c, rem, sm, tau, need_eq);
    return;
  }
  const float xlo = key_score(umin);
  const float scale = lin_scale(xlo, key_score(umax), kSubBins);
  for (int b = tid; b < kSubBins; b += NT) sm.hist[b] = 0u;
  if (tid == 0) sm.nlist = 0;
  __syncthreads();
  for (int i = tid; i < c; i += NT) atomicAdd(&sm.hist[lin_bin(key_at(i), xlo, scale, kSubBins)], 1u);
  __syncthreads();
  find_bin<NT>(sm.hist, kSubBins, rem, sm);  // synchronises
  const uint32_t bstar = (uint32_t)sm.digit;
  const int nl = (int)sm.hist[bstar];
  const int r2 = sm.rem;
  if (nl > kRankCap) {
    __syncthreads();  // everyone has read the histogram before it is reused
    radix_threshold<NT>(key_at, c, rem, umin, umax, sm, tau, need_eq);
    return;
  }
  for (int i0 = 0; i0 < c; i0 += NT) {
    const int i = i0 + tid;
    const uint32_t x = i < c ? key_at(i) : 0u;
    const bool keep = i < c && lin_bin(x, xlo, scale, kSubBins) == bstar;
    const uint64_t m = wave_ballot(keep);
    int at = 0;
    if ((tid & 63) == 0 && m) at = atomicAdd(&sm.nlist, __popcll(m));
    at = __shfl(at, 0, kWave);
    if (keep) sm.list[at + lanes_below(m)] = x;
  }
  __syncthreads();
  rank_in_list<NT>(nl, r2, sm, tau, need_eq);
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


// ---------------------------------------------------------------------------
// Long rows: three passes, each spread over (chunk, row) workgroups.
//   hist  : coarse histogram of the row (bins linear in the score) into ghist
//   count : threshold bin b* (the bin holding the k-th largest) from ghist;
//           per chunk, the items above b*, and the items inside b* written in
//           position order to the chunk's own region of the boundary list
//   emit  : tau (k-th largest key) and need_eq (items equal to tau that are
//           kept, lowest positions first) from the boundary list; kept items
//           before the chunk; the chunk's kept items in position order
// Positions are indices inside the row; with row_idx the emitted index is
// row_idx[position].

struct LongRec {
  float xlo;       // smallest score of the row
  float scale;     // bin = lin_bin(key, xlo, scale, kCoarseBins)
  uint32_t bstar;  // threshold bin
  uint32_t rem;    // rank of the k-th item inside the threshold bin (1-based)
};

__device__ __forceinline__ uint32_t coarse_bin(uint32_t u, float xlo, float scale) {
  return lin_bin(u, xlo, scale, kCoarseBins);
}

// Keys of items [s0 + 4 (j0 + dj g), ... + 4) of a row for g < G (groups of
// four), with positions past s1 marked absent. Row starts are 16-byte aligned
// and every score row is stored with a stride that is a multiple of 64 items,
// so the aligned group holding item s1 - 1 lies inside the row's storage: each
// group is one 16-byte load from a clamped address, with no branch per group
// (all G loads are in flight together).
// The loads alone (load_raw4) and the conversion (keys4) are separate so that
// a caller can issue its other reads in between: a use of a load's value makes
// the compiler wait for every read issued before it.
template <int G>
__device__ __forceinline__ void load_raw4(const float* row, int s0, int s1, int j0, int dj, f32x4 (&v)[G]) {
  const int last = s1 > s0 ? (s1 - 1) & ~3 : 0;  // an empty range reads item 0 (ignored)
#pragma unroll
  for (int g = 0; g < G; ++g) v[g] = *reinterpret_cast<const f32x4*>(row + min(s0 + 4 * (j0 + dj * g), last));
}
template <int G>
__device__ __forceinline__ void keys4(const f32x4 (&v)[G], int s0, int s1, int j0, int dj, uint32_t (&u)[G][4],
                                      bool (&in)[G][4]) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int s = s0 + 4 * (j0 + dj * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      in[g][e] = s + e < s1;
      u[g][e] = in[g][e] ? score_key(v[g][e]) : 0u;
    }
  }
}
template <int G>
__device__ __forceinline__ void load_groups4(const float* row, int s0, int s1, int j0, int dj,
                                             uint32_t (&u)[G][4], bool (&in)[G][4]) {
  f32x4 v[G];
  if (s1 > s0) {
    const int last = (s1 - 1) & ~3;
#pragma unroll
    for (int g = 0; g < G; ++g)
      v[g] = *reinterpret_cast<const f32x4*>(row + min(s0 + 4 * (j0 + dj * g), last));
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  keys4<G>(v, s0, s1, j0, dj, u, in);
}

// Workgroup layout of a chunk in the count and emit passes: wave w owns the
// contiguous items [w * kChunk / NW, (w + 1) * kChunk / NW); its g-th group of
// four items at lane l starts at item 4 * (l + 64 * g) of that range.
constexpr int kLongNT = 256;
constexpr int kGroups = kChunk / 4 / kLongNT;  // groups of four items per lane

template <int NT>
__global__ __launch_bounds__(NT) void k_long_hist(TopkArgs a, const uint32_t* rmm, int nmm,
                                                  uint32_t* ghist) {
  __shared__ __attribute__((aligned(16))) uint32_t lh[kCoarseBins];
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int n = row_length(a, row);
  const int s0 = chunk * kChunk, s1 = min(n, s0 + kChunk);
  if (s0 >= s1 || a.k >= n) return;  // uniform
  // keys first, the row range (a reduction over the scoring splits) meanwhile
  const float* src = a.S + (size_t)row * a.S_ld;
  uint32_t u[kGroups][4];
  bool in[kGroups][4];
  load_groups4<kGroups>(src, s0, s1, tid, NT, u, in);
  for (int b = tid; b < kCoarseBins; b += NT) lh[b] = 0u;
  row_range<NT>(rmm, nmm, a.rows, row, sm);
  const float xlo = key_score(sm.umin), scale = lin_scale(xlo, key_score(sm.umax), kCoarseBins);
#pragma unroll
  for (int g = 0; g < kGroups; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (in[g][e]) atomicAdd(&lh[coarse_bin(u[g][e], xlo, scale)], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (size_t)row * kCoarseBins;
  for (int b = tid; b < kCoarseBins; b += NT) {
    const uint32_t c = lh[b];
    if (c) atomicAdd(&gh[b], c);
  }
}

// grid (nchunk, rows): every workgroup finds the row's threshold bin from the
// finished histogram (the same answer in each), counts its chunk's items above
// that bin, and writes the items inside it, in position order, to the chunk's
// own region of the boundary list. Chunk 0 records the rank rem of the k-th
// item in the bin.
template <int NT>
__global__ __launch_bounds__(NT) void k_long_count(TopkArgs a, const uint32_t* rmm, int nmm,
                                                   const uint32_t* ghist, LongRec* rec, int32_t* gcnt,
                                                   int32_t* bcnt, int nch, uint32_t* bkeys,
                                                   long long rld) {
  constexpr int NW = NT / kWave;
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int n = row_length(a, row);
  const int s0 = chunk * kChunk, s1 = min(n, s0 + kChunk);
  if (s0 >= s1 || a.k >= n) return;  // uniform
  const float* src = a.S + (size_t)row * a.S_ld;
  const int ws0 = s0 + w * (kChunk / NW);
  uint32_t u[kGroups][4];
  bool in[kGroups][4];
  load_groups4<kGroups>(src, ws0, s1, lane, kWave, u, in);
  uint32_t hb[16];  // the finished histogram, loaded beside the keys
  load_bins<NT>(ghist + (size_t)row * kCoarseBins, kCoarseBins, hb);
  row_range<NT>(rmm, nmm, a.rows, row, sm);
  const float xlo = key_score(sm.umin), scale = lin_scale(xlo, key_score(sm.umax), kCoarseBins);
  find_bin_in<NT>(hb, kCoarseBins, a.k, sm);
  const uint32_t bstar = (uint32_t)sm.digit;
  if (chunk == 0 && tid == 0) {
    LongRec r{};
    r.xlo = xlo;
    r.scale = scale;
    r.bstar = bstar;
    r.rem = (uint32_t)sm.rem;
    rec[row] = r;
  }
  // per lane and group: items above the bin (low half) and inside it (high half)
  int cnt[kGroups];
  int tot = 0;
  bool inb[kGroups][4];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b = coarse_bin(u[g][e], xlo, scale);
      inb[g][e] = in[g][e] && b == bstar;
      c += (in[g][e] && b > bstar) ? 1 : 0;
      c += inb[g][e] ? (1 << 16) : 0;
    }
    cnt[g] = c;
    tot += c;
  }
  tot = (int)wave_total_u32((uint32_t)tot);
  if (lane == 0) {
    sm.wgt[w] = tot & 0xffff;
    sm.weq[w] = tot >> 16;
  }
  __syncthreads();
  int above = 0, nb = 0, run = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    above += sm.wgt[i];
    nb += sm.weq[i];
    run += i < w ? sm.weq[i] : 0;
  }
  if (tid == 0) {
    gcnt[(size_t)row * nch + chunk] = above;
    bcnt[(size_t)row * nch + chunk] = nb;
  }
  if (nb == 0) return;  // uniform
  uint32_t* kd = bkeys + (size_t)row * rld + (size_t)chunk * kChunk;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int inc = wave_inclusive_scan(cnt[g] >> 16);
    int at = run + inc - (cnt[g] >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (inb[g][e]) kd[at++] = u[g][e];
    run += __builtin_amdgcn_readlane(inc, kWave - 1);
  }
}

// grid (nchunk, rows): every workgroup resolves tau (the k-th largest key) and
// need_eq (items equal to tau that are kept, lowest positions first) from the
// boundary list, counts the kept items of the chunks before its own, and
// writes its chunk's kept items in position order.
// Rescoring of a chunk's kept candidates with every head (MISA technical
// summary, "Variante Jerarquica": the routed top-k' candidates are rescored by
// all H indexer heads before the final top-k), for the rerank form of the
// emission: candidate c of the chunk (key cl[c], output position pj + c) gets
// S[row, pj + c] = sum_h w[row,h] ReLU(q[row,h] . k) * scale, the sum the
// gather form of the scoring kernel forms, in the same order and with the same
// operand layout: rows (heads) and columns (keys) of v_mfma_f32_16x16x32_bf16,
// lane l covering head / key l mod 16 with dims [32 (l / 16), 32 (l / 16) + 32).
// QF8 (fp8 queries, fp8 keys): the staged rows are E4M3 codes with the sign of
// their scale folded in and the weights are w |scale|, and one
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales) per row tile takes all
// 128 dims of the codes, as in the gather kernel's fp8 form.
// qsh / wsh: the query's 64 head rows (kRerankQStride 16-byte words apart;
// rows past H zero) and weights (zero past H), staged in LDS.
constexpr int kRerankQStride = kHeadDim / 8 + 1;  // one pad word per row: conflict-free row reads
                                                  // (a bf16 row fills 16 words, an fp8 row 8)
template <int NT, bool FP8, bool QF8>
__device__ __forceinline__ void rerank_kept(const RerankArgs& rr, int row, const int32_t* cl, int pj, int kj,
                                            const u32x4* qsh, const float* wsh) {
  static_assert(!QF8 || FP8, "fp8 queries are scored against fp8 keys");
  constexpr int NW = NT / kWave;
  constexpr int NV = FP8 ? 2 : 4;  // 16-byte words of a lane's 32 dims of a key
  constexpr int D = 2;             // key groups in flight per wave
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x >> 6;
  const int kcol = lane & 15, slice = lane >> 4;
  const int ng = (kj + 15) >> 4;  // groups of 16 candidates
  if (w >= ng) return;  // uniform: no group for this wave
  bf16x8 af[QF8 ? 1 : 4][4];
  i32x8 af8[QF8 ? 4 : 1];
  float wv[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x4* qrow = qsh + (16 * r + kcol) * kRerankQStride;
    if constexpr (QF8) {
      const u32x4 lo = qrow[2 * slice], hi = qrow[2 * slice + 1];
      af8[r] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[r][ks] = __builtin_bit_cast(bf16x8, qrow[4 * slice + ks]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[r][i] = wsh[16 * r + 4 * slice + i];
  }
  float* out = rr.S + (size_t)row * rr.S_ld + pj;
  for (int g0 = w; g0 < ng; g0 += NW * D) {
    // every group's key rows are requested before any is used (a column past
    // the list reads its last candidate and is not written)
    u32x4 kv[D][NV];
    float ksc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int key = cl[min(16 * (g0 + NW * d) + kcol, kj - 1)];
      const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(rr.K) +
                                                        (size_t)key * (FP8 ? kHeadDim : 2 * kHeadDim) +
                                                        slice * NV * 16);
#pragma unroll
      for (int v = 0; v < NV; ++v) kv[d][v] = src[v];
      ksc[d] = FP8 ? rr.kscale[key] : 1.f;
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int gi = g0 + NW * d;
      if (gi >= ng) break;  // uniform
      bf16x8 bf[4];
      if constexpr (QF8) {
        // the key's 32 codes are used as they are
      } else if constexpr (FP8) {
        // 32 E4M3 codes -> 32 bf16 (exact), in dimension order
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            u32x4 x;
            x[0] = fp8x2_to_bf16x2<false>(kv[d][v][2 * e]);
            x[1] = fp8x2_to_bf16x2<true>(kv[d][v][2 * e]);
            x[2] = fp8x2_to_bf16x2<false>(kv[d][v][2 * e + 1]);
            x[3] = fp8x2_to_bf16x2<true>(kv[d][v][2 * e + 1]);
            bf[2 * v + e] = __builtin_bit_cast(bf16x8, x);
          }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) bf[v] = __builtin_bit_cast(bf16x8, kv[d][v]);
      }
      f32x4 acc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (QF8) {
          const i32x8 b8 = i32x8{(int)kv[d][0][0], (int)kv[d][0][1], (int)kv[d][0][2], (int)kv[d][0][3],
                                 (int)kv[d][1][0], (int)kv[d][1][1], (int)kv[d][1][2], (int)kv[d][1][3]};
          a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af8[r], b8, a4, 0, 0, 0, 127, 0, 127);
        } else {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) a4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r][ks], bf[ks], a4, 0, 0, 0);
        }
        acc[r] = a4;
      }
      // ReLU, times w, the head sum, times |scale| (a negative scale flips the
      // key's sign inside the ReLU)
      const float sc = ksc[d];
      const float sgn = sc < 0.f ? -1.f : 1.f;
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wv[r][i] * relu(sgn * acc[r][i]);
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      const int c = 16 * gi + kcol;
      if (slice == 0 && c < kj) out[c] = part * fabsf(sc);
    }
  }
}

// RR: the rerank form (rr: the query rows, weights and keys; FP8: fp8 keys;
// QF8: fp8 queries), which also rescores the chunk's kept candidates into rr.S
// at their output positions; otherwise rr is unused. IDX: the row has explicit item indices
// (row_idx), read beside the scores; without them the index is the position
// (no read in the emission loop, whose stores would otherwise each wait for
// every earlier memory operation behind that conditional read).
template <int NT, bool RR, bool FP8, bool QF8, bool IDX>
__device__ __forceinline__ void long_emit(const TopkArgs& a, const LongRec* rec, const int32_t* gcnt,
                                          const int32_t* bcnt, int nch, const uint32_t* bkeys, long long rld,
                                          const RerankArgs& rr) {
  constexpr int NW = NT / kWave;
  __shared__ TopkShared<NT> sm;
  __shared__ __attribute__((aligned(16))) uint32_t blist[kBoundaryCap];
  __shared__ int boff[kMaxChunks + 1];  // region offsets of the concatenated list
  const int row = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int n = row_length(a, row);
  const bool take_all = a.k >= n;
  const int nsel = take_all ? n : a.k;
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  if (chunk == 0) {
    for (int p = nsel + tid; p < a.k; p += NT) {
      oi[p] = -1;
      if (os) os[p] = -__builtin_huge_valf();
    }
    if (a.out_count && tid == 0) a.out_count[row] = nsel;
  }
  const int s0 = chunk * kChunk, s1 = min(n, s0 + kChunk);
  if (s0 >= s1) return;  // uniform
  const float* src = a.S + (size_t)row * a.S_ld;
  const int32_t* ri = IDX ? a.row_idx + (size_t)row * a.idx_ld : nullptr;
  const int ws0 = s0 + w * (kChunk / NW);
  // every read that does not depend on another is issued here, before any is
  // used: the chunk's scores, the row record, the first NT chunks' counts and
  // the first kPre keys of every region of the boundary list (with take_all
  // the count pass did not run and these are ignored)
  f32x4 sv[kGroups];
  load_raw4<kGroups>(src, ws0, s1, lane, kWave, sv);
  i32x4 ix[IDX ? kGroups : 1];  // explicit indices, same clamped 16-byte groups as the scores
  if constexpr (IDX) {
    const int last = s1 > ws0 ? (s1 - 1) & ~3 : 0;
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
      ix[g] = *reinterpret_cast<const i32x4*>(ri + min(ws0 + 4 * (lane + kWave * g), last));
  }
  auto idx_of = [&](int g, int e, int s) {
    if constexpr (IDX) return ix[g][e];
    else return s;
  };
  const int nc = (n + kChunk - 1) / kChunk;
  const int rem_raw = (int)rec[row].rem;
  const uint32_t* gk = bkeys + (size_t)row * rld;
  constexpr int kPre = 32;                        // keys prefetched per region
  constexpr int kPreRegions = 2 * NT * 4 / kPre;  // two 16-byte words per thread
  u32x4 pf[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const int wi = tid + NT * v, r = min(wi / (kPre / 4), nch - 1);
    pf[v] = *reinterpret_cast<const u32x4*>(gk + (size_t)r * kChunk + 4 * (wi % (kPre / 4)));
  }
  const int bc0 = bcnt[(size_t)row * nch + min(tid, nch - 1)];
  const int gc0 = gcnt[(size_t)row * nch + min(tid, nch - 1)];
  // rerank form: the query's head rows and weights (16 KiB of bf16 or 8 KiB of
  // fp8 codes, and 256 B), one 16-byte word per thread and round, requested
  // after the reads above so that their first use does not wait for these;
  // staged in LDS below. fp8 rows: the scale's sign goes into the codes (bit 7
  // of each), its magnitude into the weight.
  __shared__ u32x4 qsh[RR ? kMaxHeads * kRerankQStride : 1];
  __shared__ float wsh[RR ? kMaxHeads : 1];
  constexpr int kRowWords = QF8 ? kHeadDim / 16 : kHeadDim / 8;  // 16-byte words per q row
  constexpr int kQRounds = kMaxHeads * kRowWords / NT;             // words per thread
  u32x4 qst[RR ? kQRounds : 1];
  float qss[QF8 ? kQRounds : 1];  // fp8 rows: the scale of each word's row
  float wst = 0.f, wsc = 1.f;
  if constexpr (RR) {
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(rr.q);
#pragma unroll
    for (int u = 0; u < kQRounds; ++u) {
      const int i = tid + NT * u, h = min(i / kRowWords, rr.H - 1);
      qst[u] = reinterpret_cast<const u32x4*>(qb + ((size_t)row * rr.H + h) * kRowWords * 16)[i % kRowWords];
      if constexpr (QF8) qss[u] = rr.qscale[(size_t)row * rr.H + h];
    }
    const int hw = min(tid & (kMaxHeads - 1), rr.H - 1);
    wst = rr.w[(size_t)row * rr.H + hw];
    if constexpr (QF8) wsc = rr.qscale[(size_t)row * rr.H + hw];
  }
  auto stage_q = [&]() {  // rows past H and their weights are zero
    if constexpr (RR) {
#pragma unroll
      for (int u = 0; u < kQRounds; ++u) {
        const int i = tid + NT * u, h = i / kRowWords;
        u32x4 x = h < rr.H ? qst[u] : u32x4{0u, 0u, 0u, 0u};
        if constexpr (QF8) {
          const uint32_t f = (h < rr.H && qss[u] < 0.f) ? 0x80808080u : 0u;  // the row's scale sign
          x[0] ^= f;
          x[1] ^= f;
          x[2] ^= f;
          x[3] ^= f;
        }
        qsh[h * kRerankQStride + i % kRowWords] = x;
      }
      if (tid < kMaxHeads) wsh[tid] = tid < rr.H ? (QF8 ? wst * fabsf(wsc) : wst) : 0.f;
    }
  };
  // kept candidates of the chunk, in output order (rerank form: the boundary
  // list's buffer, free once the threshold is known)
  int32_t* cl = reinterpret_cast<int32_t*>(blist);
  if (take_all) {  // every item, scores as stored (-0 folded to +0)
#pragma unroll
    for (int g = 0; g < kGroups; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = ws0 + 4 * (lane + kWave * g) + e;
        if (s < s1) {
          oi[s] = idx_of(g, e, s);
          if (os) os[s] = sv[g][e] == 0.f ? 0.f : sv[g][e];
          if (RR) cl[s - s0] = idx_of(g, e, s);
        }
      }
    if constexpr (RR) {
      stage_q();
      __syncthreads();
      rerank_kept<NT, FP8, QF8>(rr, row, cl, s0, s1 - s0, qsh, wsh);
    }
    return;
  }
  uint32_t u[kGroups][4];
  bool in[kGroups][4];
  keys4<kGroups>(sv, ws0, s1, lane, kWave, u, in);
  stage_q();  // read after the barriers below
  // ---- the region offsets of the concatenated boundary list
  const int rem = rem_raw;
  int gt_before = 0;
  bool spill = false;  // a region holds more keys than were prefetched
  for (int c0 = 0; c0 < nc; c0 += NT) {
    const int c = c0 + tid;
    const int cc = min(c, nch - 1);
    const int bc_raw = c0 == 0 ? bc0 : bcnt[(size_t)row * nch + cc];
    const int gc_raw = c0 == 0 ? gc0 : gcnt[(size_t)row * nch + cc];
    const int bc = c < nc ? bc_raw : 0;
    if (c < chunk) gt_before += gc_raw;
    spill |= bc > (c < kPreRegions ? kPre : 0);
    int tot_c;
    const int inc = block_scan<NT>(bc, sm, &tot_c);
    if (c < nc) boff[c + 1] = (c0 > 0 ? boff[c0] : 0) + inc;
    if (c0 == 0 && tid == 0) boff[0] = 0;
    __syncthreads();
  }
  spill = __syncthreads_or(spill);
  const int cb = boff[nc];
  // list item i lives in region c = the last with boff[c] <= i
  auto item = [=](int i) -> uint32_t {
    int lo = 0, hi = nc - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (boff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return gk[(size_t)lo * kChunk + (i - boff[lo])];
  };
  const bool in_lds = cb <= kBoundaryCap;
  uint32_t lo = 0xffffffffu, hi = 0u;
  if (in_lds) {
    // prefetched keys to their places; keys past a region's first kPre (or
    // in regions past the prefetched ones) are read now
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int wi = tid + NT * v, r = wi / (kPre / 4), o = 4 * (wi % (kPre / 4));
      if (r < nc) {
        const int b0 = boff[r], bc = boff[r + 1] - b0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (o + e < bc) {
            const uint32_t x = pf[v][e];
            blist[b0 + o + e] = x;
            lo = min(lo, x);
            hi = max(hi, x);
          }
      }
    }
    if (spill) {
      for (int i = tid; i < cb; i += NT) {
        int r = 0, top = nc - 1;
        while (r < top) {
          const int mid = (r + top + 1) >> 1;
          if (boff[mid] <= i) r = mid; else top = mid - 1;
        }
        const int k = i - boff[r];
        if (k >= kPre || r >= kPreRegions) {
          const uint32_t x = gk[(size_t)r * kChunk + k];
          blist[i] = x;
          lo = min(lo, x);
          hi = max(hi, x);
        }
      }
    }
  } else {
    for (int i = tid; i < cb; i += NT) {
      const uint32_t x = item(i);
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  block_minmax<NT>(lo, hi, sm);  // synchronises
  uint32_t tau;
  int need_eq;
  if (rem >= cb) {
    tau = sm.umin;  // every item of the boundary bin is kept
    need_eq = cb;
  } else if (in_lds) {
    auto key_at = [=](int i) { return blist[i]; };
    list_threshold<NT>(key_at, cb, rem, sm.umin, sm.umax, sm, tau, need_eq);
  } else {
    radix_threshold<NT>(item, cb, rem, sm.umin, sm.umax, sm, tau, need_eq);
  }
  // ---- kept items before this chunk: above-bin counts of earlier chunks,
  // plus the boundary items of earlier regions that are > tau or == tau
  int eq_before = 0;
  const int before = boff[chunk];
  for (int i = tid; i < before; i += NT) {
    const uint32_t x = in_lds ? blist[i] : item(i);
    gt_before += x > tau ? 1 : 0;
    eq_before += x == tau ? 1 : 0;
  }
  gt_before = (int)wave_total_u32((uint32_t)gt_before);
  eq_before = (int)wave_total_u32((uint32_t)eq_before);
  if (lane == 0) {
    sm.wgt[w] = gt_before;
    sm.weq[w] = eq_before;
  }
  __syncthreads();
  int gt_all = 0, eq_all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    gt_all += sm.wgt[i];
    eq_all += sm.weq[i];
  }
  __syncthreads();  // sm.wgt is reused below
  // ---- this chunk, in position order
  int cnt[kGroups];
  int tot = 0;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c += (in[g][e] && u[g][e] > tau) ? 1 : 0;
      c += (in[g][e] && u[g][e] == tau) ? (1 << 16) : 0;
    }
    cnt[g] = c;
    tot += c;
  }
  tot = (int)wave_total_u32((uint32_t)tot);
  if (lane == 0) {
    sm.wgt[w] = tot & 0xffff;
    sm.weq[w] = tot >> 16;
  }
  __syncthreads();
  int gt_run = gt_all, eq_run = eq_all;
  for (int i = 0; i < w; ++i) {
    gt_run += sm.wgt[i];
    eq_run += sm.weq[i];
  }
  // the chunk's kept items take output positions [pj, pend)
  const int pj = min(gt_all + min(eq_all, need_eq), a.k);
  int pend = 0;
  if constexpr (RR) {
    int gt_end = gt_all, eq_end = eq_all;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      gt_end += sm.wgt[i];
      eq_end += sm.weq[i];
    }
    pend = min(gt_end + min(eq_end, need_eq), a.k);
  }
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    const int inc = wave_inclusive_scan(cnt[g]);
    const int exc = inc - cnt[g];
    int gt_b = gt_run + (exc & 0xffff), eq_b = eq_run + (exc >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!in[g][e]) continue;
      const int s = ws0 + 4 * (lane + kWave * g) + e;
      int p = -1;
      if (u[g][e] > tau) {
        p = gt_b + min(eq_b, need_eq);
        ++gt_b;
      } else if (u[g][e] == tau) {
        if (eq_b < need_eq) p = gt_b + eq_b;
        ++eq_b;
      }
      if (p >= 0 && p < a.k) {
        oi[p] = idx_of(g, e, s);
        if (os) os[p] = key_score(u[g][e]);
        if (RR) cl[p - pj] = idx_of(g, e, s);
      }
    }
    const int wt = __builtin_amdgcn_readlane(inc, kWave - 1);
    gt_run += wt & 0xffff;
    eq_run += wt >> 16;
  }
  if constexpr (RR) {
    __syncthreads();  // the kept list is complete
    rerank_kept<NT, FP8, QF8>(rr, row, cl, pj, pend - pj, qsh, wsh);
  }
}

template <int NT, bool IDX>
__global__ __launch_bounds__(NT) void k_long_emit(TopkArgs a, const LongRec* rec, const int32_t* gcnt,
                                                  const int32_t* bcnt, int nch, const uint32_t* bkeys,
                                                  long long rld) {
  long_emit<NT, false, false, false, IDX>(a, rec, gcnt, bcnt, nch, bkeys, rld, RerankArgs{});
}

template <int NT, bool FP8, bool QF8>
__global__ __launch_bounds__(NT) void k_long_emit_rerank(TopkArgs a, const LongRec* rec, const int32_t* gcnt,
                                                         const int32_t* bcnt, int nch, const uint32_t* bkeys,
                                                         long long rld, RerankArgs rr) {
  long_emit<NT, true, FP8, QF8, false>(a, rec, gcnt, bcnt, nch, bkeys, rld, rr);
}

// ---------------------------------------------------------------------------
// Rows of up to NT * 4 * G items: one workgroup per row, keys in registers.
// Wave w owns items [w * 256G, (w + 1) * 256G); lane l holds, for g < G, the
// four items starting at w * 256G + 4 * (l + 64 g) (one 16-byte load each), so
// (g, lane, element) is the items' order inside the wave.
//
// Threshold: 4-bit digits of the offset key v = key - umin, most significant
// first. Each pass counts the 16 sub-ranges of the current range with packed
// per-thread counters (no atomics), reduces them over the workgroup, and keeps
// the sub-range that holds the rem-th largest item.


template <int NT, int G, typename In>
__device__ __forceinline__ void reg_threshold(const uint32_t (&u)[G][4], In in, int k,
                                              uint32_t umin, uint32_t umax, RegShared<NT>& sm,
                                              uint32_t& tau, int& need_eq) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint32_t span = umax - umin;
  int bits = span ? 32 - __clz(span) : 0;
  uint32_t base = 0u;  // offset of the current range [base, base + 2^bits)
  int rem = k;
  while (bits > 0) {
    const int wd = bits < 4 ? bits : 4;
    const int sh = bits - wd;
    uint32_t c[8];  // c[j]: count of sub-range 2j (low half), 2j + 1 (high half)
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = 0u;
#pragma unroll
    for (int g0 = 0; g0 < G; g0 += 2) {
      uint64_t x = 0;  // 4-bit counters: at most 8 items per round
#pragma unroll
      for (int g = g0; g < g0 + 2 && g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = u[g][e] - umin - base;
          const bool inr = in(g, e) && (bits >= 32 || (v >> bits) == 0u);
          x += inr ? (1ull << (4 * (v >> sh))) : 0ull;
        }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] += (uint32_t)((x >> (8 * j)) & 0xfu) | ((uint32_t)((x >> (8 * j + 4)) & 0xfu) << 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = wave_total_u32(c[j]);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.red[w][j] = c[j];
    }
    __syncthreads();
    if (w == 0) {
      // lanes 0..7 add one packed column over the waves; lane 0 walks the
      // sub-ranges from the top
      uint32_t col = 0u;
      if (lane < 8)
#pragma unroll
        for (int i = 0; i < NW; ++i) col += sm.red[i][lane];
      int above = 0, pick = 0, r = rem;
#pragma unroll
      for (int b = 15; b >= 0; --b) {
        const uint32_t packed = (uint32_t)__builtin_amdgcn_readlane((int)col, b >> 1);
        const int cnt = (int)((packed >> (16 * (b & 1))) & 0xffffu);
        if (b < (1 << wd) && pick == 0 && above < r && r <= above + cnt) {
          pick = b + 1;  // chosen sub-range, plus one
          r -= above;
        }
        above += b < (1 << wd) ? cnt : 0;
      }
      if (lane == 0) {
        sm.base = base + ((uint32_t)(pick > 0 ? pick - 1 : 0) << sh);
        sm.rem = r;
      }
    }
    __syncthreads();
    base = sm.base;
    rem = sm.rem;
    bits = sh;
  }
  tau = base + umin;
  need_eq = rem;
}

// Emit the selection in item order: items with key > tau, plus the first
// need_eq items equal to tau (all items when take_all). Writes positions below
// k only. Only the wave's first gl groups hold items (gl uniform over the wave).
template <int NT, int G, bool WITH_SCORE, typename In, typename IdxOf>
__device__ __forceinline__ void reg_emit(const uint32_t (&u)[G][4], In in, int seg0, int gl,
                                         bool take_all, uint32_t tau, int need_eq, int k,
                                         RegShared<NT>& sm, IdxOf idx_of, int32_t* out_idx,
                                         float* out_score) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  int cnt[G];
  int tot = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int c = 0;
    cnt[g] = 0;
    if (g >= gl) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool gt = in(g, e) && (take_all || u[g][e] > tau);
      const bool eq = in(g, e) && !take_all && u[g][e] == tau;
      c += (gt ? 1 : 0) + (eq ? (1 << 16) : 0);
    }
    cnt[g] = c;
    tot += c;
  }
  tot = (int)wave_total_u32((uint32_t)tot);
  if (lane == 0) {
    sm.wgt[w] = tot & 0xffff;
    sm.weq[w] = tot >> 16;
  }
  __syncthreads();
  if (gl == 0) return;  // uniform: no item in this wave
  int gt_run = 0, eq_run = 0;
  for (int i = 0; i < w; ++i) {
    gt_run += sm.wgt[i];
    eq_run += sm.weq[i];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g >= gl) break;  // uniform
    const int inc = wave_inclusive_scan(cnt[g]);
    const int exc = inc - cnt[g];
    int gt_b = gt_run + (exc & 0xffff), eq_b = eq_run + (exc >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!in(g, e)) continue;
      const int s = seg0 + 4 * (lane + kWave * g) + e;
      int p = -1;
      if (take_all || u[g][e] > tau) {
        p = gt_b + min(eq_b, need_eq);
        ++gt_b;
      } else if (u[g][e] == tau) {
        if (eq_b < need_eq) p = gt_b + eq_b;
        ++eq_b;
      }
      if (p >= 0 && p < k) {
        out_idx[p] = idx_of(g, e, s);
        if (WITH_SCORE) out_score[p] = key_score(u[g][e]);
      }
    }
    const int wt = __builtin_amdgcn_readlane(inc, kWave - 1);
    gt_run += wt & 0xffff;
    eq_run += wt >> 16;
  }
}

// IDX: the row has explicit key indices (row_idx); without them the emitted
// index is the position, computed where it is written rather than held in
// registers. The in-range test is likewise recomputed, and the threshold bin's
// members are kept as one bit per item between its two passes. Rows of 16,384 items are built for
// eight waves per SIMD (64 registers per lane, a few spilled), so two rows
// share a compute unit: the selection's barrier-separated phases are latency,
// and a second row fills them (16384 rows of 16384: 0.56 ms against 0.65 ms
// with one row per unit).
template <int NT, int G, bool IDX>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 1024 && G == 4 ? 8 : 1))) void k_topk_rows(TopkArgs a) {
  __shared__ TopkShared<NT> sm;
  __shared__ uint32_t cand[kListCap];  // keys of the threshold bin
  constexpr int NW = NT / kWave;
  const int row = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = min(row_length(a, row), NT * 4 * G);
  const int seg0 = w * 256 * G;
  const float* src = a.S + (size_t)row * a.S_ld;
  const int nrel = n - seg0;  // items of this wave's segment that exist (may be <= 0)
  // Rows of up to 16,384 items (G = 4), mostly shorter: gl counts the wave's
  // groups that hold items (uniform), and every per-item loop stops at the
  // first group past the row's end, so waves and groups beyond a short row
  // issue no per-item work (C3's causal rows: 0.46 ms against 0.58 ms). The
  // smaller forms, whose rows are mostly full, keep every group (gl = G).
  constexpr bool kSkip = G >= 4;
  const int gl = kSkip ? __builtin_amdgcn_readfirstlane(nrel <= 0 ? 0 : min(G, (nrel + 4 * kWave - 1) / (4 * kWave)))
                       : G;
  uint32_t u[G][4];
  if constexpr (kSkip) {
    f32x4 v[G];
    if (nrel > 0) {
      const int last = (n - 1) & ~3;
#pragma unroll
      for (int g = 0; g < G; ++g)
        v[g] = *reinterpret_cast<const f32x4*>(src + min(seg0 + 4 * (lane + kWave * g), last));
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) u[g][e] = 0u;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g >= gl) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[g][e] = 4 * (lane + kWave * g) + e < nrel ? score_key(v[g][e]) : 0u;
    }
  } else {
    bool unused[G][4];
    load_groups4<G>(src, seg0, n, lane, kWave, u, unused);
  }
  auto in = [=](int g, int e) { return 4 * (lane + kWave * g) + e < nrel; };
  i32x4 ix[IDX ? G : 1];
  if constexpr (IDX) {
    const int32_t* ri = a.row_idx + (size_t)row * a.idx_ld;
    if (n > seg0) {
      // index rows share the score rows' padded stride: same clamped 16-byte loads
      const int last = (n - 1) & ~3;
#pragma unroll
      for (int g = 0; g < G; ++g)
        ix[g] = *reinterpret_cast<const i32x4*>(ri + min(seg0 + 4 * (lane + kWave * g), last));
    }
  }
  int32_t* oi = a.out_idx + (size_t)row * a.out_ld;
  float* os = a.out_score ? a.out_score + (size_t)row * a.out_ld : nullptr;
  const int k = a.k;
  const bool take_all = k >= n;
  uint32_t tau = 0u;
  int need_eq = 0;
  if (!take_all) {
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g >= gl) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (in(g, e)) {
          lo = min(lo, u[g][e]);
          hi = max(hi, u[g][e]);
        }
    }
    for (int b = tid; b < kFineBins; b += NT) sm.hist[b] = 0u;
    if (tid == 0) {
      sm.ncand = 0;
      sm.cmin = 0xffffffffu;
      sm.cmax = 0u;
    }
    block_minmax<NT>(lo, hi, sm);  // synchronises
    const float xlo = key_score(sm.umin);
    const float scale = lin_scale(xlo, key_score(sm.umax), kFineBins);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g >= gl) break;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (in(g, e)) atomicAdd(&sm.hist[lin_bin(u[g][e], xlo, scale, kFineBins)], 1u);
    }
    __syncthreads();
    find_bin<NT>(sm.hist, kFineBins, k, sm);
    const uint32_t bstar = (uint32_t)sm.digit;
    const int rem = sm.rem;
    const int c = (int)sm.hist[bstar];
    if (c <= kListCap) {
      // the threshold bin's keys, in whatever order the atomics give (only their
      // values decide the threshold): into sm.list when few enough to rank
      // pairwise, else into cand for radix digits
      uint32_t* dst = c <= kRankCap ? sm.list : cand;
      const bool need_ext = rem >= c || c > kRankCap;  // extremes used below (uniform)
      uint32_t kbits = 0u, clo = 0xffffffffu, chi = 0u;
      int wcnt = 0;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g >= gl) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool kp = in(g, e) && lin_bin(u[g][e], xlo, scale, kFineBins) == bstar;
          kbits |= (uint32_t)kp << (4 * g + e);
          wcnt += __popcll(wave_ballot(kp));
          if (kp) {
            clo = min(clo, u[g][e]);
            chi = max(chi, u[g][e]);
          }
        }
      }
      if (wcnt) {  // uniform: one slot range per wave, taken with one atomic
        int at = 0;
        if (lane == 0) at = atomicAdd(&sm.ncand, wcnt);
        at = __shfl(at, 0, kWave);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (g >= gl) break;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool kp = (kbits >> (4 * g + e)) & 1u;
            const uint64_t m = wave_ballot(kp);
            if (kp) dst[at + lanes_below(m)] = u[g][e];
            at += __popcll(m);
          }
        }
        if (need_ext) {
          clo = wave_min_u32(clo);
          chi = wave_max_u32(chi);
          if (lane == 0) {
            atomicMin(&sm.cmin, clo);
            atomicMax(&sm.cmax, chi);
          }
        }
      }
      __syncthreads();  // the list and its extremes are complete
      if (rem >= c) {
        tau = sm.cmin;  // the whole bin is kept
        need_eq = c;
      } else if (c <= kRankCap) {
        rank_in_list<NT>(c, rem, sm, tau, need_eq);
      } else {
        auto key_at = [=](int i) { return cand[i]; };
        radix_threshold<NT>(key_at, c, rem, sm.cmin, sm.cmax, sm, tau, need_eq);
      }
    } else {
      // a crowded bin (heavy ties): digit-by-digit search over every item
      reg_threshold<NT, G>(u, in, k, sm.umin, sm.umax, sm.reg, tau, need_eq);
    }
  }
  auto idx_of = [&](int g, int e, int s) {
    if constexpr (IDX) return ix[g][e];
    else return s;
  };
  if (os) reg_emit<NT, G, true>(u, in, seg0, gl, take_all, tau, need_eq, k, sm.reg, idx_of, oi, os);
  else reg_emit<NT, G, false>(u, in, seg0, gl, take_all, tau, need_eq, k, sm.reg, idx_of, oi, os);
  const int nsel = take_all ? n : k;
  for (int p = nsel + tid; p < k; p += NT) {
    oi[p] = -1;
    if (os) os[p] = -__builtin_huge_valf();
  }
  if (a.out_count && tid == 0) a.out_count[row] = nsel;
}

// grid (nchunk, rows): {min, max} score key of each chunk into rmm[chunk, row];
// the workgroups also clear `zero`, each a share.
template <int NT>
__global__ __launch_bounds__(NT) void k_topk_range(TopkArgs a, uint32_t* rmm, uint32_t* zero,
                                                   long long zero_n) {
  __shared__ TopkShared<NT> sm;
  const int row = blockIdx.y, chunk = blockIdx.x;
  if (zero) {
    const long long nthreads = (long long)NT * gridDim.x * gridDim.y;
    for (long long i = ((long long)blockIdx.y * gridDim.x + blockIdx.x) * NT + threadIdx.x; i < zero_n;
         i += nthreads)
      zero[i] = 0u;
  }
  const int n = row_length(a, row);
  const int s0 = chunk * kChunk, s1 = min(n, s0 + kChunk);
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

// ---------------------------------------------------------------------------
// Host launchers.

int topk_lds_cap() { return kLdsCap; }
int topk_long_chunk() { return kChunk; }
int topk_coarse_bins() { return kCoarseBins; }
int topk_long_chunks(int max_n) { return max_n <= 0 ? 1 : (max_n + kChunk - 1) / kChunk; }
int topk_long_max_chunks() { return kMaxChunks; }
size_t topk_long_rec_bytes() { return sizeof(LongRec); }

hipError_t launch_topk_rows(const LaunchCtx& cx, const TopkArgs& a, int max_n) {
  if (a.rows == 0) return hipSuccess;
  if (max_n > kLdsCap) return hipErrorInvalidValue;
  const dim3 grid(a.rows);
#define MISA_ROWS(NT, G)                                                                           \
  (a.row_idx ? cx.launch("topk_rows", k_topk_rows<NT, G, true>, grid, dim3(NT), 0, a)             \
             : cx.launch("topk_rows", k_topk_rows<NT, G, false>, grid, dim3(NT), 0, a))
  if (max_n <= 1024) return MISA_ROWS(256, 1);
  if (max_n <= 4096) return MISA_ROWS(1024, 1);
  if (max_n <= 8192) return MISA_ROWS(1024, 2);
  return MISA_ROWS(1024, 4);
#undef MISA_ROWS
}

hipError_t launch_topk_long(const LaunchCtx& cx, const TopkArgs& a, const TopkLongWs& ws, int max_n,
                            const RerankArgs* rr) {
  if (a.rows == 0) return hipSuccess;
  const int nch = topk_long_chunks(max_n);
  if (nch > kMaxChunks) return hipErrorInvalidValue;
  const long long rld = (long long)nch * kChunk;
  LongRec* rec = reinterpret_cast<LongRec*>(ws.rec);
  const dim3 grid(nch, a.rows);
  hipError_t e = cx.launch("topk_hist", k_long_hist<kLongNT>, grid, dim3(kLongNT), 0, a, ws.rmm,
                           ws.nmm, ws.ghist);
  if (e != hipSuccess) return e;
  e = cx.launch("topk_count", k_long_count<kLongNT>, grid, dim3(kLongNT), 0, a, ws.rmm, ws.nmm,
                (const uint32_t*)ws.ghist, rec, ws.gcnt, ws.bcnt, nch, ws.bkeys, rld);
  if (e != hipSuccess) return e;
  if (rr) {
    if (a.row_idx || rr->H < 1 || rr->H > kMaxHeads || rr->S_ld % 4 != 0) return hipErrorInvalidValue;
    if (rr->q_fp8 && (!rr->fp8 || !rr->qscale)) return hipErrorInvalidValue;  // fp8 x fp8, scales needed
#define MISA_RERANK_LAUNCH(F8, QF)                                                                          \
  cx.launch("topk_emit_rerank", k_long_emit_rerank<kLongNT, F8, QF>, grid, dim3(kLongNT), 0, a,              \
            (const LongRec*)rec, (const int32_t*)ws.gcnt, (const int32_t*)ws.bcnt, nch, (const uint32_t*)ws.bkeys, \
            rld, *rr)
    if (rr->q_fp8) return MISA_RERANK_LAUNCH(true, true);
    return rr->fp8 ? MISA_RERANK_LAUNCH(true, false) : MISA_RERANK_LAUNCH(false, false);
#undef MISA_RERANK_LAUNCH
  }
  if (a.row_idx)
    return cx.launch("topk_emit", k_long_emit<kLongNT, true>, grid, dim3(kLongNT), 0, a, (const LongRec*)rec,
                     (const int32_t*)ws.gcnt, (const int32_t*)ws.bcnt, nch, (const uint32_t*)ws.bkeys, rld);
  return cx.launch("topk_emit", k_long_emit<kLongNT, false>, grid, dim3(kLongNT), 0, a, (const LongRec*)rec,
                   (const int32_t*)ws.gcnt, (const int32_t*)ws.bcnt, nch, (const uint32_t*)ws.bkeys, rld);
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


}  // namespace misa
