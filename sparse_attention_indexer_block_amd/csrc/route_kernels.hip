// Router side of the indexer: block statistics of the keys and the per-head
// routing score (MISA technical summary, "Metodologia: MISA": the router pools
// the prefix into M = ceil(L/B) blocks of averaged keys, scores every head
// against them and keeps the best h heads; HISA write-up, section 3 Stage 1
// uses the same block representatives for its block filter).
//
// Precision: block sums are accumulated in float64 (bf16 keys, and fp8 codes
// times fp32 scales, add up exactly at these sizes) and the head scores are
// float64 dot products, so the routed head set agrees with an exact
// evaluation except where two heads tie to float64 rounding.
#include "device_common.h"
#include "launch.h"

namespace misa {

// -------------------------------------------------------------------------
// One 16-byte slice of key s, dims [DPT*dg, DPT*dg + DPT) (DPT = 8 bf16 or 16
// fp8 codes), widened to float64; fp8 codes are multiplied by the key's scale,
// which is exact in float64.
template <bool FP8>
struct KeySlice {
  static constexpr int DPT = FP8 ? 16 : 8;
  static __device__ __forceinline__ u32x4 load(const void* K, int s, int dg) {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(K) + (size_t)s * kHeadDim * (FP8 ? 1 : 2);
    return *reinterpret_cast<const u32x4*>(base + 16 * dg);
  }
  static __device__ __forceinline__ void widen(u32x4 v, double sc, double* out) {
    if constexpr (!FP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[2 * j] = (double)bf16_bits_to_f32(v[j] & 0xffffu);
        out[2 * j + 1] = (double)bf16_bits_to_f32(v[j] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float a, b, c, d;
        fp8x2_to_f32<false>(v[j], a, b);
        fp8x2_to_f32<true>(v[j], c, d);
        out[4 * j + 0] = (double)a * sc;
        out[4 * j + 1] = (double)b * sc;
        out[4 * j + 2] = (double)c * sc;
        out[4 * j + 3] = (double)d * sc;
      }
    }
  }
};

// Sum of key rows [s0, s1) in float64, one workgroup of 256 threads; thread
// (rl, dg) takes rows rl, rl + RL, ... and one 16-byte slice of dims. Four rows
// per thread are loaded before any is added, so the loads overlap. Column sums
// are left in red[r][d] (r < RL) for the caller to add up.
// MAX: per-dimension maximum instead of the sum (max-pooled representatives;
// exact, the widened values being exact in float64).
template <bool FP8, bool MAX = false>
struct RowSum {
  static constexpr int DPT = KeySlice<FP8>::DPT;
  static constexpr int NG = kHeadDim / DPT;  // slices per key
  static constexpr int RL = 256 / NG;        // rows in flight per pass
  static __device__ __forceinline__ void run(const void* K, const float* kscale, int s0, int s1,
                                             double (*red)[kHeadDim]) {
    const int tid = threadIdx.x, dg = tid % NG, rl = tid / NG;
    double acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = MAX ? -__builtin_huge_val() : 0.0;
    constexpr int U = 4;
    for (int sb = s0 + rl; sb < s1; sb += RL * U) {
      u32x4 v[U];
      double sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int s = sb + RL * u;
        v[u] = u32x4{0u, 0u, 0u, 0u};
        sc[u] = 0.0;
        if (s < s1) {
          v[u] = KeySlice<FP8>::load(K, s, dg);
          if constexpr (FP8) sc[u] = (double)kscale[s];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        double x[DPT];
        KeySlice<FP8>::widen(v[u], sc[u], x);
        if constexpr (MAX) {
          if (sb + RL * u < s1) {
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] = x[e] > acc[e] ? x[e] : acc[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] += x[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < DPT; ++e) red[rl][dg * DPT + e] = acc[e];
    __syncthreads();
  }
};

// Workgroup b (= blockIdx.x + b_base) in [0, M): ksum[b,:] = sum of the keys of
// block b = [b*B, min((b+1)*B, L)) in float64, and (optional) kbar = ksum /
// count rounded once to float32. Workgroups [M, M+T): tsum[t,:] = sum of the
// keys of query t's last block [(M_t-1)*B, n_t), possibly partial; zero when
// the query sees no key. b_base = M computes the query tails only. MAX: the
// per-dimension maxima of the same keys instead of their sums (max-pooled
// block representatives; no kbar or kb16), zero for a query with no key.
template <bool FP8, bool MAX>
__global__ __launch_bounds__(256) void k_block_sums(const void* K, const float* kscale, int L,
                                                    int B, int M, double* ksum, float* kbar,
                                                    uint16_t* kb16, const int32_t* pos, double* tsum,
                                                    int b_base) {
  constexpr int RL = RowSum<FP8, MAX>::RL;
  __shared__ double red[RL][kHeadDim];
  const int b = (int)blockIdx.x + b_base;
  int s0, s1;
  if (b < M) {
    s0 = (int)((long long)b * B);
    s1 = (int)((long long)s0 + B < L ? (long long)s0 + B : L);
  } else {
    const int n = visible_len(pos[b - M], L);
    const int Mt = (int)(((long long)n + B - 1) / B);
    s0 = Mt > 0 ? (int)((long long)(Mt - 1) * B) : 0;
    s1 = n;
  }
  RowSum<FP8, MAX>::run(K, kscale, s0, s1, red);
  const int tid = threadIdx.x;
  if (tid < kHeadDim) {
    double s = MAX ? -__builtin_huge_val() : 0.0;
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      if constexpr (MAX) s = red[r][tid] > s ? red[r][tid] : s;
      else s += red[r][tid];
    }
    if (MAX && s1 <= s0) s = 0.0;  // no key
    if (b < M) {
      ksum[(size_t)b * kHeadDim + tid] = s;
      if constexpr (MAX) return;
      const double mean = s / (double)(s1 - s0);
      if (kbar) kbar[(size_t)b * kHeadDim + tid] = (float)mean;
      if (kb16) {
        // bf16 hi / lo split of the mean for the router's fast pass
        uint32_t hi, lo;
        split_bf16(mean, hi, lo);
        kb16[(size_t)b * 2 * kHeadDim + tid] = (uint16_t)hi;
        kb16[(size_t)b * 2 * kHeadDim + kHeadDim + tid] = (uint16_t)lo;
      }
    } else {
      tsum[(size_t)(b - M) * kHeadDim + tid] = s;
    }
  }
}

// -------------------------------------------------------------------------
// Router scores rho(t,h,b) = q[t,h] . Kbar_b as float64 matrix products.
// grid (ntiles, ceil(T / QG)), 256 threads: tile c holds blocks
// [16c, 16c + 16), staged once in LDS and kept in registers for QG queries; wave w takes heads [16w, 16w + 16). One v_mfma_f64_16x16x4 step
// takes four head dims; lane l feeds head (A) and block (B) l % 16 with dims
// [32(l/16), 32(l/16) + 32), one per step, so its operands are contiguous.
// The result D[row][col] sits at lane col + 16 * (row % 4), element row / 4.
// Writes, per (t, tile, h), max over the tile's full blocks of ReLU(rho)
// (zero for tiles past the query's blocks); the tile holding query t's last
// (possibly partial) block also writes that block's rho to ptail[t, h]. With
// WITH_BETA it writes the HISA block score beta(t,b) = sum_h w[t,h] ReLU(rho)
// of every visible block.
constexpr int kRouteTile = 16;  // blocks per workgroup

// max over the 16 lanes of each row of the wave (every lane gets its row's max)
template <int CTRL>
__device__ __forceinline__ double dpp_max(double v) {
  const int2 b = __builtin_bit_cast(int2, v);
  int2 o;
  o.x = __builtin_amdgcn_update_dpp(0, b.x, CTRL, 0xf, 0xf, false);
  o.y = __builtin_amdgcn_update_dpp(0, b.y, CTRL, 0xf, 0xf, false);
  const double ov = __builtin_bit_cast(double, o);
  return ov > v ? ov : v;
}
__device__ __forceinline__ double row_max16(double v) {
  v = dpp_max<0x121>(v);  // row_ror:1
  v = dpp_max<0x122>(v);  // row_ror:2
  v = dpp_max<0x124>(v);  // row_ror:4
  return dpp_max<0x128>(v);  // row_ror:8
}

template <bool WITH_BETA, int kRouteQG>
__global__ __launch_bounds__(256) void k_route_mfma(const uint16_t* q, const float* w,
                                                    const int32_t* pos, int T, int H, int L, int B,
                                                    int ntiles, const double* ksum,
                                                    const float* kbar, const double* tsum,
                                                    double* pmax, double* ptail, float* beta,
                                                    int beta_ld, int max_pool) {
  __shared__ f64x2 kt[kRouteTile][kHeadDim / 2 + 1];  // padded rows
  __shared__ double bsum[4][kRouteTile];
  const int tile = blockIdx.x, tq0 = blockIdx.y * kRouteQG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int M = (int)(((long long)L + B - 1) / B);
  const int b0 = tile * kRouteTile;
  const int blk = b0 + col;
  const int h_a = kRouteTile * wv + col;  // head fed by this lane's A operand
  // per query of the group: visible blocks, and the A operand (32 bf16 dims)
  // in a two-slot ring so the next query's rows load during this one's products
  int n_q[kRouteQG];
#pragma unroll
  for (int i = 0; i < kRouteQG; ++i) {
    const int t = tq0 + i;
    n_q[i] = t < T ? visible_len(pos[t], L) : 0;
  }
  u32x4 qv[2][4];
#define MISA_LOAD_Q(i, slot)                                                                     \
  do {                                                                                           \
    const int t_ = tq0 + (i);                                                                    \
    const bool ok_ = t_ < T && h_a < H;                                                          \
    const u32x4* src_ = reinterpret_cast<const u32x4*>(                                          \
        q + ((size_t)(ok_ ? t_ : 0) * H + (ok_ ? h_a : 0)) * kHeadDim + 32 * g);                 \
    _Pragma("unroll") for (int v_ = 0; v_ < 4; ++v_) qv[slot][v_] = ok_ ? src_[v_] : u32x4{0u, 0u, 0u, 0u}; \
  } while (0)
  MISA_LOAD_Q(0, 0);
  if (kbar) {
    // stage the tile's cached block means (8 KB): two 16-byte loads per thread
    f32x4 x[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, r = i >> 5, c4 = i & 31;
      x[u] = b0 + r < M ? reinterpret_cast<const f32x4*>(kbar + (size_t)(b0 + r) * kHeadDim)[c4]
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + 256 * u, r = i >> 5, c4 = i & 31;
      kt[r][2 * c4] = f64x2{(double)x[u][0], (double)x[u][1]};
      kt[r][2 * c4 + 1] = f64x2{(double)x[u][2], (double)x[u][3]};
    }
  } else {
    // stage the tile's block sums (16 KB): four 16-byte loads per thread
    f64x2 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, r = i >> 6, c2 = i & 63;
      x[u] = b0 + r < M ? reinterpret_cast<const f64x2*>(ksum + (size_t)(b0 + r) * kHeadDim)[c2] : f64x2{0.0, 0.0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      kt[i >> 6][i & 63] = x[u];
    }
  }
  // full blocks hold sums (divide by B), cached means or maxima (divide by 1)
  const double div_full = kbar || max_pool ? 1.0 : (double)B;
  __syncthreads();
  f64x2 kv[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) kv[v] = kt[col][16 * g + v];

#pragma unroll
  for (int i = 0; i < kRouteQG; ++i) {
    const int t = tq0 + i;
    if (t >= T) break;  // uniform
    if (i + 1 < kRouteQG) MISA_LOAD_Q(i + 1, (i + 1) & 1);
    const int n = n_q[i];
    const int Mt = (int)(((long long)n + B - 1) / B);
    double* pm = pmax + ((size_t)t * ntiles + tile) * kWave;
    if (b0 >= Mt) {  // uniform: no block of this tile is visible
      if (tid < kWave) pm[tid] = 0.0;
      continue;
    }
    const bool valid = blk < Mt;
    const bool tail = blk == Mt - 1;
    // B operand: the block sums, or this query's own sum for its last block
    f64x2 kb[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) kb[v] = valid ? kv[v] : f64x2{0.0, 0.0};
    if (tail) {
      const f64x2* src = reinterpret_cast<const f64x2*>(tsum + (size_t)t * kHeadDim + 32 * g);
#pragma unroll
      for (int v = 0; v < 16; ++v) kb[v] = src[v];
    }
    // two accumulation chains (even and odd dims) keep the matrix unit busy
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
      const uint32_t word = qv[i & 1][s >> 3][(s >> 1) & 3];
      const double a0 = (double)bf16_bits_to_f32(word & 0xffffu);
      const double a1 = (double)bf16_bits_to_f32(word >> 16);
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, kb[s >> 1][0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, kb[s >> 1][1], acc1, 0, 0, 0);
    }
    const f64x4 acc = acc0 + acc1;
    // this lane holds heads 16 wv + 4 e + g (e = 0..3) against block blk
    const double cnt = tail ? (max_pool ? 1.0 : (double)(n - (Mt - 1) * B)) : div_full;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double m = row_max16((valid && !tail && acc[e] > 0.0) ? acc[e] : 0.0);
      if (col == 0) pm[kRouteTile * wv + 4 * e + g] = m / div_full;
    }
    if (tail) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ptail[(size_t)t * kWave + kRouteTile * wv + 4 * e + g] = acc[e] / cnt;
    }
    if constexpr (WITH_BETA) {
      double part = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hh = kRouteTile * wv + 4 * e + g;
        const double rho = acc[e] / cnt;
        part += (hh < H && rho > 0.0) ? (double)w[(size_t)t * H + hh] * rho : 0.0;
      }
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      if (lane < kRouteTile) bsum[wv][lane] = part;
      __syncthreads();
      if (tid < kRouteTile && b0 + tid < Mt) {
        const double s = bsum[0][tid] + bsum[1][tid] + bsum[2][tid] + bsum[3][tid];
        beta[(size_t)t * beta_ld + b0 + tid] = (float)s;
      }
      __syncthreads();
    }
  }
}

#undef MISA_LOAD_Q

// Final router step, 256 threads per query: r(t,h) = w[t,h] * max_b ReLU(rho)
// over the tile maxima and the last block, then the first A heads under
// (-r, h). heads[t,:] is written in ascending head order; with qr the routed q
// rows and weights are packed in the same order for the scoring kernel. Every
// global read is issued up front (none depends on another).
__global__ __launch_bounds__(256) void k_route_select(const uint16_t* q, const float* w,
                                                     const int32_t* pos, int H, int L, int B, int A,
                                                     int ntiles, const double* pmax,
                                                     const double* ptail, int32_t* heads,
                                                     float* r_out, uint16_t* qr, float* wr) {
  __shared__ double part[4][kWave];
  __shared__ double rs[kWave];
  __shared__ int rank_part[4][kWave];
  __shared__ u32x4 qs[kWave * kHeadDim / 8];  // q[t] as 16-byte words
  const int t = blockIdx.x, tid = threadIdx.x, h = tid & 63, j = tid >> 6;
  const int n = visible_len(pos[t], L);
  const bool active = h < H;
  const float wt = active ? w[(size_t)t * H + h] : 0.f;
  const double rho_tail = ptail[(size_t)t * kWave + h];
  if (qr) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + (size_t)t * H * kHeadDim);
    const int nw = H * kHeadDim / 8;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tid + 256 * u < nw) qs[tid + 256 * u] = src[tid + 256 * u];
  }
  const double* pm = pmax + (size_t)t * ntiles * kWave + h;
  double m = 0.0;
  constexpr int U = 16;
  for (int c0 = j; c0 < ntiles; c0 += 4 * U) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      v[u] = c < ntiles ? pm[(size_t)c * kWave] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m = v[u] > m ? v[u] : m;
  }
  part[j][h] = m;
  __syncthreads();
  const int Mt = (int)(((long long)n + B - 1) / B);
  double r = 0.0;
  if (j == 0) {
    m = part[0][h];
#pragma unroll
    for (int jj = 1; jj < 4; ++jj) m = part[jj][h] > m ? part[jj][h] : m;
    if (Mt > 0) m = rho_tail > m ? rho_tail : m;
    r = active ? (double)wt * m + 0.0 : -__builtin_huge_val();
    if (r_out && active) r_out[(size_t)t * H + h] = (float)r;
    rs[h] = r;
  }
  __syncthreads();
  if (!heads) return;
  {
    // rank of head h: wave j compares it with heads [16j, 16j + 16)
    const double rh = rs[h];
    double r2[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) r2[u] = rs[16 * j + u];
    int c = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) c += (r2[u] > rh) || (r2[u] == rh && 16 * j + u < h);
    rank_part[j][h] = c;
  }
  __syncthreads();
  if (j != 0) return;
  const int rank = rank_part[0][h] + rank_part[1][h] + rank_part[2][h] + rank_part[3][h];
  const bool sel = active && rank < A;
  const uint64_t mask = wave_ballot(sel);
  if (sel) {
    const int slot = lanes_below(mask);
    heads[(size_t)t * A + slot] = h;
    if (qr) {
      wr[(size_t)t * A + slot] = wt;
      u32x4* dst = reinterpret_cast<u32x4*>(qr + ((size_t)t * A + slot) * kHeadDim);
#pragma unroll
      for (int v = 0; v < kHeadDim / 8; ++v) dst[v] = qs[h * (kHeadDim / 8) + v];
    }
  }
}

// Pack the q rows and weights of caller-given heads in slot order; one wave
// per (query, slot), each lane copying 4 bytes.
__global__ __launch_bounds__(64) void k_gather_heads(const uint16_t* q, const float* w,
                                                     const int32_t* heads, int H, int A,
                                                     uint16_t* qr, float* wr) {
  const int t = blockIdx.y, j = blockIdx.x, lane = threadIdx.x;
  const int h = heads[(size_t)t * A + j];
  const bool ok = h >= 0 && h < H;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(q + ((size_t)t * H + (ok ? h : 0)) * kHeadDim);
  uint32_t* dst = reinterpret_cast<uint32_t*>(qr + ((size_t)t * A + j) * kHeadDim);
  dst[lane] = ok ? src[lane] : 0u;
  if (lane == 0) wr[(size_t)t * A + j] = ok ? w[(size_t)t * H + h] : 0.f;
}

// -------------------------------------------------------------------------
// Host launchers.

hipError_t launch_block_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                             int L, int B, double* ksum, float* kbar, int T, const int32_t* pos,
                             double* tsum, bool tails_only, uint16_t* kb16, int first_block, bool max_pool) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int base = tails_only ? M : (first_block < M ? first_block : M);
  const int grid = M - base + (tsum ? T : 0);
  if (grid == 0) return hipSuccess;
  const char* nm = tails_only ? "tail_sums" : "block_sums";
#define MISA_SUMS_LAUNCH(F8, MX)                                                                    \
  cx.launch(nm, k_block_sums<F8, MX>, dim3(grid), dim3(256), 0, K, kscale, L, B, M, ksum,            \
            MX ? nullptr : kbar, MX ? nullptr : kb16, pos, tsum, base)
  if (max_pool) return fp8 ? MISA_SUMS_LAUNCH(true, true) : MISA_SUMS_LAUNCH(false, true);
  return fp8 ? MISA_SUMS_LAUNCH(true, false) : MISA_SUMS_LAUNCH(false, false);
#undef MISA_SUMS_LAUNCH
}

int route_chunks(int L, int B) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int c = (M + kRouteTile - 1) / kRouteTile;
  return c < 1 ? 1 : c;
}

hipError_t launch_route(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                        int T, int H, int L, int B, int A, const double* ksum, const float* kbar,
                        const double* tsum, double* pmax, int32_t* heads, float* r_out,
                        float* beta, int beta_ld, uint16_t* qr, float* wr, bool max_pool) {
  if (T == 0) return hipSuccess;
  const int nt = route_chunks(L, B);
  double* ptail = pmax + (size_t)T * nt * kWave;
  hipError_t e;
  // one query per workgroup while that leaves few workgroups per CU; past
  // that, groups of queries share each staged tile
  const long long work = (long long)nt * T;
  const int qg = work > 16384 ? 8 : (work > 2048 ? 2 : 1);
  const dim3 grid(nt, (T + qg - 1) / qg);
#define MISA_ROUTE_LAUNCH(BETA, QG)                                                                \
  cx.launch("route_mfma", k_route_mfma<BETA, QG>, grid, dim3(256), 0, q, w, pos, T, H, L, B, nt, ksum, \
            kbar, tsum, pmax, ptail, beta, beta_ld, max_pool ? 1 : 0)
  if (beta)
    e = qg == 8 ? MISA_ROUTE_LAUNCH(true, 8) : (qg == 2 ? MISA_ROUTE_LAUNCH(true, 2) : MISA_ROUTE_LAUNCH(true, 1));
  else
    e = qg == 8 ? MISA_ROUTE_LAUNCH(false, 8) : (qg == 2 ? MISA_ROUTE_LAUNCH(false, 2) : MISA_ROUTE_LAUNCH(false, 1));
#undef MISA_ROUTE_LAUNCH
  if (e != hipSuccess) return e;
  if (!heads && !r_out) return hipSuccess;  // block scores only
  return cx.launch("route_select", k_route_select, dim3(T), dim3(256), 0, q, w, pos, H, L, B, A, nt,
                   (const double*)pmax, (const double*)ptail, heads, r_out, qr, wr);
}

hipError_t launch_gather_heads(const LaunchCtx& cx, const uint16_t* q, const float* w,
                               const int32_t* heads, int T, int H, int A, uint16_t* qr, float* wr) {
  if (T == 0) return hipSuccess;
  return cx.launch("gather_heads", k_gather_heads, dim3(A, T), dim3(64), 0, q, w, heads, H, A, qr, wr);
}

}  // namespace misa
