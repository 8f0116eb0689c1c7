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
template <bool FP8>
struct RowSum {
  static constexpr int DPT = KeySlice<FP8>::DPT;
  static constexpr int NG = kHeadDim / DPT;  // slices per key
  static constexpr int RL = 256 / NG;        // rows in flight per pass
  static __device__ __forceinline__ void run(const void* K, const float* kscale, int s0, int s1,
                                             double (*red)[kHeadDim]) {
    const int tid = threadIdx.x, dg = tid % NG, rl = tid / NG;
    double acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.0;
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
#pragma unroll
        for (int e = 0; e < DPT; ++e) acc[e] += x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < DPT; ++e) red[rl][dg * DPT + e] = acc[e];
    __syncthreads();
  }
};

// Workgroups [0, M): ksum[b,:] = sum of the keys of block b = [b*B, min((b+1)*B, L))
// in float64, and (optional) kbar = ksum / count rounded once to float32.
// Workgroups [M, M+T): tsum[t,:] = sum of the keys of query t's last block
// [(M_t-1)*B, n_t), possibly partial; zero when the query sees no key.
template <bool FP8>
__global__ __launch_bounds__(256) void k_block_sums(const void* K, const float* kscale, int L,
                                                    int B, int M, double* ksum, float* kbar,
                                                    const int32_t* pos, double* tsum) {
  constexpr int RL = RowSum<FP8>::RL;
  __shared__ double red[RL][kHeadDim];
  const int b = blockIdx.x;
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
  RowSum<FP8>::run(K, kscale, s0, s1, red);
  const int tid = threadIdx.x;
  if (tid < kHeadDim) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < RL; ++r) s += red[r][tid];
    if (b < M) {
      ksum[(size_t)b * kHeadDim + tid] = s;
      if (kbar) kbar[(size_t)b * kHeadDim + tid] = (float)(s / (double)(s1 - s0));
    } else {
      tsum[(size_t)(b - M) * kHeadDim + tid] = s;
    }
  }
}

// -------------------------------------------------------------------------
// Router over the full blocks that precede each query's last block.
// grid (nchunk, T), 256 threads: lane = head h, wave j takes a contiguous
// quarter of this chunk's blocks. Writes, per (t, chunk, h), the largest
// block sum . q[t,h] floored at zero, divided by B (= max_b ReLU(rho)).
// With WITH_BETA it also writes the HISA block score
// beta(t,b) = sum_h w[t,h] ReLU(rho(t,h,b)) of every full block.
constexpr int kRouteChunk = 32;  // blocks per workgroup

template <bool WITH_BETA>
__global__ __launch_bounds__(256) void k_route_partial(const uint16_t* q, const float* w,
                                                       const int32_t* pos, int H, int L, int B,
                                                       int nchunk, const double* ksum,
                                                       double* pmax, float* beta, int beta_ld) {
  // rows past the chunk's last block stay zero, so every wave can always
  // process four rows at a time (kRouteChunk + 4 rows)
  __shared__ double ks[kRouteChunk + 4][kHeadDim];
  __shared__ float qs[kHeadDim][kWave];  // q[t, h, i] at qs[i][h]: lanes read consecutive words
  __shared__ double wmax[4][kWave];
  const int c = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, h = tid & 63;
  const int j = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  const int F = Mt > 0 ? Mt - 1 : 0;  // full blocks before the last one
  const int b0 = c * kRouteChunk;
  const int b1 = min(b0 + kRouteChunk, F);
  double* out = pmax + ((size_t)t * nchunk + c) * kWave;
  if (b0 >= b1) {
    if (tid < kWave) out[tid] = 0.0;
    return;
  }
  const int nb = b1 - b0;
  {
    // stage this chunk's block sums (16 B per load, all loads issued first)
    constexpr int U = kRouteChunk * kHeadDim / 2 / 256;
    const f64x2* src = reinterpret_cast<const f64x2*>(ksum + (size_t)b0 * kHeadDim);
    f64x2* dst = reinterpret_cast<f64x2*>(&ks[0][0]);
    const int n2 = nb * kHeadDim / 2;
    f64x2 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      v[u] = f64x2{0.0, 0.0};
      if (tid + 256 * u < n2) v[u] = src[tid + 256 * u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) dst[tid + 256 * u] = v[u];
    if (tid < 4 * kHeadDim / 2) dst[kRouteChunk * kHeadDim / 2 + tid] = f64x2{0.0, 0.0};
  }
  {
    // stage q[t, :, :] transposed; wave j loads dims [32j, 32j+32) of every head
    const bool act = h < H;
    u32x4 x[4];
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)t * H + (act ? h : 0)) * kHeadDim + 32 * j);
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = act ? src[v] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[32 * j + 8 * v + 2 * e][h] = bf16_bits_to_f32(x[v][e] & 0xffffu);
        qs[32 * j + 8 * v + 2 * e + 1][h] = bf16_bits_to_f32(x[v][e] >> 16);
      }
  }
  const bool active = h < H;
  const double wh = active ? (double)w[(size_t)t * H + h] : 0.0;
  __syncthreads();

  const int per = (nb + 3) / 4;
  const int bl0 = j * per, bl1 = min(nb, bl0 + per);
  double m = 0.0;
  for (int bl = bl0; bl < bl1; bl += 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const int cnt = min(4, bl1 - bl);
#pragma unroll 8
    for (int i = 0; i < kHeadDim; ++i) {
      const double qd = (double)qs[i][h];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = fma(qd, ks[bl + u][i], acc[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < cnt) {
        m = acc[u] > m ? acc[u] : m;
        if constexpr (WITH_BETA) {
          const double rho = acc[u] / (double)B;
          const double contrib = active ? wh * (rho > 0.0 ? rho : 0.0) : 0.0;
          const double s = wave_sum(contrib);
          if (h == 0) beta[(size_t)t * beta_ld + b0 + bl + u] = (float)s;
        }
      }
    }
  }
  wmax[j][h] = m;
  __syncthreads();
  if (tid < kWave) {
    double mm = wmax[0][tid];
#pragma unroll
    for (int jj = 1; jj < 4; ++jj) mm = wmax[jj][tid] > mm ? wmax[jj][tid] : mm;
    out[tid] = mm / (double)B;
  }
}

// Final router step, one wave per query: fold in the query's last (possibly
// partial) block, form r(t,h) = w[t,h] * max_b ReLU(rho), and keep the first A
// heads under (-r, h). heads[t,:] is written in ascending head order.
__global__ __launch_bounds__(64) void k_route_select(const uint16_t* q, const float* w,
                                                    const int32_t* pos, int H, int L, int B, int A,
                                                    int nchunk, const double* pmax,
                                                    const double* tsum, int32_t* heads,
                                                    float* r_out, float* beta, int beta_ld,
                                                    uint16_t* qr, float* wr) {
  __shared__ double rs[kWave];
  __shared__ double ts[kHeadDim];
  const int t = blockIdx.x, h = threadIdx.x;
  const bool active = h < H;
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  {
    const f64x2 v = reinterpret_cast<const f64x2*>(tsum + (size_t)t * kHeadDim)[h];
    reinterpret_cast<f64x2*>(ts)[h] = v;
  }
  u32x4 qv[kHeadDim / 8];
  if (active) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)t * H + h) * kHeadDim);
#pragma unroll
    for (int v = 0; v < kHeadDim / 8; ++v) qv[v] = src[v];
  }
  double m = 0.0;
  const double* pm = pmax + (size_t)t * nchunk * kWave + h;
  int c = 0;
  for (; c + 8 <= nchunk; c += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = pm[(size_t)(c + u) * kWave];
#pragma unroll
    for (int u = 0; u < 8; ++u) m = v[u] > m ? v[u] : m;
  }
  for (; c < nchunk; ++c) {
    const double v = pm[(size_t)c * kWave];
    m = v > m ? v : m;
  }
  __syncthreads();
  if (Mt > 0) {
    const int cnt = n - (int)((long long)(Mt - 1) * B);
    double acc = 0.0;
    if (active) {
#pragma unroll
      for (int v = 0; v < kHeadDim / 8; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fma((double)bf16_bits_to_f32(qv[v][e] & 0xffffu), ts[8 * v + 2 * e], acc);
          acc = fma((double)bf16_bits_to_f32(qv[v][e] >> 16), ts[8 * v + 2 * e + 1], acc);
        }
    }
    const double rho = acc / (double)cnt;
    m = rho > m ? rho : m;
    if (beta) {
      const double contrib = active ? (double)w[(size_t)t * H + h] * (rho > 0.0 ? rho : 0.0) : 0.0;
      const double s = wave_sum(contrib);
      if (h == 0) beta[(size_t)t * beta_ld + Mt - 1] = (float)s;
    }
  }
  const double r = active ? (double)w[(size_t)t * H + h] * m + 0.0 : -__builtin_huge_val();
  if (r_out && active) r_out[(size_t)t * H + h] = (float)r;
  if (heads) {
    rs[h] = r;
    __syncthreads();
    int rank = 0;
    for (int h2 = 0; h2 < kWave; ++h2) rank += (rs[h2] > r) || (rs[h2] == r && h2 < h);
    const bool sel = active && rank < A;
    const uint64_t mask = wave_ballot(sel);
    if (sel) heads[(size_t)t * A + lanes_below(mask)] = h;
    if (qr) {
      // the routed q rows and weights, packed in slot order for the scoring kernel
      if (sel) {
        const int j = lanes_below(mask);
        wr[(size_t)t * A + j] = w[(size_t)t * H + h];
        const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)t * H + h) * kHeadDim);
        u32x4* dst = reinterpret_cast<u32x4*>(qr + ((size_t)t * A + j) * kHeadDim);
#pragma unroll
        for (int v = 0; v < kHeadDim / 8; ++v) dst[v] = src[v];
      }
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
                             double* tsum) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int grid = M + (tsum ? T : 0);
  if (grid == 0) return hipSuccess;
  if (fp8)
    return cx.launch("block_sums", k_block_sums<true>, dim3(grid), dim3(256), 0, K, kscale, L, B, M,
                     ksum, kbar, pos, tsum);
  return cx.launch("block_sums", k_block_sums<false>, dim3(grid), dim3(256), 0, K, kscale, L, B, M,
                   ksum, kbar, pos, tsum);
}

int route_chunks(int L, int B) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int c = (M + kRouteChunk - 1) / kRouteChunk;
  return c < 1 ? 1 : c;
}

hipError_t launch_route(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                        int T, int H, int L, int B, int A, const double* ksum, const double* tsum,
                        double* pmax, int32_t* heads, float* r_out, float* beta, int beta_ld,
                        uint16_t* qr, float* wr) {
  if (T == 0) return hipSuccess;
  const int nch = route_chunks(L, B);
  hipError_t e;
  if (beta)
    e = cx.launch("route_partial", k_route_partial<true>, dim3(nch, T), dim3(256), 0, q, w, pos, H,
                  L, B, nch, ksum, pmax, beta, beta_ld);
  else
    e = cx.launch("route_partial", k_route_partial<false>, dim3(nch, T), dim3(256), 0, q, w, pos,
                  H, L, B, nch, ksum, pmax, beta, beta_ld);
  if (e != hipSuccess) return e;
  return cx.launch("route_select", k_route_select, dim3(T), dim3(64), 0, q, w, pos, H, L, B, A, nch,
                   (const double*)pmax, tsum, heads, r_out, beta, beta_ld, qr, wr);
}

hipError_t launch_gather_heads(const LaunchCtx& cx, const uint16_t* q, const float* w,
                               const int32_t* heads, int T, int H, int A, uint16_t* qr, float* wr) {
  if (T == 0) return hipSuccess;
  return cx.launch("gather_heads", k_gather_heads, dim3(A, T), dim3(64), 0, q, w, heads, H, A, qr, wr);
}

}  // namespace misa
