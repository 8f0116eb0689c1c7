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
// Eight consecutive key dims [8*dg, 8*dg+8) of key s, widened to float64.
template <bool FP8>
__device__ __forceinline__ void load_key8_f64(const void* K, const float* kscale, int s, int dg,
                                              double out[8]) {
  if constexpr (!FP8) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(K) +
                                                    (size_t)s * kHeadDim + dg * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = (double)bf16_bits_to_f32(v[j] & 0xffffu);
      out[2 * j + 1] = (double)bf16_bits_to_f32(v[j] >> 16);
    }
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(K) +
                                                    (size_t)s * kHeadDim + dg * 8);
    const double sc = (double)kscale[s];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
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

// Sum of key rows [s0, s1) in float64, one workgroup of 256 threads; thread
// (rl, dg) takes rows rl, rl+16, ... and dims [8dg, 8dg+8). Result lands in
// red[0][*] ... the caller reads column sums from `red`.
template <bool FP8>
__device__ __forceinline__ void sum_rows_f64(const void* K, const float* kscale, int s0, int s1,
                                             double (*red)[kHeadDim]) {
  const int tid = threadIdx.x, dg = tid & 15, rl = tid >> 4;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int s = s0 + rl; s < s1; s += 16) {
    double v[8];
    load_key8_f64<FP8>(K, kscale, s, dg, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][dg * 8 + e] = acc[e];
  __syncthreads();
}

// ksum[b,:] = sum of keys of block b = [b*B, min((b+1)*B, L)) (float64).
// kbar (optional) = ksum / count rounded once to float32.
template <bool FP8>
__global__ __launch_bounds__(256) void k_block_sums(const void* K, const float* kscale, int L,
                                                    int B, double* ksum, float* kbar) {
  __shared__ double red[16][kHeadDim];
  const int b = blockIdx.x;
  const long long s0 = (long long)b * B;
  const int s1 = (int)(s0 + B < L ? s0 + B : L);
  sum_rows_f64<FP8>(K, kscale, (int)s0, s1, red);
  const int tid = threadIdx.x;
  if (tid < kHeadDim) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    ksum[(size_t)b * kHeadDim + tid] = s;
    if (kbar) kbar[(size_t)b * kHeadDim + tid] = (float)(s / (double)(s1 - (int)s0));
  }
}

// tsum[t,:] = sum of the keys of query t's last block [(M_t-1)*B, n_t)
// (possibly partial); zero when the query sees no key.
template <bool FP8>
__global__ __launch_bounds__(256) void k_tail_sums(const void* K, const float* kscale, int L, int B,
                                                   const int32_t* pos, double* tsum) {
  __shared__ double red[16][kHeadDim];
  const int t = blockIdx.x;
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  const int s0 = Mt > 0 ? (int)((long long)(Mt - 1) * B) : 0;
  sum_rows_f64<FP8>(K, kscale, s0, n, red);
  const int tid = threadIdx.x;
  if (tid < kHeadDim) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    tsum[(size_t)t * kHeadDim + tid] = s;
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
  __shared__ double ks[kRouteChunk][kHeadDim];
  __shared__ double wmax[4][kWave];
  const int c = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, h = tid & 63, j = tid >> 6;
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
  for (int e = tid; e < nb * kHeadDim; e += 256) ks[e / kHeadDim][e % kHeadDim] = ksum[(size_t)b0 * kHeadDim + e];

  const bool active = h < H;
  float qf[kHeadDim];
  if (active) {
    const u32x4* src = reinterpret_cast<const u32x4*>(q + ((size_t)t * H + h) * kHeadDim);
#pragma unroll
    for (int v = 0; v < kHeadDim / 8; ++v) {
      const u32x4 x = src[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[8 * v + 2 * e] = bf16_bits_to_f32(x[e] & 0xffffu);
        qf[8 * v + 2 * e + 1] = bf16_bits_to_f32(x[e] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kHeadDim; ++i) qf[i] = 0.f;
  }
  const double wh = active ? (double)w[(size_t)t * H + h] : 0.0;
  __syncthreads();

  const int per = (nb + 3) / 4;
  const int bl0 = j * per, bl1 = min(nb, bl0 + per);
  double m = 0.0;
  for (int bl = bl0; bl < bl1; bl += 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const int cnt = min(4, bl1 - bl);
#pragma unroll
    for (int i = 0; i < kHeadDim; ++i) {
      const double qd = (double)qf[i];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < cnt) acc[u] = fma(qd, ks[bl + u][i], acc[u]);
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
                                                    float* r_out, float* beta, int beta_ld) {
  __shared__ double rs[kWave];
  const int t = blockIdx.x, h = threadIdx.x;
  const bool active = h < H;
  const int n = visible_len(pos[t], L);
  const int Mt = (int)(((long long)n + B - 1) / B);
  double m = 0.0;
  for (int c = 0; c < nchunk; ++c) {
    const double v = pmax[((size_t)t * nchunk + c) * kWave + h];
    m = v > m ? v : m;
  }
  if (Mt > 0) {
    const int cnt = n - (int)((long long)(Mt - 1) * B);
    double acc = 0.0;
    if (active) {
      const uint16_t* qr = q + ((size_t)t * H + h) * kHeadDim;
      const double* ts = tsum + (size_t)t * kHeadDim;
      for (int i = 0; i < kHeadDim; ++i) acc = fma((double)bf16_bits_to_f32(qr[i]), ts[i], acc);
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
  }
}

// -------------------------------------------------------------------------
// Host launchers.

hipError_t launch_block_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                             int L, int B, double* ksum, float* kbar) {
  const int M = (int)(((long long)L + B - 1) / B);
  if (M == 0) return hipSuccess;
  if (fp8)
    return cx.launch("block_sums", k_block_sums<true>, dim3(M), dim3(256), 0, K, kscale, L, B, ksum, kbar);
  return cx.launch("block_sums", k_block_sums<false>, dim3(M), dim3(256), 0, K, kscale, L, B, ksum, kbar);
}

hipError_t launch_tail_sums(const LaunchCtx& cx, const void* K, const float* kscale, bool fp8,
                            int L, int B, int T, const int32_t* pos, double* tsum) {
  if (T == 0) return hipSuccess;
  if (fp8)
    return cx.launch("tail_sums", k_tail_sums<true>, dim3(T), dim3(256), 0, K, kscale, L, B, pos, tsum);
  return cx.launch("tail_sums", k_tail_sums<false>, dim3(T), dim3(256), 0, K, kscale, L, B, pos, tsum);
}

int route_chunks(int L, int B) {
  const int M = (int)(((long long)L + B - 1) / B);
  const int c = (M + kRouteChunk - 1) / kRouteChunk;
  return c < 1 ? 1 : c;
}

hipError_t launch_route(const LaunchCtx& cx, const uint16_t* q, const float* w, const int32_t* pos,
                        int T, int H, int L, int B, int A, const double* ksum, const double* tsum,
                        double* pmax, int32_t* heads, float* r_out, float* beta, int beta_ld) {
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
                   (const double*)pmax, tsum, heads, r_out, beta, beta_ld);
}

}  // namespace misa
