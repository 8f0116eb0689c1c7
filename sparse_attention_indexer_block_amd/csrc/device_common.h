// Device-side helpers shared by the indexer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace misa {

constexpr int kHeadDim = 128;   // d supported by the kernels
constexpr int kMaxHeads = 64;   // H supported by the kernels
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// Visible prefix length of a query at position `pos` among L keys (clamped).
__device__ __forceinline__ int visible_len(int pos, int L) {
  int n = pos + 1;
  return n < 0 ? 0 : (n > L ? L : n);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// Two OCP E4M3FN bytes (byte 0/1 or 2/3 of `packed`) -> two bf16 packed in a
// dword (HIGH_WORD selects bytes 2/3). The conversion is exact: E4M3 values have 4 significant bits and an
// exponent range inside bf16's. Scale 1.0 (exponent 127) leaves values as is.
template <bool HIGH_WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t packed) {
  bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)packed, 1.0f, HIGH_WORD);
  return __builtin_bit_cast(uint32_t, v);
}

// Two E4M3FN bytes -> two fp32 values (exact, one conversion instruction).
template <bool HIGH_WORD>
__device__ __forceinline__ void fp8x2_to_f32(uint32_t packed, float& a, float& b) {
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)packed, 1.0f, HIGH_WORD);
  a = v.x;
  b = v.y;
}

// ReLU on the bits: negative values (and -0.0) give +0.0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Order-preserving map float -> uint32 (larger float -> larger key); -0.0 is
// folded onto +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t u) {
  uint32_t b = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(b);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// A float64 value as bf16 hi + lo (hi = bf16(float(m)), lo = bf16(float(m - hi)));
// |m - hi - lo| <= 2^-17.9 |m|.
__device__ __forceinline__ void split_bf16(double m, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne((float)m);
  lo = bf16_rne((float)(m - (double)bf16_bits_to_f32(hi)));
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

template <typename Tv>
__device__ __forceinline__ Tv wave_sum(Tv v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <typename Tv>
__device__ __forceinline__ Tv wave_max(Tv v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Tv o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// Inclusive prefix sum across one wave, on the DPP network: a Hillis-Steele
// scan inside each row of 16 lanes, then row 15's total is broadcast into rows
// 1 and 3, and lane 31's into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31
  return v;
}

// Wave-wide minimum / maximum (every lane gets the result): DPP rotations inside
// each row of 16 lanes, then the four row results through readlane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = pick(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x121, 0xf, 0xf, false));  // row_ror:1
  const uint32_t a = pick((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = pick((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return pick(a, b);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_ext_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_ext_u32<true>(v); }

// Sum over the wave, returned in every lane: rows of 16 lanes reduce with
// rotations, then the four row totals are read out as scalars.
__device__ __forceinline__ uint32_t wave_total_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false);  // row_ror:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false);  // row_ror:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false);  // row_ror:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false);  // row_ror:1
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

}  // namespace misa
