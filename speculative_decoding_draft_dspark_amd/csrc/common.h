// Device-side helpers shared by the DSpark loss kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef uint16_t bf16_t;  // bf16 stored as its raw bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_v;
typedef __attribute__((ext_vector_type(4))) float f32x4_v;

constexpr int kWave = 64;
constexpr int kStatTile = 64;   // vocab columns per softmax-statistics tile
constexpr int kGemmTileN = 256;  // output columns of a logits GEMM tile (4 statistics tiles)
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (NaN stays NaN): gfx950 converts in
// hardware (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// lo -> bits 0..15, hi -> bits 16..31, both rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static float to_f32(float x) { return x; }
  // 4 consecutive elements (16-byte aligned) widened to fp32
  __device__ static float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
  typedef float4 Raw4;  // 4 elements as loaded
  __device__ static Raw4 load4raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static float4 widen4(const Raw4& r) { return r; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;
  __device__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static float to_f32(bf16_t x) { return bf16_to_f32(x); }
  // 4 consecutive elements (8-byte aligned) widened to fp32
  __device__ static float4 load4(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  typedef uint2 Raw4;  // 4 elements as loaded
  __device__ static Raw4 load4raw(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ static float4 widen4(const Raw4& u) {
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
};

// The one exponential every softmax statistic and probability goes through,
// so that equal logits give bitwise-equal probabilities on both sides.
__device__ __forceinline__ float dexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float sgnf(float x) { return x > 0.f ? 1.f : (x < 0.f ? -1.f : 0.f); }
// exp(x - m) for x <= m in the fixed point (2^25 scale) of the tile
// exp-sums, as 2^(x log2 e + 25 - m log2 e) truncated to an integer (one fma,
// one exp2, one conversion).  At x = m the exponent is 25 plus the rounding
// error of m log2 e (below 1/2 for |m| < 10^7), so a 64-column statistics
// tile sums to less than 64 x 2^25.5 < 2^32: every tile sum is one 32-bit
// integer, exact and independent of the order of the columns.  The
// truncation costs at most 64 x 2^-25 of a sum that is at least 1.  Every
// kernel that produces tile statistics uses these routines, so equal rows
// give bitwise-equal statistics.
constexpr float kFixBits = 25.f;
__device__ __forceinline__ float fix_exp_offset(float m) { return kFixBits - m * kLog2e; }
__device__ __forceinline__ uint32_t fix_exp32o(float x, float off) {
  return static_cast<uint32_t>(__builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, off)));
}
__device__ __forceinline__ uint32_t fix_exp32(float x, float m) {
  return fix_exp32o(x, fix_exp_offset(m));
}
// A tile's fixed-point exp-sum as the float sum of exp(x - max).
__device__ __forceinline__ float fix_to_float(uint32_t s) {
  return static_cast<float>(s) * 0x1p-25f;
}

// ---- reductions -----------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Block-wide reductions with a fixed combination order (deterministic).
// `scratch` must hold blockDim.x / 64 elements; the result is returned to all threads.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* scratch) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  float r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, scratch[i]);
  return r;
}
template <int NT>
__device__ __forceinline__ double block_sum(double v, double* scratch) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  double r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r += scratch[i];
  return r;
}

}  // namespace dspark
