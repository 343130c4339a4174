// Shared device-side definitions for the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define G355_LDS __attribute__((address_space(3)))
#define G355_GLOBAL __attribute__((address_space(1)))

enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_ERF = 2, ACT_GELU_TANH = 3 };

// Everything a GEMM launch needs; passed by value as the kernel argument.
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  const uint16_t* bias;   // BF16[N] or nullptr
  const float* scale_a;   // FP32[M] (FP8 only)
  const float* scale_b;   // FP32[N] (FP8 only)
  float* workspace;       // split-K partials
  int64_t lda, ldb, ldc;
  int M, N, K;
  float alpha, beta;
  int act;
  int a_mn_major;         // 1: A stored column-major (M contiguous), read by the generic loader
  int b_mn_major;         // 1: B stored row-major (N contiguous), read by the generic loader
  int c_vec;              // 1: C rows allow 4-element vector access (aligned base, ldc % 4 == 0)
  int split_k;            // number of K partitions
  int k_split_len;        // elements of K per partition (multiple of the K tile)
  int tiles_m, tiles_n;
};

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// FP32 -> BF16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; a
// NaN stays a quiet NaN). Two values per instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2_bits(f, 0.f));
}

// ---------------------------------------------------------------- epilogue math

// e^x from the hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for x >= 0, erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5)
// e^(-x^2) with t = 1 / (1 + p x), |error| <= 1.5e-7; odd symmetry for x < 0.
// About a dozen VALU operations (one hardware exp, one hardware reciprocal)
// instead of a full-precision library erf.
__device__ __forceinline__ float erf_as7126(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * ax);
  float poly = 1.061405429f;
  poly = poly * t - 1.453152027f;
  poly = poly * t + 1.421413741f;
  poly = poly * t - 0.284496736f;
  poly = poly * t + 0.254829592f;
  poly = poly * t;
  const float r = 1.f - poly * fast_exp(-ax * ax);
  return copysignf(r, x);
}

__device__ __forceinline__ float apply_act(float z, int act) {
  if (act == ACT_RELU) return z > 0.f ? z : 0.f;
  if (act == ACT_GELU_ERF) {
    const float hz = 0.5f * z;
    return fmaf(hz, erf_as7126(z * 0.70710678118654752f), hz);
  }
  if (act == ACT_GELU_TANH) {
    // tanh(u) = 1 - 2 / (1 + e^(2u)); saturates correctly for large |u|.
    const float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);  // sqrt(2/pi) (...)
    const float th = 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + fast_exp(2.f * u));
    return 0.5f * z * (1.f + th);
  }
  return z;
}

// ---------------------------------------------------------------- tile scheduling

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8), and each XCD has its own L2. Renumber so that each XCD receives
// a contiguous range of logical tile ids; with the grouped order below, the
// tiles of one XCD then share A row-panels and B column-panels in its L2.
__device__ __forceinline__ int xcd_remap(int b, int nwg) {
  constexpr int X = 8;
  const int per = nwg / X, rem = nwg % X;
  const int x = b % X, i = b / X;
  return x * per + (x < rem ? x : rem) + i;
}

// Logical tile id -> (tile_m, tile_n), grouped GROUP_M tile rows at a time,
// column-major inside a group.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m,
                                            int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int r = t - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

}  // namespace g355
