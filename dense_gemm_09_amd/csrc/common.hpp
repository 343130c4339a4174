// Shared device-side definitions for the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define G355_LDS __attribute__((address_space(3)))

enum Act : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_ERF = 2, ACT_GELU_TANH = 3 };

// What the epilogue writes: FP32 or BF16 C (read back when beta != 0), or a
// quantised tensor of one byte per element with a per-row output scale
// (INT8 with a per-row zero point, or OCP E4M3FN), never read.
enum OutKind : int { OUT_F32 = 0, OUT_BF16 = 1, OUT_I8 = 2, OUT_E4M3 = 3 };

// Everything a GEMM launch needs; passed by value as the kernel argument.
struct GemmArgs {
  const void* A;
  const void* B;
  void* C;
  const uint16_t* bias;   // BF16[N] or nullptr
  const float* scale_a;   // FP32[M] (FP8 only)
  const float* scale_b;   // FP32[N] (FP8 only)
  float* workspace;       // split-K partials
  const float* qscale;    // FP32[M] output scale (quantised outputs)
  const int32_t* qzero;   // INT32[M] output zero point (INT8 output) or nullptr
  const uint8_t* mx_a;    // E8M0 block scales of A: M rows of ldsa bytes (MX FP8 only)
  const uint8_t* mx_b;    // E8M0 block scales of B: N rows of ldsb bytes
  int ldsa, ldsb;         // bytes per row of mx_a / mx_b (multiples of 4)
  int64_t lda, ldb, ldc;
  int M, N, K;
  float alpha, beta;
  int act;
  int a_mn_major;         // 1: A stored column-major (M contiguous), read by the generic loader
  int b_mn_major;         // 1: B stored row-major (N contiguous), read by the generic loader
  int c_vec;              // 1: C rows allow 4-element vector access (aligned base, ldc % 4 == 0)
  int ws_vec;             // 1: the workspace is 16-byte aligned
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

// Four FP32 values -> four OCP E4M3FN codes in one word (byte q holds value q):
// clamped to +-448, then gfx950's v_cvt_pk_fp8_f32 (round to nearest even).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const float lim = 448.f;
  a = __builtin_amdgcn_fmed3f(a, -lim, lim);
  b = __builtin_amdgcn_fmed3f(b, -lim, lim);
  c = __builtin_amdgcn_fmed3f(c, -lim, lim);
  d = __builtin_amdgcn_fmed3f(d, -lim, lim);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// INT8 output code of y: round to nearest even of fp32(y * s + zp) (one
// rounding, fused multiply-add), saturated to [-128, 127]; low byte of the
// result. Clamping before rounding gives the same code: the bounds are integers.
__device__ __forceinline__ uint32_t quant_i8(float y, float s, float zp) {
  const float v = __builtin_amdgcn_fmed3f(fmaf(y, s, zp), -128.f, 127.f);
  return static_cast<uint32_t>(static_cast<int>(__builtin_rintf(v))) & 0xffu;
}

// Element `off` of an output of kind OUT. s and zp: the row's output scale and
// zero point (quantised kinds only).
template <int OUT>
__device__ __forceinline__ void store_out1(void* C, int64_t off, float v, float s, float zp) {
  if constexpr (OUT == OUT_F32) {
    static_cast<float*>(C)[off] = v;
  } else if constexpr (OUT == OUT_BF16) {
    static_cast<uint16_t*>(C)[off] = f32_to_bf16_bits(v);
  } else if constexpr (OUT == OUT_I8) {
    static_cast<uint8_t*>(C)[off] = static_cast<uint8_t>(quant_i8(v, s, zp));
  } else {
    static_cast<uint8_t*>(C)[off] = static_cast<uint8_t>(e4m3x4(v * s, 0.f, 0.f, 0.f) & 0xffu);
  }
}

// Elements off..off+3 in one store (16, 8 or 4 bytes, aligned by the caller).
// The stores are non-temporal: C is written once at the end of a tile and not
// read again by the kernel, so it need not displace A and B panels from the
// caches (measured at 4096^3 together with non-temporal C_in loads: ~5% off
// the BF16 and the FP8 kernel).
template <int OUT>
__device__ __forceinline__ void store_out4(void* C, int64_t off, const float (&v)[4], float s,
                                           float zp) {
  if constexpr (OUT == OUT_F32) {
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]},
                                reinterpret_cast<f32x4*>(static_cast<float*>(C) + off));
  } else if constexpr (OUT == OUT_BF16) {
    u32x2 h;
    h.x = f32x2_to_bf16x2_bits(v[0], v[1]);
    h.y = f32x2_to_bf16x2_bits(v[2], v[3]);
    __builtin_nontemporal_store(h, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(C) + off));
  } else if constexpr (OUT == OUT_I8) {
    const uint32_t w = quant_i8(v[0], s, zp) | (quant_i8(v[1], s, zp) << 8) |
                       (quant_i8(v[2], s, zp) << 16) | (quant_i8(v[3], s, zp) << 24);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(C) + off));
  } else {
    __builtin_nontemporal_store(e4m3x4(v[0] * s, v[1] * s, v[2] * s, v[3] * s),
                                reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(C) + off));
  }
}

// The row's output scale and zero point (1 and 0 for unquantised kinds).
template <int OUT>
__device__ __forceinline__ void out_row_params(const GemmArgs& p, int m, float& s, float& zp) {
  s = 1.f;
  zp = 0.f;
  if constexpr (OUT >= OUT_I8) s = p.qscale[m];
  if constexpr (OUT == OUT_I8) {
    if (p.qzero) zp = static_cast<float>(p.qzero[m]);
  }
}

// C_in element as FP32 (only the FP32 and BF16 kinds are ever read).
template <int OUT>
__device__ __forceinline__ float load_cin1(const void* C, int64_t off) {
  if constexpr (OUT == OUT_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(C)[off]);
  else return static_cast<const float*>(C)[off];
}

// ---------------------------------------------------------------- epilogue math

// P(t) of the Chebyshev-fitted complementary error function of Numerical
// Recipes in C (2nd ed., sec. 6.2, "erfcc"): for x >= 0,
//   erfc(x) = t exp(-x^2 + P(t)),  t = 1 / (1 + x/2),
// with a fractional error below 1.2e-7 for every x. Unlike 1 - erf(x), it
// keeps its relative accuracy where erfc(x) is tiny. P(1) = 0 (erfc(0) = 1)
// and P(t) <= 0 on (0, 1].
__device__ __forceinline__ float erfc_cheb_poly(float t) {
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  return p;
}

// Q(t) = log2(e) P(t) + 63 for the same t = 1 / (1 + x/2), as one degree-7
// polynomial: a least-squares fit over t in [1/7, 1] (x <= 12), within 2e-6
// of Q there (dense_gemm_09_amd/gelu_fit.py makes the table). The 2^63 keeps
// 2^Q e^(-x^2) normal far into GELU's negative tail; the caller scales by
// 2^-64, which also supplies GELU's factor 1/2. Used for BF16 and quantised
// outputs, where it is accurate well below half a BF16 ulp.
__device__ __forceinline__ float erfc_log2_fit7(float t) {
  float q = -0.27580565214157104f;
  q = fmaf(q, t, 1.1046985387802124f);
  q = fmaf(q, t, -1.4792454242706299f);
  q = fmaf(q, t, 0.5366070866584778f);
  q = fmaf(q, t, -0.07367606461048126f);
  q = fmaf(q, t, 0.5731409788131714f);
  q = fmaf(q, t, 1.439933180809021f);
  q = fmaf(q, t, 61.174346923828125f);
  return q;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwoM64 = 5.42101086242752217e-20f;  // 2^-64

// 2^q for a double q <= 0 as (r, n) with 2^q = r * 2^n, n integral, r in
// [2^-0.5, 2^0.5] from the hardware exponential: the FP32 rounding sees only
// the fraction, so r carries about one FP32 ulp of error whatever q is.
__device__ __forceinline__ float exp2_split(double q, int& n) {
  q = q < -400.0 ? -400.0 : q;  // far past FP32's range either way
  const double nd = __builtin_rint(q);
  n = static_cast<int>(nd);
  return __builtin_amdgcn_exp2f(static_cast<float>(q - nd));
}

// GELU(z) = z Phi(z) = z - w for z >= 0 and w for z < 0, where
//   w = (z/2) erfc(|z|/sqrt 2) = (z/2) t exp(P(t) - z^2/2)
// (Phi(z) = erfc(-z/sqrt 2)/2). No difference of nearby numbers is formed, so
// the result keeps its relative accuracy far into the negative range, and the
// exponential's power-of-two scale is applied last, so that w stays accurate
// down into FP32's subnormal range (erfc alone, smaller by |z|/2, would
// underflow first). The exponent P - z^2/2 is one fused multiply-add from z
// itself (z/2 is exact). PRECISE forms it in double and splits off its power
// of two exactly (relative error ~5e-7 for every z; FP32 outputs). Otherwise
// (BF16 and quantised outputs) the exponent is log2(e) (P - z^2/2) + 63 from
// the fitted Q(t) and one fused multiply-add, the result is scaled by 2^-64
// at the end, and the FP32 roundings leave a relative error of up to ~1e-5
// at the far negative end, far below a BF16 ulp.
template <bool PRECISE>
__device__ __forceinline__ float gelu_erf(float z) {
  // t = 1 / (1 + x/2), x = |z| / sqrt 2
  const float t = __builtin_amdgcn_rcpf(fmaf(fabsf(z), 0.35355339059327376f, 1.f));
  float w;
  if constexpr (PRECISE) {
    const float hz = 0.5f * z;
    const float p = erfc_cheb_poly(t);
    const double zd = z;
    int n;
    const float r = exp2_split((static_cast<double>(p) - 0.5 * zd * zd) * 1.4426950408889634074, n);
    w = __builtin_ldexpf(hz * t * r, n);
  } else {
    const float r = __builtin_amdgcn_exp2f(fmaf(z * z, -0.5f * kLog2e, erfc_log2_fit7(t)));
    w = (z * t * r) * kTwoM64;
  }
  return z < 0.f ? w : z - w;
}

// tanh-form GELU: 0.5 z (1 + tanh u) = z / (1 + e^(-a)), a = 2u = 2 sqrt(2/pi)
// (z + 0.044715 z^3). With E = e^(-|a|) in (0, 1]: z / (1 + E) for z >= 0, and
// z E / (1 + E) for z < 0 (no cancellation for either sign), E's power-of-two
// scale applied last as in gelu_erf. PRECISE forms a and E in double /
// by exp2_split.
template <bool PRECISE>
__device__ __forceinline__ float gelu_tanh(float z) {
  if constexpr (PRECISE) {
    const double zd = z;
    const double a = 1.5957691216057307118 * (zd + 0.044715 * zd * zd * zd);
    int n;
    const float r = exp2_split(-__builtin_fabs(a) * 1.4426950408889634074, n);
    const float d = __builtin_amdgcn_rcpf(1.f + __builtin_ldexpf(r, n));
    return z < 0.f ? __builtin_ldexpf(z * r * d, n) : z * d;
  } else {
    const float s = fmaf(0.044715f * z, z * z, z);  // u / sqrt(2/pi)
    const float r = __builtin_amdgcn_exp2f(fmaf(-fabsf(s), 1.5957691216057308f * kLog2e, 64.f));
    const float d = __builtin_amdgcn_rcpf(fmaf(r, kTwoM64, 1.f));
    return z < 0.f ? (z * r * d) * kTwoM64 : z * d;
  }
}

// Activation of the epilogue. OUT: the output kind; FP32 outputs take the
// precise GELU forms.
template <int OUT>
__device__ __forceinline__ float apply_act(float z, int act) {
  constexpr bool PRECISE = OUT == OUT_F32;
  if (act == ACT_RELU) return z > 0.f ? z : 0.f;
  if (act == ACT_GELU_ERF) return gelu_erf<PRECISE>(z);
  if (act == ACT_GELU_TANH) return gelu_tanh<PRECISE>(z);
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
