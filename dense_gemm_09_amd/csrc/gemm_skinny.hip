// Skinny GEMM for decode-sized M (M <= 16): HBM-bound weight streaming.
//
// With M this small the GEMM reads each weight byte (B, N x K, K-major) once
// and does little arithmetic with it (the M = 1 row of the first DeepGEMM
// page's sec. 5.1 table runs at 15% of peak for exactly this reason: the data
// is not reused). The work is therefore arranged to keep HBM busy rather than
// the matrix cores:
//
// * A workgroup owns 16 output columns; its KW waves split K into KW
//   contiguous ranges. Every lane streams its own 16 bytes of B per k-step
//   straight from HBM into the MFMA B operand (no LDS staging: each weight
//   byte is used by exactly one wave), with U k-steps of loads issued before
//   any is consumed, so each wave keeps U x 1 KB (BF16) or U x 2 KB (FP8) in
//   flight.
// * A (M x K, a few hundred KB at most) is read from L2 by every workgroup.
// * The inner product uses v_mfma_f32_16x16x32_bf16 / the 16x16x128 FP8
//   (f8f6f4, E4M3, scale 2^0) MFMA with M padded to 16 (MB blocks of 16 rows;
//   rows past M are zero lanes and are never stored). A and B fragments hold
//   the same K indices in the same register slots.
// * The KW partial sums are added through LDS in wave order 0..KW-1 (fixed
//   order: bitwise reproducible), then the same epilogue as the tile kernel
//   runs: act(alpha * scale_a[m] * scale_b[n] * acc + beta * C + bias).
//
// 16x16 MFMA accumulator layout: element e of lane l is row 4*(l/16) + e,
// column l%16.

#include "common.hpp"
#include "internal.hpp"

namespace g355 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <bool FP8, int MB, int KW, int U>
struct SkinnyCfg {
  static constexpr int ES = FP8 ? 1 : 2;
  static constexpr int KSTEP = FP8 ? 128 : 32;        // K elements per MFMA
  static constexpr int LANE_BYTES = FP8 ? 32 : 16;    // bytes of one operand row per lane per MFMA
  static constexpr int NT = KW * 64;
};

template <class S, int OUT, int MB, int ACT>
__device__ __forceinline__ void skinny_epilogue(const GemmArgs& p, const f32x4 (&acc)[MB], int n0,
                                                int lane) {
  const int n = n0 + (lane & 15);
  if (n >= p.N) return;
  float sb = 1.f, bias_v = 0.f;
  if constexpr (S::ES == 1) sb = p.scale_b[n];
  if (p.bias) bias_v = bf16_bits_to_f32(p.bias[n]);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 16 * mb + 4 * (lane >> 4) + e;
      if (m >= p.M) continue;
      float z = acc[mb][e];
      if constexpr (S::ES == 1) z = z * (p.scale_a[m] * sb);
      z = p.alpha * z;
      const int64_t off = static_cast<int64_t>(m) * p.ldc + n;
      if constexpr (OUT == OUT_F32 || OUT == OUT_BF16) {
        if (p.beta != 0.f) z += p.beta * load_cin1<OUT>(p.C, off);
      }
      z = apply_act<OUT>(z + bias_v, ACT);
      float qs, qz;
      out_row_params<OUT>(p, m, qs, qz);
      store_out1<OUT>(p.C, off, z, qs, qz);
    }
  }
}

template <bool FP8, int MB, int KW, int U, int OUT>
__global__ void __launch_bounds__(KW * 64) gemm_skinny_kernel(GemmArgs p) {
  using S = SkinnyCfg<FP8, MB, KW, U>;
  __shared__ __attribute__((aligned(16))) f32x4 red[KW][MB][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int g = lane >> 4;  // K group of this lane inside one MFMA

  // K range of this wave (multiples of KSTEP; the last ranges may be short or empty).
  const int ksteps = (p.K + S::KSTEP - 1) / S::KSTEP;
  const int per = (ksteps + KW - 1) / KW;
  const int kb = wave * per * S::KSTEP;
  const int ke = min(p.K, kb + per * S::KSTEP);

  // B row of this lane (clamped past N; those columns are never stored).
  int nb = n0 + (lane & 15);
  nb = nb < p.N ? nb : p.N - 1;
  const char* brow = static_cast<const char*>(p.B) + static_cast<int64_t>(nb) * p.ldb * S::ES;
  const char* arow[MB];
  bool a_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + (lane & 15);
    a_ok[mb] = m < p.M;
    arow[mb] = static_cast<const char*>(p.A) +
               static_cast<int64_t>(a_ok[mb] ? m : 0) * p.lda * S::ES;
  }

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One MFMA's worth of a lane's operand: 16 (BF16) or 32 (FP8) bytes at
  // element k = k0 + g * (LANE_BYTES / ES); chunks at or past K are zero
  // (K is a multiple of 16 bytes' worth of elements on this path).
  auto ld = [&](const char* row, int k0, bool ok) {
    i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    const int k = k0 + g * (S::LANE_BYTES / S::ES);
    const char* a = row + static_cast<int64_t>(k) * S::ES;
    if (ok && k < ke) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(a);
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    }
    if constexpr (S::LANE_BYTES == 32) {
      if (ok && k + 16 < ke) {
        const i32x4 hi = *reinterpret_cast<const i32x4*>(a + 16);
        v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      }
    }
    return v;
  };

  for (int k0 = kb; k0 < ke; k0 += U * S::KSTEP) {
    i32x8 bv[U], av[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) bv[u] = ld(brow, k0 + u * S::KSTEP, true);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) av[u][mb] = ld(arow[mb], k0 + u * S::KSTEP, a_ok[mb]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if constexpr (FP8) {
          acc[mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[u][mb], bv[u], acc[mb], 0,
                                                                     0, 0, 127, 0, 127);
        } else {
          const i32x4 a4 = {av[u][mb][0], av[u][mb][1], av[u][mb][2], av[u][mb][3]};
          const i32x4 b4 = {bv[u][0], bv[u][1], bv[u][2], bv[u][3]};
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a4), __builtin_bit_cast(bf16x8_t, b4), acc[mb], 0, 0, 0);
        }
      }
    }
  }

  // Fixed-order reduction of the KW partial sums.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) red[wave][mb][lane] = acc[mb];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x4 s = red[0][mb][lane];
#pragma unroll
    for (int w = 1; w < KW; ++w) s += red[w][mb][lane];
    acc[mb] = s;
  }
  const int act = p.act;
  if (act == ACT_NONE) skinny_epilogue<S, OUT, MB, ACT_NONE>(p, acc, n0, lane);
  else if (act == ACT_RELU) skinny_epilogue<S, OUT, MB, ACT_RELU>(p, acc, n0, lane);
  else if (act == ACT_GELU_ERF) skinny_epilogue<S, OUT, MB, ACT_GELU_ERF>(p, acc, n0, lane);
  else skinny_epilogue<S, OUT, MB, ACT_GELU_TANH>(p, acc, n0, lane);
}

#ifndef G355_KERNELS_ONLY
// KW = 16 K-split waves per workgroup; U k-steps of loads in flight per wave
// (BF16 4 x 1 KB, FP8 2 x 2 KB). Chosen by a sweep at K = 4096, N = 4096..18432.
template <bool FP8, int MB>
static hipError_t launch_mb(const GemmArgs& a, int out, hipStream_t stream) {
  constexpr int KW = 16;
  constexpr int U = FP8 ? 2 : 4;
  const dim3 grid(static_cast<unsigned>((a.N + 15) / 16)), block(KW * 64);
  if (out == OUT_BF16)
    hipLaunchKernelGGL((gemm_skinny_kernel<FP8, MB, KW, U, OUT_BF16>), grid, block, 0, stream, a);
  else if (out == OUT_I8)
    hipLaunchKernelGGL((gemm_skinny_kernel<FP8, MB, KW, U, OUT_I8>), grid, block, 0, stream, a);
  else if (out == OUT_E4M3)
    hipLaunchKernelGGL((gemm_skinny_kernel<FP8, MB, KW, U, OUT_E4M3>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<FP8, MB, KW, U, OUT_F32>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_skinny(const Plan& plan, const LaunchSpec& spec, const GemmArgs& a,
                         hipStream_t stream) {
  (void)plan;
  if (a.M > 16) return hipErrorInvalidValue;  // the plan only selects M <= 16
  return spec.fp8 ? launch_mb<true, 1>(a, spec.out, stream)
                  : launch_mb<false, 1>(a, spec.out, stream);
}
#endif  // G355_KERNELS_ONLY

}  // namespace g355
