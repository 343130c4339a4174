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

#include <type_traits>

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

// Streaming variant, for K <= KW * KSM k-steps: one workgroup per CU walks the
// 16-column blocks b = blockIdx.x, blockIdx.x + G, ... (G workgroups). The A
// fragments of a wave's K range are the same for every block, so they are
// loaded once into registers; B, the only operand that streams from HBM, is
// loaded NBUF - 1 blocks ahead of the block being multiplied, so the loads of
// later blocks are in flight while a block's partial sums are reduced across
// the waves (in wave order 0..KW-1, as in the kernel above) and stored. The
// reduction area is double-buffered, so one barrier per block suffices.
// When the blocks do not divide into whole rounds of G and the last round
// holds at most G/2 of them, each of those can be split into two 8-column
// halves on two workgroups (the MFMA's other 8 columns get zero weights and
// are not stored): that round then moves half a block per workgroup instead
// of one block on half of them (N = 18432: 4.5 rounds instead of 5). Every
// output column is computed exactly as in a whole block.
// The last round is split for BF16 only: measured at K = 4096, it takes BF16
// M = 1 / 16, N = 18432 from 30.1 / 35.0 to 28.9 / 33.2 us, and leaves FP8
// (19 us, whose rate is not set by that round) where it was.
template <bool FP8>
constexpr bool kSplitLastRound = !FP8;

template <bool FP8, int KW, int KSM, int NBUF, int OUT, int ACT>
__global__ void __launch_bounds__(KW * 64) gemm_skinny_stream_kernel(GemmArgs p) {
  using S = SkinnyCfg<FP8, 1, KW, 1>;
  using Frag = typename std::conditional<FP8, i32x8, i32x4>::type;
  __shared__ __attribute__((aligned(16))) f32x4 red[2][KW][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;  // K group of this lane inside one MFMA
  const int ksteps = (p.K + S::KSTEP - 1) / S::KSTEP;
  const int per = (ksteps + KW - 1) / KW;  // k-steps per wave, <= KSM (checked on the host)
  const int kb = wave * per * S::KSTEP;
  const int ke = min(p.K, kb + per * S::KSTEP);
  const int nblk = (p.N + 15) / 16;
  const int G = gridDim.x;

  // One MFMA's worth of a lane's operand row (16 or 32 bytes at element
  // k0 + g * LANE_BYTES / ES); chunks at or past the wave's K end are zero.
  auto ld = [&](const char* row, int k0, bool ok) {
    Frag v = {};
    const int k = k0 + g * (S::LANE_BYTES / S::ES);
    const char* a = row + static_cast<int64_t>(k) * S::ES;
    if (ok && k < ke) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(a);
      v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
    }
    if constexpr (FP8) {
      if (ok && k + 16 < ke) {
        const i32x4 hi = *reinterpret_cast<const i32x4*>(a + 16);
        v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
      }
    }
    return v;
  };

  // A: rows 0..15 (rows past M are zero lanes, never stored).
  Frag av[KSM];
  {
    const int m = lane & 15;
    const bool ok = m < p.M;
    const char* arow = static_cast<const char*>(p.A) + static_cast<int64_t>(ok ? m : 0) * p.lda * S::ES;
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks) av[ks] = ld(arow, kb + ks * S::KSTEP, ok && ks < per);
  }
  // Work item i of this workgroup: its column range [col0, col0 + width).
  // Items 0..R-1 are the whole blocks blockIdx.x + i G; item R is its share
  // of the last, partial round (T blocks), whole or halved as described above.
  const int R = nblk / G, T = nblk - R * G;
  const bool halves = kSplitLastRound<FP8> && T > 0 && 2 * T <= G;
  const int bx = blockIdx.x;
  auto item = [&](int i, int& col0, int& width) -> bool {
    width = 16;
    if constexpr (!kSplitLastRound<FP8>) {
      const int b = bx + i * G;
      col0 = 16 * b;
      return b < nblk;
    }
    if (i < R) {
      col0 = 16 * (bx + i * G);
      width = 16;
      return true;
    }
    if (i > R || T == 0) return false;
    if (halves) {
      if (bx >= 2 * T) return false;
      col0 = 16 * (R * G + (bx >> 1)) + 8 * (bx & 1);
      width = 8;
      return col0 < p.N;
    }
    if (bx >= T) return false;
    col0 = 16 * (R * G + bx);
    width = 16;
    return true;
  };
  auto load_block = [&](int col0, int width, Frag (&bv)[KSM]) {
    const int c = lane & 15;
    int n = col0 + c;
    n = n < p.N ? n : p.N - 1;  // columns past N are computed but never stored
    const char* brow = static_cast<const char*>(p.B) + static_cast<int64_t>(n) * p.ldb * S::ES;
    const bool in = !kSplitLastRound<FP8> || c < width;
#pragma unroll
    for (int ks = 0; ks < KSM; ++ks) bv[ks] = ld(brow, kb + ks * S::KSTEP, in && ks < per);
  };

  Frag bv[NBUF][KSM];
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) {
    int c0, w0;
    if (item(u, c0, w0)) load_block(c0, w0, bv[u]);
  }

  for (int i0 = 0;; i0 += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int i = i0 + u;
      int col0, width;
      if (!item(i, col0, width)) return;
      int cn, wn;  // prefetch: NBUF - 1 items ahead
      if (item(i + NBUF - 1, cn, wn)) load_block(cn, wn, bv[(u + NBUF - 1) % NBUF]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSM; ++ks) {
        if constexpr (FP8)
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av[ks], bv[u][ks], acc, 0, 0, 0,
                                                                 127, 0, 127);
        else
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[ks]),
                                                        __builtin_bit_cast(bf16x8_t, bv[u][ks]),
                                                        acc, 0, 0, 0);
      }
      red[i & 1][wave][lane] = acc;
      __syncthreads();
      // Output (r, c) of the 16 x 16 block: MFMA lane 16 (r / 4) + c, element r % 4.
      if (tid < 256) {
        const int r = tid >> 4, c = tid & 15;
        const int n = col0 + c;
        if (r < p.M && (!kSplitLastRound<FP8> || c < width) && n < p.N) {
          const int src = 16 * (r >> 2) + c;
          float z = red[i & 1][0][src][r & 3];
#pragma unroll
          for (int w = 1; w < KW; ++w) z += red[i & 1][w][src][r & 3];
          if constexpr (S::ES == 1) z = z * (p.scale_a[r] * p.scale_b[n]);
          z = p.alpha * z;
          const int64_t off = static_cast<int64_t>(r) * p.ldc + n;
          if constexpr (OUT == OUT_F32 || OUT == OUT_BF16) {
            if (p.beta != 0.f) z += p.beta * load_cin1<OUT>(p.C, off);
          }
          if (p.bias) z += bf16_bits_to_f32(p.bias[n]);
          z = apply_act<OUT>(z, ACT);
          float qs, qz;
          out_row_params<OUT>(p, r, qs, qz);
          store_out1<OUT>(p.C, off, z, qs, qz);
        }
      }
    }
  }
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

// The streaming variant: 16 K-split waves, at most KSM k-steps each (K up to
// 4096 for both types), B prefetched NBUF - 1 blocks ahead. Measured at
// K = 4096 against the one-block-per-workgroup kernel above: FP8 M = 1,
// N = 18432 22.3 -> 18.8 us, M = 16 28.3 -> 20.1 us, BF16 M = 16 42.5 -> 35.5 us
// (M = 1 BF16 was already at ~5 TB/s: unchanged). Prefetching four FP8 blocks
// ahead instead of two needs more than the 128 VGPRs a 16-wave workgroup may
// use and spills (27 us).
template <bool FP8, int OUT>
static hipError_t launch_stream_out(const GemmArgs& a, hipStream_t stream) {
  constexpr int KW = 16, KSM = FP8 ? 2 : 8, NBUF = FP8 ? 3 : 2;
  const dim3 grid(static_cast<unsigned>(skinny_stream_grid(a.N))), block(KW * 64);
  if (a.act == ACT_NONE)
    hipLaunchKernelGGL((gemm_skinny_stream_kernel<FP8, KW, KSM, NBUF, OUT, ACT_NONE>), grid, block,
                       0, stream, a);
  else if (a.act == ACT_RELU)
    hipLaunchKernelGGL((gemm_skinny_stream_kernel<FP8, KW, KSM, NBUF, OUT, ACT_RELU>), grid, block,
                       0, stream, a);
  else if (a.act == ACT_GELU_ERF)
    hipLaunchKernelGGL((gemm_skinny_stream_kernel<FP8, KW, KSM, NBUF, OUT, ACT_GELU_ERF>), grid,
                       block, 0, stream, a);
  else
    hipLaunchKernelGGL((gemm_skinny_stream_kernel<FP8, KW, KSM, NBUF, OUT, ACT_GELU_TANH>), grid,
                       block, 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_stream(const GemmArgs& a, int out, hipStream_t stream) {
  if (out == OUT_BF16) return launch_stream_out<FP8, OUT_BF16>(a, stream);
  if (out == OUT_I8) return launch_stream_out<FP8, OUT_I8>(a, stream);
  if (out == OUT_E4M3) return launch_stream_out<FP8, OUT_E4M3>(a, stream);
  return launch_stream_out<FP8, OUT_F32>(a, stream);
}

hipError_t launch_skinny(const Plan& plan, const LaunchSpec& spec, const GemmArgs& a,
                         hipStream_t stream) {
  (void)plan;
  if (a.M > 16) return hipErrorInvalidValue;  // the plan only selects M <= 16
  if (skinny_streams(a.K))
    return spec.fp8 ? launch_stream<true>(a, spec.out, stream)
                    : launch_stream<false>(a, spec.out, stream);
  return spec.fp8 ? launch_mb<true, 1>(a, spec.out, stream)
                  : launch_mb<false, 1>(a, spec.out, stream);
}
#endif  // G355_KERNELS_ONLY

}  // namespace g355
