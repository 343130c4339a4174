// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace g355 {

// How an operand's K slices reach LDS.
enum Loader : int {
  LOAD_DIRECT = 0,   // K-major, 16-byte aligned rows: global -> LDS DMA, no registers
  LOAD_GENERIC = 1,  // any layout / alignment: element loads through registers
  LOAD_DIRECT_N = 2, // B only, BF16 N-contiguous (row-major), 16-byte aligned rows, N % 8 == 0:
                     // DMA into an N-major LDS tile, fragments by transposing LDS reads
};

enum KernelKind : int { KERNEL_TILE = 0, KERNEL_SKINNY = 1 };

struct Plan {
  int kernel;        // KernelKind
  int bm, bn, bk;    // tile (bk in elements)
  int waves;         // waves per workgroup
  int split;         // K partitions
  int k_split_len;   // K elements per partition
  int64_t grid;      // workgroups of the main kernel
  size_t workspace;  // bytes
};

// Chooses the kernel, tile and split for a shape (host arithmetic only).
Plan make_plan(int64_t M, int64_t N, int64_t K, bool fp8);

// Largest K split a plan uses (the reduction kernel holds that many partials
// per thread).
constexpr int kMaxSplit = 16;

struct LaunchSpec {
  bool fp8;
  int loader_a, loader_b;  // Loader
  bool a_kmajor, b_kmajor; // layout of each operand (true = K contiguous)
  int out;                 // OutKind
  bool mx;                 // FP8 with E8M0 block scales (GemmArgs::mx_a / mx_b)
  bool ragged;             // K not a multiple of the 16-byte chunk, a K-major operand DMA-fed
};

// Enqueue the kernels of a plan. Returns the HIP error of the launch(es).
hipError_t launch_tile(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                       hipStream_t stream);
// The same, for spec.ragged (instantiated in a translation unit of its own).
hipError_t launch_tile_ragged(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                              hipStream_t stream);
hipError_t launch_skinny(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                         hipStream_t stream);
hipError_t launch_splitk_reduce(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                                hipStream_t stream);

// Per-token FP8 quantisation of BF16 rows (quant.hip). vec: 16-byte aligned
// rows with K and ldx multiples of 8 and Q rows 8-byte aligned.
hipError_t launch_quantize_rows(int64_t M, int64_t K, const void* X, int64_t ldx, void* Q,
                                int64_t ldq, float* scale, bool vec, hipStream_t stream);

// One-time reorder of B (K x N, elements of elem_bytes) into K-major rows of
// ldbp elements (pack.hip). b_rowmajor: B is N-contiguous (b(k,n) = B[k*ldb+n]).
hipError_t launch_pack_b(int64_t K, int64_t N, const void* B, int64_t ldb, bool b_rowmajor,
                         int elem_bytes, void* Bp, int64_t ldbp, hipStream_t stream);

}  // namespace g355
