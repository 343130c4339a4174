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

// The tile kernels are instantiated per output part, each in a compile of
// its own (gemm_tile.hip built with G355_PART and G355_RAGGED).
enum OutPart : int { PART_SPLIT = 0, PART_F32 = 1, PART_BF16 = 2, PART_I8 = 3, PART_E4M3 = 4 };
constexpr int kOutParts = 5;

#define G355_PART_LAUNCHER_(r, p) launch_tile_r##r##_p##p
#define G355_PART_LAUNCHER(r, p) G355_PART_LAUNCHER_(r, p)
#define G355_DECLARE_PART(r, p)                                                              \
  hipError_t G355_PART_LAUNCHER(r, p)(const Plan& plan, const LaunchSpec& spec,              \
                                      const GemmArgs& args, hipStream_t stream);
G355_DECLARE_PART(0, 0) G355_DECLARE_PART(0, 1) G355_DECLARE_PART(0, 2) G355_DECLARE_PART(0, 3)
G355_DECLARE_PART(0, 4) G355_DECLARE_PART(1, 0) G355_DECLARE_PART(1, 1) G355_DECLARE_PART(1, 2)
G355_DECLARE_PART(1, 3) G355_DECLARE_PART(1, 4)
#undef G355_DECLARE_PART

// Enqueue the tile kernel of a plan (the part launcher for its output kind
// and ragged flag). Returns the HIP error of the launch.
hipError_t launch_tile(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                       hipStream_t stream);
hipError_t launch_skinny(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                         hipStream_t stream);
// The skinny kernel's streaming variant covers K up to 16 waves x 4096/16
// elements; its grid is one workgroup per CU at most.
inline bool skinny_streams(int64_t K) { return K <= 4096; }
inline int64_t skinny_stream_grid(int64_t N) {
  const int64_t blocks = (N + 15) / 16;
  return blocks < 256 ? blocks : 256;
}
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
