// One-time reorder of a weight matrix into the layout the fast path reads.
//
// The FP8 DeepGEMM page (sec. 3.2) describes rearranging B once, before the
// GEMMs that reuse it, into the form the matrix-core loads want, so that the
// cost is paid once per weight instead of once per call. On gfx950 that form is
// K-major rows (b(k, n) at Bp[n * ldbp + k]) whose starts are 16-byte aligned:
// such operands are copied global -> LDS by DMA, and the LDS swizzle is applied
// by the choice of source address during that copy, so nothing beyond the
// K-major layout needs to be precomputed in memory. A B stored row-major
// (N contiguous) or with an unaligned leading dimension is otherwise read by
// the register loader, which is several times slower.
//
// N-contiguous input: 64 x 64 element tiles through LDS (coalesced reads along
// n, coalesced writes along k). K-contiguous input: a row copy to the new
// leading dimension. Elements of 1 (E4M3) or 2 (BF16) bytes; moved as bits.

#include "common.hpp"
#include "internal.hpp"

namespace g355 {

constexpr int kPackTile = 64;
constexpr int kPackThreads = 256;

template <typename T>
__global__ void __launch_bounds__(kPackThreads)
pack_transpose_kernel(const T* __restrict__ B, int64_t ldb, T* __restrict__ Bp, int64_t ldbp,
                      int K, int N) {
  // +1 element per LDS row: column reads of the tile hit distinct banks more often.
  __shared__ T tile[kPackTile][kPackTile + 1];
  // One workgroup per 64 x 64 tile, numbered along n first (a 1-D grid: the
  // second grid dimension is limited to 65536).
  const int tiles_n = (N + kPackTile - 1) / kPackTile;
  const int64_t b = blockIdx.x;
  const int k0 = static_cast<int>(b / tiles_n) * kPackTile;
  const int n0 = static_cast<int>(b % tiles_n) * kPackTile;
  const int tx = threadIdx.x % kPackTile, ty = threadIdx.x / kPackTile;  // 64 x 4 threads
  // read rows k of B (n contiguous)
  for (int r = ty; r < kPackTile; r += kPackThreads / kPackTile) {
    const int k = k0 + r, n = n0 + tx;
    if (k < K && n < N) tile[r][tx] = B[static_cast<int64_t>(k) * ldb + n];
  }
  __syncthreads();
  // write rows n of Bp (k contiguous)
  for (int r = ty; r < kPackTile; r += kPackThreads / kPackTile) {
    const int n = n0 + r, k = k0 + tx;
    if (k < K && n < N) Bp[static_cast<int64_t>(n) * ldbp + k] = tile[tx][r];
  }
}

template <typename T>
__global__ void __launch_bounds__(kPackThreads)
pack_rows_kernel(const T* __restrict__ B, int64_t ldb, T* __restrict__ Bp, int64_t ldbp, int K,
                 int N) {
  const int n = blockIdx.x;  // one workgroup per row
  for (int k = threadIdx.x; k < K; k += kPackThreads)
    Bp[static_cast<int64_t>(n) * ldbp + k] = B[static_cast<int64_t>(n) * ldb + k];
}

hipError_t launch_pack_b(int64_t K, int64_t N, const void* B, int64_t ldb, bool b_rowmajor,
                         int elem_bytes, void* Bp, int64_t ldbp, hipStream_t stream) {
  const dim3 block(kPackThreads);
  if (b_rowmajor) {
    const dim3 grid(static_cast<unsigned>(((N + kPackTile - 1) / kPackTile) *
                                          ((K + kPackTile - 1) / kPackTile)));
    if (elem_bytes == 2)
      hipLaunchKernelGGL(pack_transpose_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(B), ldb, static_cast<uint16_t*>(Bp), ldbp,
                         static_cast<int>(K), static_cast<int>(N));
    else
      hipLaunchKernelGGL(pack_transpose_kernel<uint8_t>, grid, block, 0, stream,
                         static_cast<const uint8_t*>(B), ldb, static_cast<uint8_t*>(Bp), ldbp,
                         static_cast<int>(K), static_cast<int>(N));
  } else {
    const dim3 grid(static_cast<unsigned>(N));
    if (elem_bytes == 2)
      hipLaunchKernelGGL(pack_rows_kernel<uint16_t>, grid, block, 0, stream,
                         static_cast<const uint16_t*>(B), ldb, static_cast<uint16_t*>(Bp), ldbp,
                         static_cast<int>(K), static_cast<int>(N));
    else
      hipLaunchKernelGGL(pack_rows_kernel<uint8_t>, grid, block, 0, stream,
                         static_cast<const uint8_t*>(B), ldb, static_cast<uint8_t*>(Bp), ldbp,
                         static_cast<int>(K), static_cast<int>(N));
  }
  return hipGetLastError();
}

}  // namespace g355
