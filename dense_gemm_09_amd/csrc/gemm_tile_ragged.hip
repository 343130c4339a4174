// The tile kernels for K ranges that end inside a 16-byte chunk of a DMA-fed
// K-major row (RAGGED = true: the kernel writes that chunk of the last slice
// itself). A translation unit of its own, so that the two sets of
// instantiations compile in parallel.
#define G355_TILE_RAGGED 1
#include "gemm_tile.hip"
