// C ABI: argument validation, launch planning and dispatch.
//
// The interface follows the FP8 DeepGEMM page's (sec. 5.1): device pointers,
// sizes, scale vectors, an optional workspace with a separate size query, a
// stream, and a status code; all checks run before anything is enqueued. The
// runtime choice of tile and split from the shape is that page's sec. 5.3
// advice (tile and pipeline depth picked per shape) made concrete for
// 256 CUs.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gemm355.h"
#include "internal.hpp"

namespace g355 {
namespace {

constexpr int kCUs = 256;
constexpr int64_t kMaxDim = int64_t{1} << 30;

struct Candidate {
  int bm, bn, waves, occupancy;  // occupancy: workgroups per CU (LDS-limited)
  double efficiency[2];          // fraction of the CU's MFMA rate a full tile sustains: BF16, FP8
};

// 256x256: 128 KB LDS, one workgroup per CU. 256x128: 96 KB, one per CU.
// 128x128: 64 KB, two per CU.
// The efficiencies rank the candidates rather than predict time. For BF16 the
// 256x128 and 128x128 figures sit below 0.68 so that a 256x256 tile split two
// ways wins where it fills the chip (M = 2048, N = 4096, K = 14336: 247 us
// against 300 us for 256x128 tiles unsplit and 278 us for 128x128), and
// 128x128 ranks above 256x128 (two per CU: 512 x 12288 x 4096 80 us against
// 85 us, 256^3 8.6 us against 10.1 us). FP8's 128x128 tile keeps its matrix
// cores busier still: at 1024 x 4096 x 4096 it runs 35 us against 46 us for
// 256x128 tiles, and at 2048 x 4096 x 14336 131 us against 160 us.
constexpr Candidate kCandidates[] = {
    {256, 256, 8, 1, {0.85, 0.85}},
    {256, 128, 8, 1, {0.62, 0.65}},
    {128, 128, 4, 2, {0.67, 0.80}},
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Rows up to which the 64-row tile is used.
constexpr int64_t kThinMaxM = 64;

// Tile-kernel plan (any M): tile shape and split from the cost model.
static Plan make_tile_plan(int64_t M, int64_t N, int64_t K, bool fp8) {
  const int bke = fp8 ? 128 : 64;
  const double flops_per_clk = fp8 ? 8192.0 : 4096.0;  // per CU, dense
  const double clk = 2.4e9;
  const double hbm = 5.0e12;        // bytes/s assumed for split-K partial traffic
  const double reduce_launch = 4e-6;
  const int64_t kslices = std::max<int64_t>(1, ceil_div(K, bke));

  Plan best{};
  double best_t = 1e30;
  for (const Candidate& c : kCandidates) {
    const int64_t tiles = ceil_div(M, c.bm) * ceil_div(N, c.bn);
    for (int s = 1; s <= kMaxSplit; s *= 2) {
      if (s > 1 && (K == 0 || s > kslices)) break;
      const int64_t slices_per_split = ceil_div(kslices, s);
      const int64_t splits = ceil_div(kslices, slices_per_split);  // non-empty partitions
      if (splits != s) continue;
      const int64_t wgs = tiles * s;
      const int64_t slots = int64_t{kCUs} * c.occupancy;
      const double rounds = static_cast<double>(ceil_div(wgs, slots));
      const double tile_time = 2.0 * c.bm * c.bn * slices_per_split * bke /
                               (flops_per_clk * c.efficiency[fp8 ? 1 : 0] / c.occupancy) / clk;
      double t = rounds * tile_time;
      if (s > 1) t += 2.0 * s * static_cast<double>(M) * N * 4 / hbm + reduce_launch;
      if (t < best_t * 0.98) {
        best_t = t;
        best.kernel = KERNEL_TILE;
        best.bm = c.bm;
        best.bn = c.bn;
        best.bk = bke;
        best.waves = c.waves;
        best.split = s;
        best.k_split_len = static_cast<int>(slices_per_split * bke);
        best.grid = wgs;
        best.workspace = s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
      }
    }
  }
  if (K == 0) best.k_split_len = bke;
  // Few rows: 64-row tiles with deep rings. They stream B and are bound by
  // HBM, so the width (256 or 128 columns) and the K split are chosen from
  // bytes: B spread over the workgroups that run at once (one per CU), plus,
  // when split, the FP32 partial sums written and read back and the
  // reduction's launch.
  if (M <= kThinMaxM) {
    const double es = fp8 ? 1.0 : 2.0;
    const double b_time = static_cast<double>(N) * K * es / hbm;
    double thin_t = 1e30;
    for (const int bn : {256, 128}) {
      const int64_t tiles = ceil_div(N, bn);
      for (int64_t s = 1; s <= kMaxSplit; ++s) {
        if (s > 1 && (K == 0 || s > kslices)) break;
        const int64_t slices_per_split = ceil_div(kslices, s);
        if (ceil_div(kslices, slices_per_split) != s) continue;  // non-empty partitions
        const int64_t wgs = tiles * s;
        if (s > 1 && wgs > kCUs) break;
        const double fill = static_cast<double>(ceil_div(wgs, kCUs) * kCUs) / wgs;
        double t = b_time * fill;
        if (s > 1) t += 2.0 * s * static_cast<double>(M) * N * 4 / hbm + reduce_launch;
        if (t < thin_t * 0.98) {
          thin_t = t;
          best.kernel = KERNEL_TILE;
          best.bm = 64;
          best.bn = bn;
          best.bk = bke;
          best.waves = bn == 256 ? 4 : 2;
          best.split = static_cast<int>(s);
          best.k_split_len = static_cast<int>(slices_per_split * bke);
          best.grid = wgs;
          best.workspace = s > 1 ? static_cast<size_t>(s) * M * N * sizeof(float) : 0;
        }
      }
    }
  }
  return best;
}

// Decode-sized M (<= 16) with K-major, 16-byte aligned operands runs the
// skinny weight-streaming kernel (16 columns per workgroup, no workspace).
// The workspace reported is the tile plan's, which the call falls back to
// when the operands are not eligible.
constexpr int64_t kSkinnyMaxM = 16;

Plan make_plan(int64_t M, int64_t N, int64_t K, bool fp8) {
  Plan t = make_tile_plan(M, N, K, fp8);
  if (M > kSkinnyMaxM) return t;
  Plan s = t;
  s.kernel = KERNEL_SKINNY;
  s.bm = static_cast<int>(16 * ((M + 15) / 16));
  s.bn = 16;
  s.bk = fp8 ? 128 : 32;
  s.waves = 16;
  s.split = 1;
  s.k_split_len = static_cast<int>(K);
  s.grid = skinny_streams(K) ? skinny_stream_grid(N) : (N + 15) / 16;
  return s;
}

hipError_t launch_tile(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                       hipStream_t stream) {
  using Fn = hipError_t (*)(const Plan&, const LaunchSpec&, const GemmArgs&, hipStream_t);
  static constexpr Fn kParts[2][kOutParts] = {
      {launch_tile_r0_p0, launch_tile_r0_p1, launch_tile_r0_p2, launch_tile_r0_p3,
       launch_tile_r0_p4},
      {launch_tile_r1_p0, launch_tile_r1_p1, launch_tile_r1_p2, launch_tile_r1_p3,
       launch_tile_r1_p4}};
  const int part = plan.split > 1        ? PART_SPLIT
                   : spec.out == OUT_F32  ? PART_F32
                   : spec.out == OUT_BF16 ? PART_BF16
                   : spec.out == OUT_I8   ? PART_I8
                                          : PART_E4M3;
  return kParts[spec.ragged ? 1 : 0][part](plan, spec, args, stream);
}

}  // namespace g355

using namespace g355;

namespace {

bool valid_layout(int l) { return l == GEMM_ROW_MAJOR || l == GEMM_COL_MAJOR; }
bool valid_out(int d) { return d == GEMM_OUT_F32 || d == GEMM_OUT_BF16; }
bool valid_act(int a) { return a >= GEMM_ACT_NONE && a <= GEMM_ACT_GELU_TANH; }
bool valid_qout(int q) { return q == GEMM_QOUT_INT8 || q == GEMM_QOUT_E4M3; }
int qout_kind(int q) { return q == GEMM_QOUT_INT8 ? OUT_I8 : OUT_E4M3; }

// E8M0 block scales of an MX FP8 call: one byte per 32 K elements, rows of ld bytes.
struct MxScales {
  const void* a;
  int64_t lda;
  const void* b;
  int64_t ldb;
};

// out_kind: OutKind. The quantised kinds (INT8, E4M3) come with beta == 0,
// the per-row output scale qscale and, for INT8 only, an optional zero point.
// mx: block scales of an MX call (fp8 true, scale_a / scale_b unused), or null.
gemm_status run(bool fp8, int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                int64_t lda, int layout_a, const void* B, int64_t ldb, int layout_b,
                const float* scale_a, const float* scale_b, float beta, void* C, int64_t ldc,
                int out_kind, const float* qscale, const int32_t* qzero, const void* bias,
                int act, void* workspace, size_t workspace_bytes, void* stream,
                const MxScales* mx = nullptr) {
  // ---- enums and sizes
  if (!valid_layout(layout_a) || !valid_layout(layout_b) || !valid_act(act))
    return GEMM_ERR_BAD_ENUM;
  const bool quant_out = out_kind == OUT_I8 || out_kind == OUT_E4M3;
  if (out_kind == OUT_E4M3 && qzero != nullptr) return GEMM_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return GEMM_ERR_BAD_DIM;
  if (fp8 && (layout_a != GEMM_ROW_MAJOR || layout_b != GEMM_COL_MAJOR))
    return GEMM_ERR_UNSUPPORTED;
  // ---- leading dimensions
  const int64_t need_lda = layout_a == GEMM_ROW_MAJOR ? K : M;
  const int64_t need_ldb = layout_b == GEMM_ROW_MAJOR ? N : K;
  if (lda < std::max<int64_t>(1, need_lda) || ldb < std::max<int64_t>(1, need_ldb) ||
      ldc < std::max<int64_t>(1, N))
    return GEMM_ERR_BAD_LD;
  if (mx) {
    // A row of scales is read one 4-byte word (four blocks) per 128-element
    // K slice: at least ceil(K/32) bytes, a multiple of 4.
    const int64_t nblk = std::max<int64_t>(4, (K + 31) / 32);
    if (mx->lda < nblk || mx->ldb < nblk || mx->lda % 4 != 0 || mx->ldb % 4 != 0)
      return GEMM_ERR_BAD_LD;
    // 32-bit byte offsets into the scale arrays, rows of a partial tile included.
    if ((M + 256) * mx->lda >= (int64_t{1} << 31) || (N + 256) * mx->ldb >= (int64_t{1} << 31))
      return GEMM_ERR_BAD_DIM;
  }
  if (M == 0 || N == 0) return GEMM_OK;
  // ---- pointers
  if (C == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL_POINTER;
  if (fp8 && !mx && (scale_a == nullptr || scale_b == nullptr)) return GEMM_ERR_NULL_POINTER;
  if (mx && K > 0) {
    if (mx->a == nullptr || mx->b == nullptr) return GEMM_ERR_NULL_POINTER;
    if ((reinterpret_cast<uintptr_t>(mx->a) & 3u) || (reinterpret_cast<uintptr_t>(mx->b) & 3u))
      return GEMM_ERR_UNSUPPORTED;
  }
  if (quant_out && qscale == nullptr) return GEMM_ERR_NULL_POINTER;

  const Plan plan = make_plan(M, N, K, fp8);
  // Every tile size in use is >= 128, so this bounds the grid of any variant.
  if (((M + 127) / 128) * ((N + 127) / 128) * plan.split > INT32_MAX) return GEMM_ERR_BAD_DIM;
  if (plan.workspace > 0) {
    if (workspace == nullptr) return GEMM_ERR_NULL_POINTER;
    if (workspace_bytes < plan.workspace) return GEMM_ERR_WORKSPACE_TOO_SMALL;
  }

  // ---- how each operand reaches LDS
  const int ce = fp8 ? 16 : 8;  // elements per 16-byte chunk
  auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  LaunchSpec spec{};
  spec.fp8 = fp8;
  spec.a_kmajor = layout_a == GEMM_ROW_MAJOR;
  spec.b_kmajor = layout_b == GEMM_COL_MAJOR;
  spec.out = out_kind;
  spec.mx = mx != nullptr;
  const bool k_ok = K % ce == 0;
  // The DMA loader addresses an operand with 32-bit byte offsets from its base
  // and marks chunks past K with an offset just beyond the operand's extent:
  // the extent must stay under 2 GiB. K need not be a multiple of the 16-byte
  // chunk (the kernel writes each row's last, partial chunk itself), and rows
  // need not be 16-byte aligned: the buffer loads take any byte offset (BF16
  // elements must still be 2-byte aligned).
  const int64_t es = fp8 ? 1 : 2;
  const auto under2g = [&](int64_t rows, int64_t ld) {
    return ((rows - 1) * ld + K) * es < (int64_t{1} << 31);
  };
  const auto rows16 = [&](const void* p, int64_t ld) { return aligned16(p) && ld % ce == 0; };
  const auto dma_ok = [&](bool kmajor, const void* p, int64_t ld, int64_t rows) {
    const bool even = (reinterpret_cast<uintptr_t>(p) & 1u) == 0;
    return kmajor && under2g(rows, ld) && (fp8 || even);
  };
  spec.loader_a = dma_ok(spec.a_kmajor, A, lda, M) ? LOAD_DIRECT : LOAD_GENERIC;
  spec.loader_b = dma_ok(spec.b_kmajor, B, ldb, N) ? LOAD_DIRECT : LOAD_GENERIC;
  // BF16 B stored N-contiguous: DMA into an N-major tile (transposing reads)
  // when its rows are 16-byte aligned, N is a multiple of 8 and A is DMA-fed.
  if (!fp8 && !spec.b_kmajor && spec.loader_a == LOAD_DIRECT && ldb % 8 == 0 && N % 8 == 0 &&
      aligned16(B) && ((K - 1) * ldb + N) * es < (int64_t{1} << 31))
    spec.loader_b = LOAD_DIRECT_N;
  if (K == 0) spec.loader_a = spec.loader_b = LOAD_DIRECT;  // nothing is loaded

  const bool direct = spec.loader_a == LOAD_DIRECT &&
                      (spec.loader_b == LOAD_DIRECT || spec.loader_b == LOAD_DIRECT_N);
  // MX runs on the DMA-fed tile kernel only (no skinny kernel).
  if (mx && !direct) return GEMM_ERR_UNSUPPORTED;
  // K ends inside a 16-byte chunk of a DMA-fed K-major row: the tile kernels
  // that write that chunk themselves. (FP8 with one operand not DMA-fed reads
  // both through registers.)
  spec.ragged = !k_ok && (direct || (!fp8 && (spec.loader_a == LOAD_DIRECT ||
                                              spec.loader_b == LOAD_DIRECT)));
  // The skinny kernel reads K-major operands with 16-byte aligned rows and K a
  // multiple of the chunk only.
  const bool skinny_ok = direct && !mx && spec.loader_b == LOAD_DIRECT && k_ok &&
                         rows16(A, lda) && rows16(B, ldb);
  Plan p = (plan.kernel == KERNEL_SKINNY && !skinny_ok) ? make_tile_plan(M, N, K, fp8) : plan;
  if (p.kernel == KERNEL_TILE && !direct) {
    p.bm = 128;
    p.bn = 128;
    p.waves = 4;
  }
  GemmArgs a{};
  a.A = A;
  a.B = B;
  a.C = C;
  a.bias = static_cast<const uint16_t*>(bias);
  a.scale_a = scale_a;
  a.scale_b = scale_b;
  a.workspace = static_cast<float*>(workspace);
  a.qscale = quant_out ? qscale : nullptr;
  a.qzero = out_kind == OUT_I8 ? qzero : nullptr;
  if (mx) {
    a.mx_a = static_cast<const uint8_t*>(mx->a);
    a.mx_b = static_cast<const uint8_t*>(mx->b);
    a.ldsa = static_cast<int>(mx->lda);
    a.ldsb = static_cast<int>(mx->ldb);
  }
  a.lda = lda;
  a.ldb = ldb;
  a.ldc = ldc;
  a.M = static_cast<int>(M);
  a.N = static_cast<int>(N);
  a.K = static_cast<int>(K);
  a.alpha = alpha;
  a.beta = quant_out ? 0.f : beta;
  a.act = act;
  {
    const uintptr_t cbase = reinterpret_cast<uintptr_t>(C);
    // Bytes of one 4-element store: FP32 16, BF16 8, quantised 4.
    const uintptr_t need = out_kind == OUT_F32 ? 16u : out_kind == OUT_BF16 ? 8u : 4u;
    a.c_vec = (cbase % need == 0 && ldc % 4 == 0) ? 1 : 0;
  }
  a.split_k = p.split;
  a.k_split_len = p.k_split_len;
  a.tiles_m = static_cast<int>((M + p.bm - 1) / p.bm);
  a.tiles_n = static_cast<int>((N + p.bn - 1) / p.bn);
  a.ws_vec = (reinterpret_cast<uintptr_t>(workspace) & 15u) == 0 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // hipGetLastError after a launch also returns an error that an earlier,
  // unrelated HIP call on this thread left pending: consume any such error
  // first, so that GEMM_ERR_HIP reports this call's own launches only.
  (void)hipGetLastError();
  if (p.kernel == KERNEL_SKINNY) {
    a.a_mn_major = a.b_mn_major = 0;
    return launch_skinny(p, spec, a, s) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
  }
  p.grid = static_cast<int64_t>(a.tiles_m) * a.tiles_n * p.split;
  if (launch_tile(p, spec, a, s) != hipSuccess) return GEMM_ERR_HIP;
  if (p.split > 1 && launch_splitk_reduce(p, spec, a, s) != hipSuccess) return GEMM_ERR_HIP;
  return GEMM_OK;
}

// ---- scratch of the entry point that allocates nothing (gemm_bf16_noalloc)
//
// A file-scope device array: every GPU the library runs on holds one copy of
// it from the module load until the process ends. In host code the name
// `scratch` is only a host-side stand-in for the array, not a device
// address, so it is never passed to a kernel or a copy: the device address of
// each GPU's copy is taken once per device with hipGetSymbolAddress (with
// that device current) and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on the first call on that
// device).
gemm_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GEMM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

}  // namespace

extern "C" {

gemm_status gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                      gemm_layout layout_a, const void* B, int64_t ldb, gemm_layout layout_b,
                      float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype, const void* bias,
                      gemm_act act, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_out(c_dtype)) return GEMM_ERR_BAD_ENUM;
  return run(false, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, nullptr, nullptr, beta,
             C, ldc, c_dtype, nullptr, nullptr, bias, act, workspace, workspace_bytes, stream);
}

gemm_status gemm_bf16_noalloc(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                              int64_t lda, gemm_layout layout_a, const void* B, int64_t ldb,
                              gemm_layout layout_b, float beta, void* C, int64_t ldc,
                              gemm_out_dtype c_dtype, const void* bias, gemm_act act,
                              void* stream) {
  if (!valid_out(c_dtype)) return GEMM_ERR_BAD_ENUM;
  // The split-K partials go to this device's scratch array: no allocation.
  // The partials are written in full before they are read (nothing needs to
  // start at zero); calls that overlap on one GPU share the array and race.
  size_t need = 0;
  if (M > 0 && N > 0 && K >= 0 && M <= kMaxDim && N <= kMaxDim && K <= kMaxDim)
    need = make_plan(M, N, K, false).workspace;
  if (need > kNoAllocScratchBytes) return GEMM_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need > 0) {
    const gemm_status st = scratch_of_current_device(&ws);
    if (st != GEMM_OK) return st;
  }
  return run(false, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, nullptr, nullptr, beta,
             C, ldc, c_dtype, nullptr, nullptr, bias, act, ws, ws ? kNoAllocScratchBytes : 0,
             stream);
}

gemm_status gemm_fp8_scaled(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                            int64_t lda, gemm_layout layout_a, const void* B, int64_t ldb,
                            gemm_layout layout_b, const float* scale_a, const float* scale_b,
                            float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype,
                            const void* bias, gemm_act act, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!valid_out(c_dtype)) return GEMM_ERR_BAD_ENUM;
  return run(true, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, scale_a, scale_b, beta,
             C, ldc, c_dtype, nullptr, nullptr, bias, act, workspace, workspace_bytes, stream);
}

gemm_status gemm_mxfp8(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       gemm_layout layout_a, const void* B, int64_t ldb, gemm_layout layout_b,
                       const void* scale_a, int64_t ldsa, const void* scale_b, int64_t ldsb,
                       float beta, void* C, int64_t ldc, gemm_out_dtype c_dtype, const void* bias,
                       gemm_act act, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_out(c_dtype)) return GEMM_ERR_BAD_ENUM;
  const MxScales mx{scale_a, ldsa, scale_b, ldsb};
  return run(true, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, nullptr, nullptr, beta, C,
             ldc, c_dtype, nullptr, nullptr, bias, act, workspace, workspace_bytes, stream, &mx);
}

gemm_status gemm_bf16_quant(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                            int64_t lda, gemm_layout layout_a, const void* B, int64_t ldb,
                            gemm_layout layout_b, const void* bias, gemm_act act,
                            const float* out_scale, const int32_t* out_zero, void* Q,
                            int64_t ldq, gemm_qout_dtype q_dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!valid_qout(q_dtype)) return GEMM_ERR_BAD_ENUM;
  return run(false, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, nullptr, nullptr, 0.f,
             Q, ldq, qout_kind(q_dtype), out_scale, out_zero, bias, act, workspace,
             workspace_bytes, stream);
}

gemm_status gemm_fp8_scaled_quant(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                                  int64_t lda, gemm_layout layout_a, const void* B, int64_t ldb,
                                  gemm_layout layout_b, const float* scale_a,
                                  const float* scale_b, const void* bias, gemm_act act,
                                  const float* out_scale, const int32_t* out_zero, void* Q,
                                  int64_t ldq, gemm_qout_dtype q_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!valid_qout(q_dtype)) return GEMM_ERR_BAD_ENUM;
  return run(true, M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, scale_a, scale_b, 0.f,
             Q, ldq, qout_kind(q_dtype), out_scale, out_zero, bias, act, workspace,
             workspace_bytes, stream);
}

gemm_status gemm_quantize_fp8_rows(int64_t M, int64_t K, const void* X, int64_t ldx, void* Q,
                                   int64_t ldq, float* scale, void* stream) {
  if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return GEMM_ERR_BAD_DIM;
  if (ldx < std::max<int64_t>(1, K) || ldq < std::max<int64_t>(1, K)) return GEMM_ERR_BAD_LD;
  if (M == 0) return GEMM_OK;
  if (scale == nullptr) return GEMM_ERR_NULL_POINTER;
  if (K > 0 && (X == nullptr || Q == nullptr)) return GEMM_ERR_NULL_POINTER;
  const auto aligned = [](const void* p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
  };
  const bool vec = K % 8 == 0 && ldx % 8 == 0 && ldq % 8 == 0 && aligned(X, 16) && aligned(Q, 8);
  return launch_quantize_rows(M, K, X, ldx, Q, ldq, scale, vec,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status gemm_pack_b(int64_t K, int64_t N, const void* B, int64_t ldb, gemm_layout layout_b,
                        int elem_bytes, void* Bp, int64_t ldbp, void* stream) {
  if (!valid_layout(layout_b) || (elem_bytes != 1 && elem_bytes != 2)) return GEMM_ERR_BAD_ENUM;
  if (K < 0 || N < 0 || K > kMaxDim || N > kMaxDim) return GEMM_ERR_BAD_DIM;
  const bool rowmajor = layout_b == GEMM_ROW_MAJOR;
  if (ldb < std::max<int64_t>(1, rowmajor ? N : K) || ldbp < std::max<int64_t>(1, K))
    return GEMM_ERR_BAD_LD;
  if (K == 0 || N == 0) return GEMM_OK;
  if (B == nullptr || Bp == nullptr) return GEMM_ERR_NULL_POINTER;
  if (rowmajor && ((K + 63) / 64) * ((N + 63) / 64) > INT32_MAX) return GEMM_ERR_BAD_DIM;
  return launch_pack_b(K, N, B, ldb, rowmajor, elem_bytes, Bp, ldbp,
                       static_cast<hipStream_t>(stream)) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int is_fp8) {
  if (M <= 0 || N <= 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  return make_plan(M, N, K, is_fp8 != 0).workspace;
}

gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, int is_fp8, gemm_plan_info* out) {
  if (out == nullptr) return GEMM_ERR_NULL_POINTER;
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return GEMM_ERR_BAD_DIM;
  const Plan p = make_plan(std::max<int64_t>(M, 1), std::max<int64_t>(N, 1), K, is_fp8 != 0);
  out->kernel = p.kernel;
  out->tile_m = p.bm;
  out->tile_n = p.bn;
  out->tile_k = p.bk;
  out->split_k = p.split;
  out->waves = p.waves;
  out->grid = (M == 0 || N == 0) ? 0 : p.grid;
  out->workspace_bytes = (M == 0 || N == 0) ? 0 : p.workspace;
  return GEMM_OK;
}

const char* gemm_status_string(gemm_status s) {
  switch (s) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_NULL_POINTER: return "GEMM_ERR_NULL_POINTER";
    case GEMM_ERR_BAD_DIM: return "GEMM_ERR_BAD_DIM";
    case GEMM_ERR_BAD_LD: return "GEMM_ERR_BAD_LD";
    case GEMM_ERR_BAD_ENUM: return "GEMM_ERR_BAD_ENUM";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_WORKSPACE_TOO_SMALL: return "GEMM_ERR_WORKSPACE_TOO_SMALL";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP";
  }
  return "GEMM_ERR_UNKNOWN";
}

}  // extern "C"
