// Tiled MFMA GEMM for gfx950: BF16 x BF16 and FP8-E4M3 x FP8-E4M3, FP32 accumulate.
//
// The three-level tiling of the first DeepGEMM page (sec. 2.1: an output tile
// per workgroup, K slices staged in on-chip memory, a register tile per wave),
// its software pipeline (sec. 3.3: copies of later slices overlap the
// matrix-core work on the current one; a barrier separates a buffer's last
// read from its next overwrite, sec. 4.3), its XOR swizzle of the staged
// tiles (sec. 3.2) and the zero contribution of out-of-range K (sec. 4.3),
// laid out for CDNA4:
//
// * A K slice is ROWB bytes (64 or 128) of every tile row: 32 or 64 BF16, or
//   64 or 128 FP8 elements, i.e. CPR = ROWB/16 chunks of 16 bytes. Operand
//   tiles live in LDS as rows of ROWB bytes with chunk c of row r at physical
//   chunk c ^ swz(r). The MFMA fragment reads (ds_read_b128; lanes 0..31 on 32
//   consecutive rows, one chunk each) then hit distinct 16-byte slots within
//   every 8 and every 16 consecutive lanes, so they are conflict-free whether
//   the LDS serves 128 or 256 bytes of a 128-bit read per cycle.
// * STAGES slices are in flight in a ring of LDS buffers. K-major operands
//   (any row alignment) are copied global -> LDS by buffer_load_dwordx4 ... lds
//   (64 lanes x 16 B into one contiguous 1 KB segment per instruction). The
//   lane that lands on physical chunk p of row r fetches logical chunk
//   p ^ swz(r), so the swizzle costs nothing and no VGPRs hold staged data.
//   Chunks that do not end before the end of K read zeros through the buffer
//   range check; a chunk that straddles it is written by patch_tail; rows
//   past M (or N) read a clamped valid row whose results are never stored.
//   Every iteration issues the same number of DMA instructions (slices past
//   the end read zeros), so waiting for the oldest slice is a fixed vmcnt.
// * A BF16 B stored N-contiguous is copied the same way into an N-major tile
//   (NmajorLoader). Other operands (A column-major, an E4M3 B row-major,
//   operands of 2 GiB or more) are loaded element-wise into registers and
//   written to the same swizzled layout after the slice's MFMAs.
// * BF16 uses v_mfma_f32_32x32x16_bf16; FP8 uses v_mfma_scale_f32_32x32x64_f8f6f4
//   with the E4M3 format code and the neutral block scale 2^0 (E8M0 code 127).
//   The per-token / per-channel scales are FP32 and applied in the epilogue.
//   A and B fragments put the same K indices in the same register slots, so the
//   result does not depend on how the hardware orders K inside one MFMA.

#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace g355 {

// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format,
// no swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// Physical chunk offset of row r for CPR chunks per row (see file comment).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

template <int BM_, int BN_, int WM_, int WN_, bool FP8_, int ROWB_, int STAGES_, int SPREAD_ = 1,
          bool MX_ = false>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, ROWB = ROWB_, STAGES = STAGES_;
  // K-steps over which the global->LDS loads of one slice are issued.
  static constexpr int SPREAD = SPREAD_;
  static constexpr bool FP8 = FP8_;
  // MX: FP8 with one E8M0 scale per 32 K elements of each row of A and column
  // of B, applied by the MFMA itself (no FP32 per-row / per-column scales).
  static constexpr bool MX = MX_;
  static_assert(!MX || (FP8 && ROWB == 128), "MX scales: FP8 with four 32-element blocks per slice");
  static constexpr int NWAVES = WM * WN;
  static constexpr int NT = NWAVES * 64;
  static constexpr int ES = FP8 ? 1 : 2;      // bytes per element
  static constexpr int CPR = ROWB / 16;       // 16-byte chunks per row
  static constexpr int BKE = ROWB / ES;       // K elements per slice
  static constexpr int CE = 16 / ES;          // K elements per chunk
  static constexpr int RPS = 1024 / ROWB;     // rows per 1 KB DMA segment
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BN * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int WTM = BM / WM;         // wave tile
  static constexpr int WTN = BN / WN;
  static constexpr int FM = WTM / 32;         // 32x32 MFMA blocks per wave
  static constexpr int FN = WTN / 32;
  // MFMA k-steps per slice: BF16 32x32x16 eats 32 B of a row, FP8 32x32x64 64 B.
  static constexpr int KSTEPS = FP8 ? ROWB / 64 : ROWB / 32;
  static_assert(ROWB == 64 || ROWB == 128, "row bytes");
  static_assert(KSTEPS >= 1, "k steps");
  static_assert((BM / RPS) % NWAVES == 0 && (BN / RPS) % NWAVES == 0, "DMA segments per wave");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(STAGES >= 2 && STAGES * STAGE <= 160 * 1024, "LDS budget");
  static_assert(SPREAD >= 1 && SPREAD <= KSTEPS, "load spread");
};

// ------------------------------------------------------------------ DMA loader

// Cache-policy operand of the buffer loads: bit 1 marks an access
// non-temporal on gfx950.
constexpr int kPolicyNonTemporal = 2;

// POL: cache policy of the copies (0, or kPolicyNonTemporal for an operand
// that is read once).
template <class C, int ROWS, int NW = C::NWAVES, int POL = 0>
struct DirectLoader {
  // NW waves issue the loads of a tile; each issues IPW 1 KB segments per slice.
  static constexpr int IPW = ROWS / C::RPS / NW;
  // Byte offset of this lane's chunk (row start + chunk, k excluded) from the
  // operand base. Offsets are 32-bit (operands under 2 GiB, checked on the
  // host), so a load is one VGPR plus the slice's wave-uniform offset (an
  // SGPR): the per-slice advance is a scalar add. Rows need not be 16-byte
  // aligned (BF16 rows at any 2-byte alignment: buffer loads take unaligned
  // addresses).
  uint32_t off[IPW];
  // One past the last K element of the lane's chunk (slice-relative) in
  // segments of even and of odd index: a segment holds RPS consecutive rows
  // starting at a multiple of RPS, so the swizzle of a lane's row depends on
  // the segment only through its parity.
  int kce2[2];

  __device__ __forceinline__ void init(int64_t ld, int row0, int rows, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int s = wave * IPW + i;
      const int r = C::RPS * s + lane / C::CPR;
      const int c = (lane % C::CPR) ^ swz<C::CPR>(r);
      int g = row0 + r;
      g = g < rows ? g : rows - 1;
      off[i] = static_cast<uint32_t>(static_cast<int64_t>(g) * ld * C::ES) + c * 16;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = C::RPS * q + lane / C::CPR;
      kce2[q] = ((lane % C::CPR) ^ swz<C::CPR>(r)) * C::CE + C::CE;
    }
  }

  // Loads of a slice as buffer loads: the operand's descriptor (whose range
  // is the operand's extent), this lane's 32-bit offset and the slice's
  // wave-uniform byte offset koff = k0 * ES. Only chunks that end at or before
  // k_end are copied; the others use the offset `oob` (the extent), which the
  // buffer's range check turns into zeros without a memory access. (The range
  // check sees the per-lane offset only, not koff, so a chunk that straddles
  // k_end is never copied: on the operand's last row its bytes past K may lie
  // past the allocation. Such chunks are written by patch_tail.)
  // full: every chunk of the slice ends at or before k_end.
  template <int I0 = 0, int I1 = IPW>
  __device__ __forceinline__ void issue_buf(char* lds_tile, int wave, __amdgpu_buffer_rsrc_t rsrc,
                                            int koff, uint32_t oob, int k0, int k_end,
                                            bool full) const {
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int s = wave * IPW + i;
      const uint32_t vo = (full || k0 + kce2[s & 1] <= k_end) ? off[i] : oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (G355_LDS void*)(lds_tile + s * 1024), 16,
                                               static_cast<int>(vo), koff, 0, POL);
    }
  }
};

// ------------------------------------------------ DMA loader, N-contiguous B

// B stored N-contiguous (BF16, row-major K x N): a slice's BKE rows of k are
// copied as they lie in memory into an N-major LDS tile (one row of BN*2
// bytes per k), 16-byte chunk c of row k at physical chunk c ^ (4 * (k % 4)):
// a transposing fragment read (ds_read_b64_tr_b16) takes four consecutive k
// rows at once, and the XOR puts those rows on different banks. As with the
// K-major loader the swizzle is applied by the source address each DMA lane
// fetches. Every byte offset is in the per-lane offset (row * ldb * 2 +
// column * 2, the slice's k0 * ldb * 2 added per slice), so the buffer range
// check turns rows past the last k and chunks past the array into zeros;
// chunks at or past N (N is a multiple of 8) get the out-of-range offset.
template <class C, int NW = C::NWAVES>
struct NmajorLoader {
  static constexpr int ROWN = C::BN * 2;     // bytes per LDS row (one k)
  static constexpr int CPRN = ROWN / 16;     // 16-byte chunks per row
  static constexpr int RPSN = 1024 / ROWN;   // rows per 1 KB DMA segment
  static constexpr int SEGS = C::BKE / RPSN; // segments per slice
  static constexpr int IPW = SEGS / NW;
  static_assert(1024 % ROWN == 0 && SEGS % NW == 0, "N-major B tile");  // used for BF16 only
  uint32_t off[IPW];  // row * ldb * 2 + column bytes of this lane's chunk, or `oob`
  uint32_t ldb2;      // bytes per row of B
  int lrow;           // this lane's row inside a segment

  __device__ __forceinline__ void init(int64_t ldb, int n0, int N, uint32_t oob, int wave,
                                       int lane) {
    ldb2 = static_cast<uint32_t>(ldb * 2);
    lrow = lane / CPRN;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int r = (wave * IPW + i) * RPSN + lrow;
      const int lc = (lane % CPRN) ^ (4 * (r & 3));
      const int n = n0 + 8 * lc;
      off[i] = n < N ? static_cast<uint32_t>(static_cast<int64_t>(r) * ldb * 2 + n * 2) : oob;
    }
  }

  // Same interface as DirectLoader::issue_buf (koff unused: the slice offset
  // k0 * ldb * 2 goes into the per-lane offset so the range check covers it).
  template <int I0 = 0, int I1 = IPW>
  __device__ __forceinline__ void issue_buf(char* lds_tile, int wave, __amdgpu_buffer_rsrc_t rsrc,
                                            int koff, uint32_t oob, int k0, int k_end,
                                            bool full) const {
    (void)koff;
    const uint32_t kbytes = static_cast<uint32_t>(k0) * ldb2;
#pragma unroll
    for (int i = I0; i < I1; ++i) {
      const int s = wave * IPW + i;
      const int r = s * RPSN + lrow;
      // off[i] == oob stays past the extent after the add (both are below 2^31).
      const uint32_t vo = (full || k0 + r < k_end) ? off[i] + kbytes : oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (G355_LDS void*)(lds_tile + s * 1024), 16,
                                               static_cast<int>(vo), 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------- register loader

template <class C, int ROWS>
struct GenericLoader {
  static constexpr int CHUNKS = ROWS * C::CPR;
  static constexpr int ITEMS = (CHUNKS + C::NT - 1) / C::NT;  // 16-byte chunks per thread
  uint32_t v[ITEMS][4];
  const char* base;
  int64_t ld;
  int row0, rows;
  bool kmajor;

  __device__ __forceinline__ bool item(int j, int tid, int& r, int& c) const {
    const int q = tid + C::NT * j;
    if (kmajor) { r = q / C::CPR; c = q % C::CPR; }
    else        { r = q % ROWS; c = q / ROWS; }
    return q < CHUNKS;
  }

  __device__ __forceinline__ void load(int tid, int k0, int k_end) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      int r, c;
      const bool in = item(j, tid, r, c);
      const int g = row0 + r;
      const bool row_ok = in && g < rows;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < C::CE; ++e) {
        const int k = k0 + c * C::CE + e;
        uint32_t x = 0u;
        if (row_ok && k < k_end) {
          const int64_t off = kmajor ? static_cast<int64_t>(g) * ld + k
                                     : static_cast<int64_t>(k) * ld + g;
          if constexpr (C::ES == 2) x = reinterpret_cast<const uint16_t*>(base)[off];
          else x = reinterpret_cast<const uint8_t*>(base)[off];
        }
        w[(e * C::ES) >> 2] |= x << (((e * C::ES) & 3) * 8);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) v[j][d] = w[d];
    }
  }

  __device__ __forceinline__ void store(char* lds_tile, int tid) const {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      int r, c;
      if (!item(j, tid, r, c)) continue;
      uint4 val = make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]);
      *reinterpret_cast<uint4*>(lds_tile + r * C::ROWB + ((c ^ swz<C::CPR>(r)) << 4)) = val;
    }
  }
};

// ------------------------------------------------------------ MFMA schedule

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <bool FP8> struct FragOf { using type = bf16x8; };   // 8 BF16: one ds_read_b128
template <> struct FragOf<true> { using type = i32x8; };     // 32 FP8: two ds_read_b128

// Wait until at most N of this wave's global loads are outstanding and all of
// its LDS operations are done, then barrier. (N is the number of loads of
// later slices that may stay in flight; loads complete in issue order.)
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Instruction order inside one k-step (sched_group_barrier masks: 0x008
// MFMA, 0x010 VMEM, 0x100 LDS read): each of the first R/2 MFMAs is followed
// by two fragment reads of the next k-step, so all reads are out early and
// their latency hides behind the remaining MFMAs; then the V global->LDS
// loads are spread over the MFMAs that follow.
template <int R, int M, int V>
__device__ __forceinline__ void step_hint() {
  constexpr int R2 = (R + 1) / 2;
  static_assert(R2 <= M, "reads per MFMA");
#pragma unroll
  for (int q = 0; q < R / 2; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  if constexpr (R % 2 == 1) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  constexpr int REST = M - R2;
  if constexpr (V == 0) {
    if constexpr (REST > 0) __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
  } else if constexpr (REST == 0) {
    __builtin_amdgcn_sched_group_barrier(0x010, V, 0);
  } else {
    constexpr int PER = (V + REST - 1) / REST;  // loads after each remaining MFMA
    constexpr int FULL = V / PER, LAST = V % PER;
#pragma unroll
    for (int q = 0; q < FULL; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, PER, 0);
    }
    if constexpr (LAST > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, LAST, 0);
    }
    constexpr int TAIL = REST - FULL - (LAST > 0 ? 1 : 0);
    if constexpr (TAIL > 0) __builtin_amdgcn_sched_group_barrier(0x008, TAIL, 0);
  }
}

// Part P (of SPREAD) of one wave's global->LDS loads of a slice: the A loads
// followed by the B loads, cut into SPREAD consecutive runs.
template <class C, int NA, int NB, int P>
struct DmaPart {
  static constexpr int T = NA + NB;
  static constexpr int LO = P * T / C::SPREAD, HI = (P + 1) * T / C::SPREAD;
  static constexpr int A0 = LO < NA ? LO : NA, A1 = HI < NA ? HI : NA;
  static constexpr int B0 = LO > NA ? LO - NA : 0, B1 = HI > NA ? HI - NA : 0;
  static constexpr int COUNT = P < C::SPREAD ? HI - LO : 0;
  template <class DA, class DB>
  __device__ __forceinline__ static void issue(const DA& da, const DB& db, char* at, char* bt,
                                               int wave, __amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rb, uint32_t oob_a,
                                               uint32_t oob_b, int koff, int k0, int k_end,
                                               bool full) {
    if constexpr (P < C::SPREAD && A1 > A0)
      da.template issue_buf<A0, A1>(at, wave, ra, koff, oob_a, k0, k_end, full);
    if constexpr (P < C::SPREAD && B1 > B0)
      db.template issue_buf<B0, B1>(bt, wave, rb, koff, oob_b, k0, k_end, full);
  }
};

// ------------------------------------------------------------------ epilogue

// Output tile epilogue for one wave, staged through LDS so that global C
// traffic is row-contiguous: the wave writes one 32-row strip of its
// accumulators (all FN column blocks) into a private LDS area, then reads it
// back with each lane holding 4 consecutive columns of one row, and applies
//   v = act(alpha * scale_a[m] * scale_b[n] * acc + beta * C_in[m,n] + bias[n])
// on float4 / 4-wide BF16 vectors. MFMA 32x32 accumulator layout: element e of
// lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32 of its 32x32 block.
// The LDS row stride is WTN+8 floats, which puts the two half-waves of an
// accumulator write (rows 4 apart) in opposite halves of the 64 banks.
template <class C>
struct EpiLayout {
  static constexpr int STR = C::WTN + 8;            // floats per LDS row
  static constexpr int WAVE_BYTES = 32 * STR * 4;   // one strip
  static constexpr int CG = C::WTN / 4;             // lanes per row (4 columns each)
  static constexpr int RPI = 64 / CG;               // rows per read instruction
  static constexpr int ITERS = 32 / RPI;
  static constexpr int TOTAL = C::NWAVES * WAVE_BYTES;
  static_assert(64 % CG == 0, "lanes per row");
};

template <class C, int OUT, bool SPLIT, int ACT>
__device__ __forceinline__ void epilogue(const GemmArgs& p, const f32x16 (&acc)[C::FM][C::FN],
                                         float* lds, int row0, int col0, int lane, int split) {
  using E = EpiLayout<C>;
  const int M = p.M, N = p.N;
  const int half = lane >> 5;
  const int cq = lane % E::CG;   // column group of this lane
  const int rq = lane / E::CG;   // row within a read instruction
  const int n = col0 + 4 * cq;
  const bool vec_ok = p.c_vec != 0 && n + 3 < N;

  // Per-column factors, fixed for this lane: alpha * scale_b[n] and bias[n].
  // An element is then fma(acc, scale_a[m] * cs[q], bias[q]) (+ beta * C_in).
  float cs[4], bias_v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) cs[q] = p.alpha;
  if constexpr (!SPLIT) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (n + q < N) {
        if constexpr (C::FP8 && !C::MX) cs[q] = p.alpha * p.scale_b[n + q];
        if (p.bias) bias_v[q] = bf16_bits_to_f32(p.bias[n + q]);
      }
    }
  }

  // C_in of strip i+1 is requested before strip i is processed, so its HBM
  // latency overlaps the epilogue math and stores of strip i. Quantised
  // outputs have no C_in.
  constexpr bool HAS_CIN = !SPLIT && (OUT == OUT_F32 || OUT == OUT_BF16);
  // Double-buffered C_in, except where the FP32 C_in of a 256-wide FP8 tile
  // would not fit next to its accumulators (it is then loaded per strip). A
  // BF16 C_in is held as its packed bits (two registers per four elements) and
  // widened where it is used.
  constexpr int CIN_BUFS = (C::FP8 && OUT == OUT_F32 && C::FN * C::FM >= 8) ? 1 : 2;
  using CinT = std::conditional_t<OUT == OUT_BF16, u32x2, float4>;
  CinT cin[CIN_BUFS][E::ITERS];
  auto load_cin = [&](int i, CinT (&dst)[E::ITERS]) {
#pragma unroll
    for (int it = 0; it < E::ITERS; ++it) {
      const int m = row0 + 32 * i + it * E::RPI + rq;
      if constexpr (OUT == OUT_BF16) dst[it] = u32x2{0u, 0u};
      else dst[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m >= M) continue;
      const int64_t off = static_cast<int64_t>(m) * p.ldc + n;
      if constexpr (OUT == OUT_BF16) {
        const uint16_t* c16 = static_cast<const uint16_t*>(p.C) + off;
        if (vec_ok) {
          // C_in is read once (non-temporal, like the stores of C).
          dst[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(c16));
        } else {
          unsigned h[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) h[q] = c16[q];
          dst[it] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        }
      } else {
        if (vec_ok) {
          const f32x4 c = __builtin_nontemporal_load(
              reinterpret_cast<const f32x4*>(static_cast<const float*>(p.C) + off));
          dst[it] = make_float4(c[0], c[1], c[2], c[3]);
        } else {
          float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) t[q] = load_cin1<OUT>(p.C, off + q);
          dst[it] = make_float4(t[0], t[1], t[2], t[3]);
        }
      }
    }
  };
  const bool use_c = HAS_CIN && p.beta != 0.f;
  if constexpr (HAS_CIN && CIN_BUFS == 2) {
    if (use_c) load_cin(0, cin[0]);
  }

  // Per-row factors (scale_a for FP8, the output scale and zero point for
  // quantised outputs) of the wave's 32*FM rows, loaded once up front: lane l
  // holds rows l and 64 + l. A row's value is later taken from its lane with
  // a cross-lane read, so no global load (and no wait on one, which on this
  // chip would also wait for every earlier store) sits inside the row loop.
  constexpr bool ROW_SA = !SPLIT && C::FP8 && !C::MX;
  constexpr bool ROW_QS = !SPLIT && OUT >= OUT_I8;
  constexpr bool ROW_QZ = !SPLIT && OUT == OUT_I8;
  constexpr int RREG = (32 * C::FM + 63) / 64;
  float row_sa[RREG], row_qs[RREG], row_qz[RREG];
#pragma unroll
  for (int j = 0; j < RREG; ++j) {
    const int lr = 64 * j + lane;
    const int m = row0 + lr;
    const bool ok = lr < 32 * C::FM && m < M;
    row_sa[j] = 1.f;
    row_qs[j] = 1.f;
    row_qz[j] = 0.f;
    if constexpr (ROW_SA) {
      if (ok) row_sa[j] = p.scale_a[m];
    }
    if constexpr (ROW_QS) {
      if (ok) row_qs[j] = p.qscale[m];
    }
    if constexpr (ROW_QZ) {
      if (ok && p.qzero) row_qz[j] = static_cast<float>(p.qzero[m]);
    }
  }

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    if constexpr (HAS_CIN) {
      if constexpr (CIN_BUFS == 2) {
        if (use_c && i + 1 < C::FM) load_cin(i + 1, cin[(i + 1) & 1]);
      } else {
        if (use_c) load_cin(i, cin[0]);
      }
    }
    // accumulators of rows 32i..32i+31 -> LDS strip
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        lds[(8 * (e >> 2) + 4 * half + (e & 3)) * E::STR + 32 * j + (lane & 31)] = acc[i][j][e];

#pragma unroll
    for (int it = 0; it < E::ITERS; ++it) {
      const int r = it * E::RPI + rq;
      const int m = row0 + 32 * i + r;
      const float4 a4 = *reinterpret_cast<const float4*>(lds + r * E::STR + 4 * cq);
      // Row m's factors sit in lane 32*(i&1) + r, register i/2. Read them
      // while every lane is active: a cross-lane read from a lane that has
      // left the loop below would not see its register.
      const int src = 32 * (i & 1) + r;
      float sa = 1.f, qs = 1.f, qz = 0.f;
      if constexpr (ROW_SA) sa = __shfl(row_sa[i >> 1], src);
      if constexpr (ROW_QS) qs = __shfl(row_qs[i >> 1], src);
      if constexpr (ROW_QZ) qz = __shfl(row_qz[i >> 1], src);
      if (m >= M) continue;
      float v[4] = {a4.x, a4.y, a4.z, a4.w};
      if constexpr (SPLIT) {
        // Partials are written once and read once by the reduction: non-temporal.
        float* w = p.workspace + (static_cast<int64_t>(split) * M + m) * N + n;
        // 16-byte stores where the workspace row start and this lane's
        // column group are 16-byte aligned and the group lies inside N.
        if (p.ws_vec && (N & 3) == 0 && n + 3 < N) {
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(w));
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) __builtin_nontemporal_store(v[q], w + q);
        }
        continue;
      } else {
        if constexpr (ROW_SA) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(v[q], sa * cs[q], bias_v[q]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = fmaf(v[q], cs[q], bias_v[q]);
        }
        if constexpr (HAS_CIN) {
          float c4[4];
          if constexpr (OUT == OUT_BF16) {
            const u32x2 h = cin[CIN_BUFS == 2 ? (i & 1) : 0][it];
            c4[0] = __uint_as_float(h.x << 16);
            c4[1] = __uint_as_float(h.x & 0xffff0000u);
            c4[2] = __uint_as_float(h.y << 16);
            c4[3] = __uint_as_float(h.y & 0xffff0000u);
          } else {
            const float4 cc = cin[CIN_BUFS == 2 ? (i & 1) : 0][it];
            c4[0] = cc.x;
            c4[1] = cc.y;
            c4[2] = cc.z;
            c4[3] = cc.w;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (use_c) v[q] = fmaf(p.beta, c4[q], v[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = apply_act<OUT>(v[q], ACT);
        const int64_t off = static_cast<int64_t>(m) * p.ldc + n;
        if (vec_ok) {
          store_out4<OUT>(p.C, off, v, qs, qz);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (n + q < N) store_out1<OUT>(p.C, off + q, v[q], qs, qz);
        }
      }
    }
  }
}

// Runs the epilogue with the activation as a compile-time parameter.
template <class C, int OUT, bool SPLIT>
__device__ __forceinline__ void run_epilogue(const GemmArgs& p, const f32x16 (&acc)[C::FM][C::FN],
                                             float* lds, int row0, int col0, int lane, int split) {
  if constexpr (SPLIT) {
    epilogue<C, OUT, true, ACT_NONE>(p, acc, lds, row0, col0, lane, split);
  } else {
    const int act = p.act;
    if (act == ACT_NONE)
      epilogue<C, OUT, false, ACT_NONE>(p, acc, lds, row0, col0, lane, split);
    else if (act == ACT_RELU)
      epilogue<C, OUT, false, ACT_RELU>(p, acc, lds, row0, col0, lane, split);
    else if (act == ACT_GELU_ERF)
      epilogue<C, OUT, false, ACT_GELU_ERF>(p, acc, lds, row0, col0, lane, split);
    else
      epilogue<C, OUT, false, ACT_GELU_TANH>(p, acc, lds, row0, col0, lane, split);
  }
}

// ------------------------------------------------------------------- the kernel

// RAGGED: K may end inside a 16-byte chunk of a DMA-fed row (patch_tail).
// Kept out of the other instantiations: the patch's code perturbs the
// register allocation of the K loop.
template <class C, int LA, int LB, int OUT, bool SPLIT, bool RAGGED>
__global__ void __launch_bounds__(C::NT)
gemm_tile_kernel(GemmArgs p) {
  // The LDS block holds the ring of K slices, and after the main loop the
  // epilogue's staging strips.
  constexpr int LDS_BYTES = C::STAGES * C::STAGE > EpiLayout<C>::TOTAL ? C::STAGES * C::STAGE
                                                                       : EpiLayout<C>::TOTAL;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which tile and which K range
  const int tiles = p.tiles_m * p.tiles_n;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int split = L / tiles;
  int tm, tn;
  tile_coords(L - split * tiles, p.tiles_m, p.tiles_n, 4, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int k_begin = split * p.k_split_len;
  const int k_end = min(p.K, k_begin + p.k_split_len);
  const int nk = k_end > k_begin ? (k_end - k_begin + C::BKE - 1) / C::BKE : 0;

  // ---- loaders
  // With 64-row tiles every byte of B is read by one workgroup only (each
  // column tile and K range is owned by one workgroup, and there are no other
  // row tiles when M <= 64): its copies are non-temporal (measured at the
  // M = 64 decode shapes: up to 13% faster). Other tiles re-read B panels
  // through the caches.
  DirectLoader<C, C::BM> da;
  DirectLoader<C, C::BN, C::NWAVES, (C::BM == 64 ? kPolicyNonTemporal : 0)> db;
  using NLoader = NmajorLoader<C>;
  NLoader dn;
  GenericLoader<C, C::BM> ga;
  GenericLoader<C, C::BN> gb;
  if constexpr (LA == LOAD_DIRECT) {
    da.init(p.lda, m0, p.M, wave, lane);
  } else {
    ga.base = static_cast<const char*>(p.A); ga.ld = p.lda; ga.row0 = m0; ga.rows = p.M;
    ga.kmajor = p.a_mn_major == 0;
  }
  // Buffer descriptors over each operand's extent (under 2 GiB, checked on
  // the host, so an offset past the extent plus the slice offset cannot wrap
  // into range).
  const uint32_t ext_a = static_cast<uint32_t>(
      (static_cast<int64_t>(p.M - 1) * p.lda + p.K) * C::ES);
  const uint32_t ext_b = static_cast<uint32_t>(
      LB == LOAD_DIRECT_N ? (static_cast<int64_t>(p.K - 1) * p.ldb + p.N) * C::ES
                          : (static_cast<int64_t>(p.N - 1) * p.ldb + p.K) * C::ES);
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.A), 0, static_cast<int>(ext_a), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.B), 0, static_cast<int>(ext_b), kBufferWord3);
  if constexpr (LB == LOAD_DIRECT) {
    db.init(p.ldb, n0, p.N, wave, lane);
  } else if constexpr (LB == LOAD_DIRECT_N) {
    dn.init(p.ldb, n0, p.N, ext_b, wave, lane);
  } else {
    gb.base = static_cast<const char*>(p.B); gb.ld = p.ldb; gb.row0 = n0; gb.rows = p.N;
    gb.kmajor = p.b_mn_major == 0;
  }
  constexpr int DMA_PER_SLICE = (LA == LOAD_DIRECT ? DirectLoader<C, C::BM>::IPW : 0) +
                                (LB == LOAD_DIRECT     ? DirectLoader<C, C::BN>::IPW
                                 : LB == LOAD_DIRECT_N ? NLoader::IPW
                                                       : 0);
  // At boundary j the loads of slice j+1 must be complete; those of slices
  // j+2 .. j+STAGES-1 (issued at the STAGES-2 boundaries before) may still
  // be in flight. Register-loaded slices are already in LDS by then.
  constexpr int DMA_BEHIND = DMA_PER_SLICE * (C::STAGES - 2);

  auto a_tile = [&](int st) { return smem + st * C::STAGE; };
  auto b_tile = [&](int st) { return smem + st * C::STAGE + C::A_BYTES; };

  auto fetch = [&](int st, int k0) __attribute__((always_inline)) {
    const bool full = k0 + C::BKE <= k_end;
    if constexpr (LA == LOAD_DIRECT)
      da.issue_buf(a_tile(st), wave, rsrc_a, k0 * C::ES, ext_a, k0, k_end, full);
    else ga.load(tid, k0, k_end);
    if constexpr (LB == LOAD_DIRECT)
      db.issue_buf(b_tile(st), wave, rsrc_b, k0 * C::ES, ext_b, k0, k_end, full);
    else if constexpr (LB == LOAD_DIRECT_N)
      dn.issue_buf(b_tile(st), wave, rsrc_b, 0, ext_b, k0, k_end, full);
    else gb.load(tid, k0, k_end);
  };
  auto commit = [&](int st) __attribute__((always_inline)) {
    if constexpr (LA == LOAD_GENERIC) ga.store(a_tile(st), tid);
    if constexpr (LB == LOAD_GENERIC) gb.store(b_tile(st), tid);
  };
  // K range ending inside a 16-byte chunk (K not a multiple of CE, last
  // split): the DMA copies no chunk that straddles k_end, so in the last
  // slice (stage st, once its copies have landed) each K-major DMA-fed row
  // gets that chunk written here: its elements below k_end, then zeros. The
  // tail tile then runs the full-tile MFMA path, as with zero-filled boundary
  // loads. Ends with a barrier that publishes the chunks.
  static_assert(!RAGGED || LA == LOAD_DIRECT || LB == LOAD_DIRECT, "ragged: a DMA-fed row");
  const bool ragged = k_end % C::CE != 0;
  auto patch_tail = [&](int st) {
    constexpr int RA = LA == LOAD_DIRECT ? C::BM : 0;
    constexpr int ROWS = RA + (LB == LOAD_DIRECT ? C::BN : 0);
    const int kc = k_end - k_end % C::CE;   // first element of the straddling chunk
    const int nb = (k_end - kc) * C::ES;    // its bytes below k_end: 1 .. 15
    const int cl = (kc - (k_begin + (nk - 1) * C::BKE)) / C::CE;  // its chunk in the slice
    // The thread index passes through an opaque move, so that none of the
    // per-lane address arithmetic below is hoisted out of the K loop (where
    // it would hold registers for the whole loop).
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid));
#pragma unroll
    for (int q0 = 0; q0 < ROWS; q0 += C::NT) {
      const int q = q0 + t;
      if (ROWS % C::NT != 0 && q >= ROWS) break;
      const bool is_a = q < RA;
      const int r = is_a ? q : q - RA;
      const int rows = is_a ? p.M : p.N;
      int g = (is_a ? m0 : n0) + r;
      g = g < rows ? g : rows - 1;  // rows past the operand repeat its last row, as the DMA does
      const uintptr_t src = reinterpret_cast<uintptr_t>(is_a ? p.A : p.B) +
                            (static_cast<int64_t>(g) * (is_a ? p.lda : p.ldb) + kc) * C::ES;
      // The valid bytes, read as the 4-byte aligned words that hold them (each
      // such word holds at least one byte of the operand, so no read leaves
      // the operand's pages), then shifted into place; bytes past k_end are 0.
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(src & ~uintptr_t{3});
      const int sh = static_cast<int>(src & 3);
      const int ndw = (sh + nb + 3) >> 2;   // 1 .. 5
      uint32_t d[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) d[i] = i < ndw ? wp[i] : 0u;
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t v = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
        const int keep = nb - 4 * i;        // valid bytes of word i
        w[i] = keep >= 4 ? v : keep <= 0 ? 0u : (v & ((1u << (8 * keep)) - 1u));
      }
      char* dst = (is_a ? a_tile(st) : b_tile(st)) + r * C::ROWB + ((cl ^ swz<C::CPR>(r)) << 4);
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  // ---- per-lane fragment addresses (bytes inside a tile)
  const int wm0 = (wave / C::WN) * C::WTM;
  const int wn0 = (wave % C::WN) * C::WTN;
  const int sw = swz<C::CPR>(lane & 31);  // a lane's rows all share their low 5 bits
  const int half = lane >> 5;
  const int a_row = (wm0 + (lane & 31)) * C::ROWB;
  const int b_row = (wn0 + (lane & 31)) * C::ROWB;
  // N-major B: within each group of 16 lanes, lane j points its transposing
  // read at row (j / 4) of a 4-row band and columns 4*(j % 4) .. +3 of the
  // group's 16 columns; lane i then receives column i of the 4 rows. kq =
  // (lane%16)/4 is the lane's row in the band, so its chunks are XORed with 4*kq.
  int ntr_row = 0, ntr_col[C::FN];
  if constexpr (LB == LOAD_DIRECT_N) {
    const int kq = (lane & 15) >> 2;
    ntr_row = (8 * half + kq) * NLoader::ROWN + 8 * (lane & 1);
    const int lc0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      ntr_col[j] = ((((wn0 + 32 * j) >> 3) ^ (4 * kq)) + lc0) << 4;
  }

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Fragment registers: two sets, so that the reads of the next k-step go to
  // one set while the MFMAs of the current k-step consume the other.
  using Frag = typename FragOf<C::FP8>::type;
  Frag fa0[C::FM], fb0[C::FN], fa1[C::FM], fb1[C::FN];

  // LDS -> registers: the fragments of k-step t of the slice in stage st.
  auto reads = [&](int st, int t, Frag (&fa)[C::FM], Frag (&fb)[C::FN]) {
    const char* at = a_tile(st);
    const char* bt = b_tile(st);
    if constexpr (!C::FP8) {
      const int co = ((2 * t + half) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(at + a_row + i * 32 * C::ROWB + co);
      if constexpr (LB == LOAD_DIRECT_N) {
        // k rows 16t + 8*half + 0..7 of the lane's column, as two transposing
        // reads of four rows each (rows 16t + 8*half + 4r + kq, kq = (lane%16)/4).
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const char* q = bt + ntr_row + ntr_col[j] + (16 * t) * NLoader::ROWN;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((G355_LDS s16x4*)(q));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (G355_LDS s16x4*)(q + 4 * NLoader::ROWN));
          fb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      } else {
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          fb[j] = *reinterpret_cast<const bf16x8*>(bt + b_row + j * 32 * C::ROWB + co);
      }
    } else {
      // Registers 0-3 and 4-7 of a lane take two 16-byte chunks of its row.
      // The MX scaled MFMA treats registers 0-3 of lanes i and i+32 as one
      // 32-element K block (scaled by lane i's scale byte) and registers 4-7
      // as the next (lane i+32's byte), so with MX the chunks are 4t+half and
      // 4t+2+half: block 2t of the slice, then block 2t+1. Without block
      // scales any assignment works as long as A and B agree; the plain path
      // keeps a lane's 32 bytes contiguous.
      const int c0 = C::MX ? 4 * t + half : 4 * t + 2 * half;
      const int c1 = C::MX ? c0 + 2 : c0 + 1;
      const int co0 = (c0 ^ sw) << 4;
      const int co1 = (c1 ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(at + a_row + i * 32 * C::ROWB + co0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(at + a_row + i * 32 * C::ROWB + co1);
        fa[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const i32x4 lo = *reinterpret_cast<const i32x4*>(bt + b_row + j * 32 * C::ROWB + co0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(bt + b_row + j * 32 * C::ROWB + co1);
        fb[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  // MX block scales of the slice being multiplied: per A row block i (B
  // column block j) the word holding the four E8M0 scales of the lane's row
  // (column) for this slice, shifted right by 8*half, so that byte 2t is the
  // scale of the block k-step t takes from this lane (block 2t for lanes
  // 0-31, 2t+1 for lanes 32-63).
  constexpr int SFM = C::MX ? C::FM : 1, SFN = C::MX ? C::FN : 1;
  uint32_t mxa[SFM], mxb[SFN];
#pragma unroll
  for (int i = 0; i < SFM; ++i) mxa[i] = 0x7f7f7f7fu;
#pragma unroll
  for (int j = 0; j < SFN; ++j) mxb[j] = 0x7f7f7f7fu;

  auto mfmas_sel = [&](auto sel, const Frag (&fa)[C::FM], const Frag (&fb)[C::FN]) {
    constexpr int S = decltype(sel)::value;  // byte of the scale words (2t)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (C::MX)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0, 0, S, static_cast<int>(mxa[i]), S,
              static_cast<int>(mxb[j]));
        else if constexpr (C::FP8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 0,
                                                                     0, 0, 127, 0, 127);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
  };
  auto mfmas = [&](const Frag (&fa)[C::FM], const Frag (&fb)[C::FN], int t) {
    if (!C::MX || t == 0) mfmas_sel(std::integral_constant<int, 0>{}, fa, fb);
    else mfmas_sel(std::integral_constant<int, 2>{}, fa, fb);
  };

  // The K loop is one stream of k-steps. Each k-step issues its MFMAs on the
  // fragment set read during the previous k-step, interleaved with the reads
  // of the next k-step into the other set. Where the next k-step opens slice
  // j+1 ("boundary j"), the wave first waits for its share of that slice's
  // loads and for its own LDS traffic, and one barrier then publishes slice
  // j+1 and certifies that every wave has finished reading slice j; the loads
  // of slice j+STAGES then go into slice j's buffer. So the MFMAs of a
  // slice's last k-step overlap the barrier's aftermath and the first reads
  // of the next slice, and a slice's loads have STAGES-1 slices of MFMA work
  // to arrive. Register-loaded operands hold the slice fetched at boundary j
  // in registers and write it to LDS just before boundary j+1.
  // LDS fragment reads per k-step (an N-major B block takes two 8-byte
  // transposing reads).
  constexpr int READS = C::FP8              ? 2 * (C::FM + C::FN)
                        : LB == LOAD_DIRECT_N ? C::FM + 2 * C::FN
                                              : C::FM + C::FN;
  constexpr int MFMAS = C::FM * C::FN;
  constexpr bool ALL_DMA = LA == LOAD_DIRECT && (LB == LOAD_DIRECT || LB == LOAD_DIRECT_N);
  // With both operands on the DMA path, the loads of slice s are issued in
  // SPREAD parts: part 0 at boundary s-STAGES, part p in the (p-1)-th k-step
  // after it, so that the loads of all waves do not queue up at once.
  constexpr int NA = LA == LOAD_DIRECT ? DirectLoader<C, C::BM>::IPW : 0;
  constexpr int NB = LB == LOAD_DIRECT     ? DirectLoader<C, C::BN>::IPW
                     : LB == LOAD_DIRECT_N ? NLoader::IPW
                                           : 0;
  using Part0 = DmaPart<C, NA, NB, 0>;
  using Part1 = DmaPart<C, NA, NB, 1>;
  using Part2 = DmaPart<C, NA, NB, 2>;
  using Part3 = DmaPart<C, NA, NB, 3>;
  auto dma_part = [&](auto part, int s) {
    using Pt = decltype(part);
    const int k0 = k_begin + s * C::BKE;
    const int st = s % C::STAGES;
    if constexpr (LB == LOAD_DIRECT_N)
      Pt::issue(da, dn, a_tile(st), b_tile(st), wave, rsrc_a, rsrc_b, ext_a, ext_b, k0 * C::ES,
                k0, k_end, k0 + C::BKE <= k_end);
    else
      Pt::issue(da, db, a_tile(st), b_tile(st), wave, rsrc_a, rsrc_b, ext_a, ext_b, k0 * C::ES,
                k0, k_end, k0 + C::BKE <= k_end);
  };
  // ---- MX scale words. Every byte offset (row * ld + 4 * slice) is in the
  // per-lane offset and checked against the array's extent by the buffer
  // descriptor: rows past M (N) and words past the end read zeros.
  uint32_t mxa_raw[SFM], mxb_raw[SFN];
  // (Unused, and removed by the compiler, on the other paths.)
  const __amdgpu_buffer_rsrc_t rsrc_sa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.mx_a), 0, C::MX ? p.M * p.ldsa : 0, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrc_sb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.mx_b), 0, C::MX ? p.N * p.ldsb : 0, kBufferWord3);
  uint32_t voff_sa = 0, voff_sb = 0;
  int mx_blocks = 0;
  if constexpr (C::MX) {
    voff_sa = static_cast<uint32_t>(m0 + wm0 + (lane & 31)) * static_cast<uint32_t>(p.ldsa);
    voff_sb = static_cast<uint32_t>(n0 + wn0 + (lane & 31)) * static_cast<uint32_t>(p.ldsb);
    mx_blocks = (p.K + 31) >> 5;
  }
  // Issue the scale-word loads of slice s.
  auto mx_load = [&](int s) __attribute__((always_inline)) {
    const uint32_t kb = static_cast<uint32_t>((k_begin + s * C::BKE) >> 5);
#pragma unroll
    for (int i = 0; i < SFM; ++i)
      mxa_raw[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rsrc_sa, voff_sa + static_cast<uint32_t>(32 * i * p.ldsa) + kb, 0, 0);
#pragma unroll
    for (int j = 0; j < SFN; ++j)
      mxb_raw[j] = __builtin_amdgcn_raw_buffer_load_b32(
          rsrc_sb, voff_sb + static_cast<uint32_t>(32 * j * p.ldsb) + kb, 0, 0);
  };
  // Make slice s's loaded words current: blocks at or past ceil(K/32) get the
  // neutral scale 127 (their data are zeros, and a NaN scale code in the
  // caller's padding must not turn them into NaN), then the per-half shift.
  auto mx_ready = [&](int s) __attribute__((always_inline)) {
    const int rem = mx_blocks - ((k_begin + s * C::BKE) >> 5);
    const uint32_t keep = rem >= 4 ? 0xffffffffu : rem <= 0 ? 0u : (0xffffffffu >> (8 * (4 - rem)));
    const uint32_t fill = 0x7f7f7f7fu & ~keep;
#pragma unroll
    for (int i = 0; i < SFM; ++i) mxa[i] = ((mxa_raw[i] & keep) | fill) >> (8 * half);
#pragma unroll
    for (int j = 0; j < SFN; ++j) mxb[j] = ((mxb_raw[j] & keep) | fill) >> (8 * half);
  };

  // PATCH: this boundary publishes the last slice (nk - 1) of a ragged K range.
  auto boundary = [&](auto patch, int j) {
    commit((j + C::STAGES - 1) % C::STAGES);
    wait_loads_and_barrier<DMA_BEHIND>();
    if constexpr (decltype(patch)::value) {
      if (ragged) patch_tail((j + 1) % C::STAGES);
    }
    if constexpr (ALL_DMA) dma_part(Part0{}, j + C::STAGES);
    else fetch(j % C::STAGES, k_begin + (j + C::STAGES) * C::BKE);
  };
  auto step = [&](auto patch, int j, int t, const Frag (&ca)[C::FM], const Frag (&cb)[C::FN],
                  Frag (&na)[C::FM], Frag (&nb)[C::FN]) {
    if (t == C::KSTEPS - 1) {
      boundary(patch, j);
      reads((j + 1) % C::STAGES, 0, na, nb);
      mfmas(ca, cb, t);
      if constexpr (C::MX) mx_ready(j + 1);
      step_hint<READS, MFMAS, ALL_DMA ? Part0::COUNT : 0>();
    } else {
      // Later parts of the loads of slice j-1+STAGES.
      if constexpr (ALL_DMA) {
        if (t == 0) dma_part(Part1{}, j - 1 + C::STAGES);
        if (t == 1) dma_part(Part2{}, j - 1 + C::STAGES);
        if (t == 2) dma_part(Part3{}, j - 1 + C::STAGES);
      }
      if constexpr (C::MX) {
        if (t == 0) mx_load(j + 1);
      }
      reads(j % C::STAGES, t + 1, na, nb);
      mfmas(ca, cb, t);
      if (t == 0) step_hint<READS, MFMAS, ALL_DMA ? Part1::COUNT : 0>();
      else if (t == 1) step_hint<READS, MFMAS, ALL_DMA ? Part2::COUNT : 0>();
      else if (t == 2) step_hint<READS, MFMAS, ALL_DMA ? Part3::COUNT : 0>();
      else step_hint<READS, MFMAS, 0>();
    }
  };

  if (nk > 0) {
    // Prologue: slices 0..STAGES-2 in flight, then "boundary -1" publishes
    // slice 0 and the first k-step's fragments are read.
#pragma unroll
    for (int s = 0; s < C::STAGES - 1; ++s) {
      fetch(s, k_begin + s * C::BKE);
      commit(s);
    }
    if constexpr (C::MX) mx_load(0);
    wait_loads_and_barrier<DMA_BEHIND>();
    if constexpr (RAGGED) {
      if (ragged && nk == 1) patch_tail(0);
    }
    if constexpr (C::MX) mx_ready(0);
    fetch(C::STAGES - 1, k_begin + (C::STAGES - 1) * C::BKE);
    reads(0, 0, fa0, fb0);
    // Slices are taken U at a time so that each loop iteration holds an even
    // number of k-steps and the two fragment sets alternate statically. With
    // U = 2 and nk odd the last pass runs on slice nk, whose loads read zeros:
    // it adds exact zeros.
    constexpr int U = C::KSTEPS % 2 == 0 ? 1 : 2;
    // Ragged K: the last two slices run after the loop, so that the tail
    // patch (at the boundary that opens slice nk - 1) stays out of the loop
    // body and its register allocation.
    static_assert(!RAGGED || U == 1, "peeled slices assume one slice per pass");
    const int n_loop = (RAGGED && nk >= 2) ? nk - 2 : nk;
    for (int j0 = 0; j0 < n_loop; j0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
          if (((u * C::KSTEPS + t) & 1) == 0)
            step(std::false_type{}, j0 + u, t, fa0, fb0, fa1, fb1);
          else
            step(std::false_type{}, j0 + u, t, fa1, fb1, fa0, fb0);
        }
    }
    if constexpr (RAGGED) {
      if (nk >= 2) {
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
          if ((t & 1) == 0) step(std::true_type{}, nk - 2, t, fa0, fb0, fa1, fb1);
          else step(std::true_type{}, nk - 2, t, fa1, fb1, fa0, fb0);
        }
#pragma unroll
        for (int t = 0; t < C::KSTEPS; ++t) {
          if ((t & 1) == 0) step(std::false_type{}, nk - 1, t, fa0, fb0, fa1, fb1);
          else step(std::false_type{}, nk - 1, t, fa1, fb1, fa0, fb0);
        }
      }
    }
  }

  // The LDS ring becomes the epilogue's staging area: wait until no load into
  // it is in flight (the trailing zero-block loads included) and every wave is
  // done reading it.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float* elds = reinterpret_cast<float*>(smem + wave * EpiLayout<C>::WAVE_BYTES);
  const int row0 = m0 + wm0, col0 = n0 + wn0;
  run_epilogue<C, OUT, SPLIT>(p, acc, elds, row0, col0, lane, split);
}

// ----------------------------------------------------------- split-K reduction

// C = epilogue(sum over splits s = 0..S-1, in that order, of workspace[s]).
template <bool FP8, int OUT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(GemmArgs p) {
  const int64_t MN = static_cast<int64_t>(p.M) * p.N;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= MN) return;
  const int m = static_cast<int>(idx / p.N);
  const int n = static_cast<int>(idx - static_cast<int64_t>(m) * p.N);
  // All partials are loaded before the first add (one memory round trip
  // instead of split_k dependent ones), then summed in split order. Each is
  // read once: non-temporal.
  float part[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.split_k) part[s] = __builtin_nontemporal_load(p.workspace + s * MN + idx);
  float v = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.split_k) v += part[s];
  if constexpr (FP8) v = v * (p.scale_a[m] * p.scale_b[n]);
  v = p.alpha * v;
  const int64_t off = static_cast<int64_t>(m) * p.ldc + n;
  if constexpr (OUT == OUT_F32 || OUT == OUT_BF16) {
    if (p.beta != 0.f) v += p.beta * load_cin1<OUT>(p.C, off);
  }
  if (p.bias) v += bf16_bits_to_f32(p.bias[n]);
  v = apply_act<OUT>(v, p.act);
  float qs, qz;
  out_row_params<OUT>(p, m, qs, qz);
  store_out1<OUT>(p.C, off, v, qs, qz);
}

// The same, four consecutive elements of one row per thread (N and ldc
// multiples of 4, workspace and C 16-byte aligned): 16-byte partial loads and
// one vector store. The per-element arithmetic is the scalar kernel's.
template <bool FP8, int OUT>
__global__ void __launch_bounds__(256) splitk_reduce4_kernel(GemmArgs p) {
  const int64_t MN = static_cast<int64_t>(p.M) * p.N;
  const int64_t idx = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (idx >= MN) return;
  const int m = static_cast<int>(idx / p.N);
  const int n = static_cast<int>(idx - static_cast<int64_t>(m) * p.N);
  f32x4 part[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.split_k)
      part[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.workspace + s * MN + idx));
  float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < p.split_k) {
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] += part[s][q];
    }
  const int64_t off = static_cast<int64_t>(m) * p.ldc + n;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (FP8) v[q] = v[q] * (p.scale_a[m] * p.scale_b[n + q]);
    v[q] = p.alpha * v[q];
    if constexpr (OUT == OUT_F32 || OUT == OUT_BF16) {
      if (p.beta != 0.f) v[q] += p.beta * load_cin1<OUT>(p.C, off + q);
    }
    if (p.bias) v[q] += bf16_bits_to_f32(p.bias[n + q]);
    v[q] = apply_act<OUT>(v[q], p.act);
  }
  float qs, qz;
  out_row_params<OUT>(p, m, qs, qz);
  store_out4<OUT>(p.C, off, v, qs, qz);
}

// ------------------------------------------------------------------- launchers
//
// This file is compiled once per (ragged, output part) pair, with G355_PART
// (an OutPart) and G355_RAGGED (0 or 1) defined, and once with G355_REDUCE
// for the split-K reduction: each compile instantiates only the kernels of its
// output kind, so the kernel variants build in parallel.
#if defined(G355_PART)

template <class C, int LA, int LB, bool RAGGED, bool QUANT_OUT = true>
static hipError_t launch_cfg(const Plan& plan, const LaunchSpec& spec, const GemmArgs& a,
                             hipStream_t stream) {
  (void)spec;
  const dim3 grid(static_cast<unsigned>(plan.grid)), block(C::NT);
  constexpr int PART = G355_PART;
  if constexpr (PART == PART_SPLIT) {
    hipLaunchKernelGGL((gemm_tile_kernel<C, LA, LB, OUT_F32, true, RAGGED>), grid, block, 0,
                       stream, a);
  } else if constexpr (PART == PART_F32 || PART == PART_BF16) {
    constexpr int OUT = PART == PART_F32 ? OUT_F32 : OUT_BF16;
    hipLaunchKernelGGL((gemm_tile_kernel<C, LA, LB, OUT, false, RAGGED>), grid, block, 0, stream,
                       a);
  } else if constexpr (QUANT_OUT) {
    constexpr int OUT = PART == PART_I8 ? OUT_I8 : OUT_E4M3;
    hipLaunchKernelGGL((gemm_tile_kernel<C, LA, LB, OUT, false, RAGGED>), grid, block, 0, stream,
                       a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile shapes in use. 256x256 (one workgroup per CU): 128-byte K slices
// (64 BF16 / 128 FP8 elements) in two LDS stages; BF16 spreads each slice's
// loads over three k-steps, FP8 issues them at once. Measured at 4096^3:
// 128-byte slices beat 64-byte ones in a deeper ring (a 64-byte row is half
// a cache line, so twice the L2 requests), and four waves of 128x128 lost to
// eight waves of 128x64.
using Big16 = TileCfg<256, 256, 2, 4, false, 128, 2, 3>;
using Big8 = TileCfg<256, 256, 2, 4, true, 128, 2, 1>;
using Mid16 = TileCfg<256, 128, 4, 2, false, 128, 2, 2>;
using Mid8 = TileCfg<256, 128, 4, 2, true, 128, 2, 2>;
using Small16 = TileCfg<128, 128, 2, 2, false, 128, 2>;
using Small8 = TileCfg<128, 128, 2, 2, true, 128, 2>;
// MX (E8M0 block-scaled) FP8: the scale words take up to 12 more VGPRs per
// lane. With the slice's loads spread over both k-steps the 256x256 loop has
// room for them.
using Big8X = TileCfg<256, 256, 2, 4, true, 128, 2, 2, true>;
using Mid8X = TileCfg<256, 128, 4, 2, true, 128, 2, 2, true>;
using Small8X = TileCfg<128, 128, 2, 2, true, 128, 2, 1, true>;
// Few rows (M <= 64): 64x256 tiles, four waves of 64x64, and a ring of four
// slices (160 KB). Such a tile does little MFMA work per slice, so it is the
// memory latency that must be covered: three slices in flight instead of one.
// 64x128 (two waves of 64x64, six slices, 144 KB) for narrow N, where the
// wider tile would need a deep K split.
using Thin16 = TileCfg<64, 256, 1, 4, false, 128, 4>;
using Thin8 = TileCfg<64, 256, 1, 4, true, 128, 4>;
using Thin8X = TileCfg<64, 256, 1, 4, true, 128, 4, 1, true>;
using Narrow16 = TileCfg<64, 128, 1, 2, false, 128, 6>;
using Narrow8 = TileCfg<64, 128, 1, 2, true, 128, 6>;
using Narrow8X = TileCfg<64, 128, 1, 2, true, 128, 6, 1, true>;

// The launches of launch_tile, with the kernels' RAGGED flag R. Register
// loading of both operands has no ragged variant (it bounds every element).
template <bool R>
static hipError_t launch_tile_t(const Plan& plan, const LaunchSpec& spec, const GemmArgs& args,
                                hipStream_t stream) {
  GemmArgs a = args;
  a.a_mn_major = spec.a_kmajor ? 0 : 1;
  a.b_mn_major = spec.b_kmajor ? 0 : 1;
  const bool direct = spec.loader_a == LOAD_DIRECT && spec.loader_b == LOAD_DIRECT;
  if (spec.loader_b == LOAD_DIRECT_N) {
    // BF16, K-major A by DMA, N-contiguous B by DMA (checked by the caller).
    if (spec.fp8 || spec.loader_a != LOAD_DIRECT) return hipErrorInvalidValue;
    if (plan.bm == 64)
      return plan.bn == 256
                 ? launch_cfg<Thin16, LOAD_DIRECT, LOAD_DIRECT_N, R>(plan, spec, a, stream)
                 : launch_cfg<Narrow16, LOAD_DIRECT, LOAD_DIRECT_N, R>(plan, spec, a, stream);
    if (plan.bm == 256 && plan.bn == 256)
      return launch_cfg<Big16, LOAD_DIRECT, LOAD_DIRECT_N, R>(plan, spec, a, stream);
    if (plan.bm == 256 && plan.bn == 128)
      return launch_cfg<Mid16, LOAD_DIRECT, LOAD_DIRECT_N, R>(plan, spec, a, stream);
    return launch_cfg<Small16, LOAD_DIRECT, LOAD_DIRECT_N, R>(plan, spec, a, stream);
  }
  if (spec.mx) {
    // MX operands take the DMA loader only (checked by the caller).
    if (!direct) return hipErrorInvalidValue;
    if (plan.bm == 64)
      return plan.bn == 256
                 ? launch_cfg<Thin8X, LOAD_DIRECT, LOAD_DIRECT, R, false>(plan, spec, a, stream)
                 : launch_cfg<Narrow8X, LOAD_DIRECT, LOAD_DIRECT, R, false>(plan, spec, a, stream);
    if (plan.bm == 256 && plan.bn == 256)
      return launch_cfg<Big8X, LOAD_DIRECT, LOAD_DIRECT, R, false>(plan, spec, a, stream);
    if (plan.bm == 256)
      return launch_cfg<Mid8X, LOAD_DIRECT, LOAD_DIRECT, R, false>(plan, spec, a, stream);
    return launch_cfg<Small8X, LOAD_DIRECT, LOAD_DIRECT, R, false>(plan, spec, a, stream);
  }
  if (!direct) {
    // Register loading runs on the 128x128 tile only.
    if (spec.fp8) {
      if constexpr (R) return hipErrorInvalidValue;
      else return launch_cfg<Small8, LOAD_GENERIC, LOAD_GENERIC, R>(plan, spec, a, stream);
    }
    if (spec.loader_a == LOAD_DIRECT)
      return launch_cfg<Small16, LOAD_DIRECT, LOAD_GENERIC, R>(plan, spec, a, stream);
    if (spec.loader_b == LOAD_DIRECT)
      return launch_cfg<Small16, LOAD_GENERIC, LOAD_DIRECT, R>(plan, spec, a, stream);
    if constexpr (R) return hipErrorInvalidValue;
    else return launch_cfg<Small16, LOAD_GENERIC, LOAD_GENERIC, R>(plan, spec, a, stream);
  }
  if (plan.bm == 64 && plan.bn == 256)
    return spec.fp8 ? launch_cfg<Thin8, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream)
                    : launch_cfg<Thin16, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream);
  if (plan.bm == 64)
    return spec.fp8 ? launch_cfg<Narrow8, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream)
                    : launch_cfg<Narrow16, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream);
  if (plan.bm == 256 && plan.bn == 256)
    return spec.fp8 ? launch_cfg<Big8, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream)
                    : launch_cfg<Big16, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream);
  if (plan.bm == 256 && plan.bn == 128)
    return spec.fp8 ? launch_cfg<Mid8, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream)
                    : launch_cfg<Mid16, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream);
  return spec.fp8 ? launch_cfg<Small8, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream)
                  : launch_cfg<Small16, LOAD_DIRECT, LOAD_DIRECT, R>(plan, spec, a, stream);
}

hipError_t G355_PART_LAUNCHER(G355_RAGGED, G355_PART)(const Plan& plan, const LaunchSpec& spec,
                                                      const GemmArgs& args, hipStream_t stream) {
  return launch_tile_t<G355_RAGGED != 0>(plan, spec, args, stream);
}

#elif defined(G355_REDUCE)

template <bool FP8, bool VEC>
static hipError_t launch_reduce_k(const LaunchSpec& spec, const GemmArgs& a, hipStream_t stream) {
  const int64_t MN = static_cast<int64_t>(a.M) * a.N;
  const int64_t per_block = VEC ? 1024 : 256;
  const dim3 grid(static_cast<unsigned>((MN + per_block - 1) / per_block)), block(256);
  if (spec.out == OUT_BF16)
    hipLaunchKernelGGL((VEC ? splitk_reduce4_kernel<FP8, OUT_BF16> : splitk_reduce_kernel<FP8, OUT_BF16>),
                       grid, block, 0, stream, a);
  else if (spec.out == OUT_I8)
    hipLaunchKernelGGL((VEC ? splitk_reduce4_kernel<FP8, OUT_I8> : splitk_reduce_kernel<FP8, OUT_I8>),
                       grid, block, 0, stream, a);
  else if (spec.out == OUT_E4M3)
    hipLaunchKernelGGL((VEC ? splitk_reduce4_kernel<FP8, OUT_E4M3> : splitk_reduce_kernel<FP8, OUT_E4M3>),
                       grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((VEC ? splitk_reduce4_kernel<FP8, OUT_F32> : splitk_reduce_kernel<FP8, OUT_F32>),
                       grid, block, 0, stream, a);
  return hipGetLastError();
}

template <bool FP8>
static hipError_t launch_reduce(const LaunchSpec& spec, const GemmArgs& a, hipStream_t stream) {
  const auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  // Four elements per thread only while that still gives 256 workgroups or
  // more (smaller outputs need the threads: 100 x 512 ran 15.6 -> 17.0 us).
  const int64_t MN = static_cast<int64_t>(a.M) * a.N;
  const bool vec = MN >= 256 * 1024 && a.N % 4 == 0 && a.ldc % 4 == 0 &&
                   aligned16(a.workspace) && aligned16(a.C);
  return vec ? launch_reduce_k<FP8, true>(spec, a, stream)
             : launch_reduce_k<FP8, false>(spec, a, stream);
}

hipError_t launch_splitk_reduce(const Plan& plan, const LaunchSpec& spec, const GemmArgs& a,
                                hipStream_t stream) {
  (void)plan;
  // The FP32 per-row / per-column scales belong to plain FP8; MX scales were
  // applied inside the MFMAs.
  return spec.fp8 && !spec.mx ? launch_reduce<true>(spec, a, stream)
                              : launch_reduce<false>(spec, a, stream);
}

#endif  // G355_PART / G355_REDUCE

}  // namespace g355
