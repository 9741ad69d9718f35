// gemm.h -- bf16 MFMA tile machinery for gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// A workgroup computes a BM x BN tile of C = A * B^T over the reduction dim K,
// where A is M x K and B is N x K (both indexed (row, k)). Each operand is read
// from global memory in one of two layouts:
//   ROWK : element (r, k) at base[r * ld + k]   (reduction dim contiguous)
//   KROW : element (r, k) at base[k * ld + r]   (row dim contiguous)
// and staged in LDS in that same orientation. MFMA fragments are read with
// ds_read_b128 from ROWK tiles and with two ds_read_b64_tr_b16 (the gfx950
// transposing LDS read) from KROW tiles, so no operand is ever transposed in
// global memory.
//
// Staging: a ring of NSTAGE LDS stages filled by global_load_lds_dwordx4 (the
// load writes LDS directly, 16 bytes per lane, a wave's 64 lanes contiguous),
// NSTAGE - 1 stages in flight ahead of the one being multiplied; one workgroup
// barrier per stage. Because a wave's DMA writes 1 KB contiguously, LDS rows
// are not padded; 16-byte chunks are XOR-swizzled by row instead, which keeps
// the fragment reads free of bank conflicts.
//
// Split A (SA = 2): A is a pair of bf16 planes, hi and lo, whose sum carries an fp32 operand to
// about 2^-17 relative; both planes are staged and contracted with the same B tile into the same
// fp32 accumulators (all hi MFMAs of a k-slice, then all lo MFMAs, so that the two products
// feeding one accumulator are never back to back).
//
// MFMA 32x32x16 bf16 lane layout (checked on the device): lane l supplies
// A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32], e = 0..7, and holds
// accumulator v = C[8 (v / 4) + 4 (l / 32) + (v % 4)][l % 32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vws {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

enum Layout : int { ROWK = 0, KROW = 1 };

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Source of the 16-byte chunks that lie past the reduction length: they must add nothing.
extern __device__ const uint32_t kZeroChunk[4];

template <int BM_, int BN_, int BK_, int WM_, int WN_, int LA_, int LB_, int NSTAGE_, int SA_ = 1, int PIECES_ = 2>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, LA = LA_, LB = LB_, NSTAGE = NSTAGE_;
  static constexpr int SA = SA_;  // planes of A: 1, or 2 for a bf16 (hi, lo) pair
  static constexpr int PIECES = PIECES_;  // buffer-path refill pieces per stage (mainloop_t, mainloop_pp_t)
  static constexpr int NW = WM * WN, NT = NW * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int A_PLANE = BM * BK * 2;  // LDS bytes of one A plane of a stage
  static constexpr int A_BYTES = SA * A_PLANE, B_BYTES = BN * BK * 2, STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
  static constexpr int AP_INSTR = A_PLANE / 1024 / NW;  // DMA loads per wave of one A plane
  static constexpr int A_INSTR = SA * AP_INSTR, B_INSTR = B_BYTES / 1024 / NW;  // DMA loads per wave
  static constexpr int LOADS_PER_STAGE = A_INSTR + B_INSTR;
  static constexpr int MFMAS = SA * FM * FN;  // MFMAs per wave per 16-wide k-slice
  static_assert(SA == 1 || SA == 2, "planes");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert(BK == 32 || BK == 64, "ROWK swizzles exist for 4 and 8 chunks per row");
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert((LA != KROW || BM % 128 == 0) && (LB != KROW || BN % 128 == 0), "KROW swizzle needs 16 chunks per k-row");
  static_assert(A_PLANE % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole DMA instructions per wave");
};

// Global operand view.
struct Operand {
  const uint16_t* base;
  int64_t ld;    // elements between consecutive rows (ROWK) or consecutive k (KROW); multiple of 8
  int64_t rows;  // valid rows (>= 8 for KROW); rows beyond are clamped on load and masked by the caller
  int64_t K;     // valid reduction length, multiple of 8 for ROWK; chunks past it read zeros
  int64_t plane = 0;  // split A: elements from the hi plane to the lo plane (same layout)
};

__device__ __forceinline__ Operand lo_plane(const Operand& a) {
  return Operand{a.base + a.plane, a.ld, a.rows, a.K, 0};
}

// Swizzled chunk of a ROWK row (BK / 8 chunks of 16 B per row; the pattern keeps 8 and
// 16 consecutive rows at one chunk on distinct banks; for BK = 32, ((r >> 1) ^ (r >> 3)) & 3
// measured 33% of the LDS cycles in bank conflicts, (r >> 2) & 3 none) and of a KROW k-row
// (R / 8 chunks).
// A transposing read takes 64 contiguous bytes of each of 4 consecutive k-rows per half
// wave; XOR-ing the chunk index with 4 (kr mod 4) puts those four 64-byte pieces in the
// four distinct 64-byte windows of the 256-byte bank space, so they do not conflict.
template <int BK>
__device__ __forceinline__ int swz_rowk(int r) {
  if constexpr (BK == 32) return (r >> 2) & 3;
  else return (r ^ (r >> 3)) & 7;
}
__device__ __forceinline__ int swz_krow(int kr) { return 4 * (kr & 3); }

// Issue this wave's DMA loads of one operand tile for reduction offset k0 into lds_tile.
// EDGE: the tile may extend past the operand's rows or the stage past its reduction length
// (rows are clamped, chunks past K read zeros); an interior tile needs neither check, which
// leaves one pointer add per load.
template <int L, int R, int BK, int NW, int NINSTR, bool EDGE>
__device__ __forceinline__ void dma_tile(const Operand& op, int64_t r0, int64_t k0, char* lds_tile, int wave,
                                         int lane) {
#pragma unroll
  for (int j = 0; j < NINSTR; ++j) {
    const int instr = wave * NINSTR + j;
    const int o = instr * 1024 + lane * 16;  // byte offset this lane fills
    const void* src;
    if constexpr (L == ROWK) {
      const int r = o / (BK * 2), pc = (o % (BK * 2)) / 16;
      const int c = pc ^ swz_rowk<BK>(r);
      int64_t row = r0 + r;
      const int64_t k = k0 + c * 8;
      if constexpr (EDGE) {
        row = row < op.rows ? row : op.rows - 1;
        src = k < op.K ? (const void*)(op.base + row * op.ld + k) : (const void*)kZeroChunk;
      } else {
        src = (const void*)(op.base + row * op.ld + k);
      }
    } else {
      const int kr = o / (R * 2), pc = (o % (R * 2)) / 16;
      const int c = pc ^ swz_krow(kr);
      int64_t row = r0 + c * 8;
      const int64_t k = k0 + kr;
      if constexpr (EDGE) {
        row = row + 8 <= op.rows ? row : op.rows - 8;
        src = k < op.K ? (const void*)(op.base + k * op.ld + row) : (const void*)kZeroChunk;
      } else {
        src = (const void*)(op.base + k * op.ld + row);
      }
    }
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds_tile + instr * 1024), 16, 0, 0);
  }
}

// LDS byte address of a generic pointer into the workgroup's LDS.
// Buffer-resource form of dma_tile for interior tiles: the resource covers one stage of the
// operand tile (the rows r0 .. r0 + R of a ROWK operand from column k0, or the k-rows k0 .. k0 + BK
// of a KROW operand from column r0), so each lane's byte offset inside it is the same in every
// stage and only the scalar base moves. The loads take the buffer path (buffer_load ... lds),
// which on gfx950 costs the main loop less than the flat-address form. Usable when a stage spans
// fewer than 2^32 bytes (stage_span_fits).
template <int L, int R, int BK>
__device__ __forceinline__ bool stage_span_fits(const Operand& op) {
  return (int64_t)(L == ROWK ? R : BK) * op.ld * 2 <= (int64_t)0xFFFFFFFF;
}

// The base and size are the same in every lane; passing them through readfirstlane lets the
// compiler see that, so the descriptor stays in scalar registers. Without it the compiler may
// keep the base in vector registers and wrap every load in a loop over the distinct descriptors
// of the wave (four lane reads, two compares and an exec-mask loop per load).
template <int L, int R, int BK>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const Operand& op, int64_t r0, int64_t k0) {
  const uint16_t* base = L == ROWK ? op.base + r0 * op.ld + k0 : op.base + k0 * op.ld + r0;
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t span = __builtin_amdgcn_readfirstlane((uint32_t)((int64_t)(L == ROWK ? R : BK) * op.ld * 2));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, (int)span,
                                           0x00020000);
}

template <int L, int R, int BK, int NW, int NINSTR, int J0 = 0, int J1 = NINSTR>
__device__ __forceinline__ void dma_tile_buf(const Operand& op, int64_t r0, int64_t k0, char* lds_tile, int wave,
                                             int lane) {
  const __amdgpu_buffer_rsrc_t rsrc = stage_rsrc<L, R, BK>(op, r0, k0);
#pragma unroll
  for (int j = J0 < 0 ? 0 : J0; j < (J1 < NINSTR ? J1 : NINSTR); ++j) {
    const int instr = wave * NINSTR + j;
    const int o = instr * 1024 + lane * 16;  // byte offset this lane fills
    uint32_t voff;
    if constexpr (L == ROWK) {
      const int r = o / (BK * 2), pc = (o % (BK * 2)) / 16;
      const int c = pc ^ swz_rowk<BK>(r);
      voff = (uint32_t)(((int64_t)r * op.ld + c * 8) * 2);
    } else {
      const int kr = o / (R * 2), pc = (o % (R * 2)) / 16;
      const int c = pc ^ swz_krow(kr);
      voff = (uint32_t)(((int64_t)kr * op.ld + c * 8) * 2);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds_tile + instr * 1024), 16, (int)voff, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Fragment reads are issued with inline asm: the compiler neither sees them as LDS
// reads (so it does not drain the in-flight DMA stages with vmcnt(0) in front of
// them) nor waits for them; settle() waits (lgkmcnt(0)) and ties the registers.
__device__ __forceinline__ void ds_b128(u32x4& r, uint32_t a) { asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(a)); }
__device__ __forceinline__ void ds_tr16(uint32_t (&r)[2], uint32_t a) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
  r[0] = v.x;
  r[1] = v.y;
}

// One MFMA fragment: 8 reduction values of one row, for rows r0 + lane % 32, k-slice kk.
template <int L, int R, int BK>
__device__ __forceinline__ void read_frag(u32x4& f, const char* lds, int r0, int kk, int lane) {
  if constexpr (L == ROWK) {
    const int row = r0 + (lane & 31);
    const int c = (kk >> 3) + (lane >> 5);
    ds_b128(f, lds_addr(lds + row * (BK * 2) + ((c ^ swz_rowk<BK>(row)) << 4)));
  } else {
    // Transposing read: within each 16-lane group, lane 4p + q addresses k-row (k0 + p),
    // rows [4q, 4q + 4) of the group's 16 rows; lane i then holds row i at k0..k0+3
    // (and k0+4..k0+7 from the second read, four k-rows further).
    const int g = lane >> 4, i = lane & 15, p = i >> 2, q = i & 3;
    const int rbase = r0 + (g & 1) * 16 + 4 * q;
    const int kr = kk + (g >> 1) * 8 + p;
    const int c = rbase >> 3, within = (rbase * 2) & 15;
    const uint32_t a = lds_addr(lds + kr * (R * 2) + ((c ^ swz_krow(kr)) << 4) + within);
    uint32_t lo[2], hi[2];
    ds_tr16(lo, a);
    ds_tr16(hi, a + 4 * (R * 2));
    f = (u32x4){lo[0], lo[1], hi[0], hi[1]};
  }
}

template <class C>
struct Frags {
  u32x4 a[C::SA][C::FM], b[C::FN];
};

template <class C>
__device__ __forceinline__ void read_frags(Frags<C>& F, const char* sa, const char* sb, int wm, int wn, int kk, int lane) {
#pragma unroll
  for (int pl = 0; pl < C::SA; ++pl)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      read_frag<C::LA, C::BM, C::BK>(F.a[pl][i], sa + pl * C::A_PLANE, wm * C::TM + i * 32, kk, lane);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) read_frag<C::LB, C::BN, C::BK>(F.b[j], sb, wn * C::TN + j * 32, kk, lane);
}

// Wait for every outstanding LDS read and make the fragments depend on that wait. The
// scheduling barrier keeps the wait below the previous slice's MFMAs: the compiler may
// otherwise hoist it above them (they touch no memory), and the fragment reads issued at
// the start of that slice would then stall its MFMAs instead of overlapping them.
template <class C>
__device__ __forceinline__ void settle(Frags<C>& F) {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
#pragma unroll
  for (int pl = 0; pl < C::SA; ++pl)
#pragma unroll
    for (int i = 0; i < C::FM; ++i) asm volatile("" : "+v"(F.a[pl][i]));
#pragma unroll
  for (int j = 0; j < C::FN; ++j) asm volatile("" : "+v"(F.b[j]));
}

// Accumulators of one wave: FM x FN blocks.
template <class C>
struct Acc {
  f32x16 c[C::FM][C::FN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) c[i][j] = (f32x16){};
  }
};

// MFMA n of a slice. One plane: block (n / FN, n mod FN). A (hi, lo) pair: B fragment j = n / (2 FM)
// stays in place for the 2 FM MFMAs that use it (both planes of every A fragment, hi before lo), so
// the B operand changes 4 times a slice instead of 16: the pair GEMMs run clock-limited by how much
// their operands toggle, and this order took the backward 0.9% faster (39.74 -> 39.40 ms at
// 8192 x 4096 x 151936, one-card A/B). Every accumulator sees the same sequence either way (hi then
// lo of each slice), so the results are the same bits.
template <class C, int N>
__device__ __forceinline__ void mfma_n(Acc<C>& acc, const Frags<C>& F) {
  constexpr int pl = C::SA == 2 ? (N / C::FM) % 2 : 0;
  constexpr int i = C::SA == 2 ? N % C::FM : N / C::FN, j = C::SA == 2 ? N / (2 * C::FM) : N % C::FN;
  acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, F.a[pl][i]),
                                                        __builtin_bit_cast(bf16x8, F.b[j]), acc.c[i][j], 0, 0, 0);
}

template <class C, int N = 0>
__device__ __forceinline__ void mfmas(Acc<C>& acc, const Frags<C>& F) {
  if constexpr (N < C::MFMAS) {
    mfma_n<C, N>(acc, F);
    mfmas<C, N + 1>(acc, F);
  }
}

// Wait until at most n of this wave's DMA loads are outstanding (loads complete in order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Stage `s` has landed in LDS for every wave once this returns (given stages up to
// min(nk - 1, s + NSTAGE - 2) were issued).
template <class C>
__device__ __forceinline__ void stage_ready(int s, int nk) {
  const int newer = min(nk - 1 - s, C::NSTAGE - 2);
  if (newer >= 2) wait_vm<2 * C::LOADS_PER_STAGE>();
  else if (newer == 1) wait_vm<C::LOADS_PER_STAGE>();
  else wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");  // keep LDS reads and DMA issues on their side of the barrier
}

// In mainloop_t, buffer-path refills go out in Cfg::PIECES pieces per stage, each interleaved one
// load per MFMA. When the plain GEMMs all ran this loop (BK = 64, four slices per stage), two
// pieces were 1.2-1.9% faster than one burst of a stage's loads after the barrier (bit-identical
// results) and four pieces slower (the last piece then has under two slices of lead time); the
// split-A GEMMs (BK = 32, two slices per stage, twice the MFMAs per slice) were 5-7% faster with
// one burst. In mainloop_pp_t, PIECES = 2 with three or more stages splits each refill over the
// two read phases of a stage.

// Loads [J0, J1) of one stage's refill, counted over the A loads then the B loads (buffer path).
template <class C, int J0, int J1>
__device__ __forceinline__ void issue_buf_range(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int s,
                                                char* lds, int wave, int lane) {
  char* st = lds + (s % C::NSTAGE) * C::STAGE_BYTES;
  const int64_t k0 = (int64_t)s * C::BK;
  constexpr int P = C::AP_INSTR;
  if constexpr (J0 < P)
    dma_tile_buf<C::LA, C::BM, C::BK, C::NW, P, J0, J1>(A, m0, k0, st, wave, lane);
  if constexpr (C::SA == 2 && J0 < 2 * P && J1 > P)
    dma_tile_buf<C::LA, C::BM, C::BK, C::NW, P, J0 - P, J1 - P>(lo_plane(A), m0, k0, st + C::A_PLANE, wave, lane);
  if constexpr (J1 > C::A_INSTR)
    dma_tile_buf<C::LB, C::BN, C::BK, C::NW, C::B_INSTR, J0 - C::A_INSTR, J1 - C::A_INSTR>(B, n0, k0,
                                                                                             st + C::A_BYTES, wave,
                                                                                             lane);
}

// MFMA n of the slice (block n / FN, n % FN), then refill load J0 + n of stage s while n < J1 - J0.
// Scheduling barriers keep that order, so a wave's refill loads sit between its MFMAs instead of
// going out in one burst.
template <class C, int J0, int J1, int N>
__device__ __forceinline__ void mfmas_loads(Acc<C>& acc, const Frags<C>& F, const Operand& A, const Operand& B,
                                            int64_t m0, int64_t n0, int s, bool live, char* lds, int wave,
                                            int lane) {
  if constexpr (N < C::MFMAS) {
    mfma_n<C, N>(acc, F);
    if constexpr (N < J1 - J0) {
      __builtin_amdgcn_sched_barrier(0);
      if (live) issue_buf_range<C, J0 + N, J0 + N + 1>(A, B, m0, n0, s, lds, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfmas_loads<C, J0, J1, N + 1>(acc, F, A, B, m0, n0, s, live, lds, wave, lane);
  }
}

// One slice's MFMAs with refill piece `piece` (loads [piece * PL, (piece + 1) * PL)) of stage s.
template <class C, int PL>
__device__ __forceinline__ void mfmas_piece(Acc<C>& acc, const Frags<C>& F, int piece, const Operand& A,
                                            const Operand& B, int64_t m0, int64_t n0, int s, bool live, char* lds,
                                            int wave, int lane) {
  if (piece == 0) mfmas_loads<C, 0, PL, 0>(acc, F, A, B, m0, n0, s, live, lds, wave, lane);
  else if (piece == 1) mfmas_loads<C, PL, 2 * PL, 0>(acc, F, A, B, m0, n0, s, live, lds, wave, lane);
  else if (piece == 2) mfmas_loads<C, 2 * PL, 3 * PL, 0>(acc, F, A, B, m0, n0, s, live, lds, wave, lane);
  else mfmas_loads<C, 3 * PL, 4 * PL, 0>(acc, F, A, B, m0, n0, s, live, lds, wave, lane);
}

// C_tile(m0, n0) = A[m0 : m0 + BM, :] * B[n0 : n0 + BN, :]^T over k in [0, K), into acc.
// lds must hold LDS_BYTES. All threads of the workgroup must call this; it ends with a
// workgroup barrier, after which lds may be reused.
//
// Schedule: the fragments of the next k-slice are read while the MFMAs of the current
// one run; at the last slice of stage s the workgroup waits for stage s + 1, refills the
// stage-s buffer with stage s + NSTAGE (on the buffer path in Cfg::PIECES pieces spread over
// the following slices), and reads stage s + 1's first fragments before stage s's last MFMAs.
template <class C, bool EDGE, bool BUF>
__device__ __forceinline__ void mainloop_t(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t K,
                                           char* lds, Acc<C>& acc) {
  static_assert(!(EDGE && BUF), "the buffer loads serve interior tiles");
  constexpr int KQ = C::BK / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS targets stay scalar
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nk = (int)((K + C::BK - 1) / C::BK);
  acc.zero();

  auto issue = [&](int s) {
    char* st = lds + (s % C::NSTAGE) * C::STAGE_BYTES;
    const int64_t k0 = (int64_t)s * C::BK;
    if constexpr (BUF) {
      dma_tile_buf<C::LA, C::BM, C::BK, C::NW, C::AP_INSTR>(A, m0, k0, st, wave, lane);
      if constexpr (C::SA == 2)
        dma_tile_buf<C::LA, C::BM, C::BK, C::NW, C::AP_INSTR>(lo_plane(A), m0, k0, st + C::A_PLANE, wave, lane);
      dma_tile_buf<C::LB, C::BN, C::BK, C::NW, C::B_INSTR>(B, n0, k0, st + C::A_BYTES, wave, lane);
    } else {
      dma_tile<C::LA, C::BM, C::BK, C::NW, C::AP_INSTR, EDGE>(A, m0, k0, st, wave, lane);
      if constexpr (C::SA == 2)
        dma_tile<C::LA, C::BM, C::BK, C::NW, C::AP_INSTR, EDGE>(lo_plane(A), m0, k0, st + C::A_PLANE, wave, lane);
      dma_tile<C::LB, C::BN, C::BK, C::NW, C::B_INSTR, EDGE>(B, n0, k0, st + C::A_BYTES, wave, lane);
    }
  };
  auto stage_a = [&](int s) -> const char* { return lds + (s % C::NSTAGE) * C::STAGE_BYTES; };

#pragma unroll
  for (int s = 0; s < C::NSTAGE - 1; ++s)
    if (s < nk) issue(s);
  Frags<C> F[2];
  if (nk > 0) {
    stage_ready<C>(0, nk);
    if (C::NSTAGE - 1 < nk) issue(C::NSTAGE - 1);
    read_frags<C>(F[0], stage_a(0), stage_a(0) + C::A_BYTES, wm, wn, 0, lane);
  }
  // Refill pieces: with SP > 1 (buffer path), stage s + NSTAGE's loads go out in SP pieces of PL
  // loads, piece 0 right after the barrier that frees its buffer, piece p during slice p - 1 of the
  // next stage, each interleaved with a slice's MFMAs.
  constexpr int SP = BUF ? C::PIECES : 1;
  constexpr int PL = C::LOADS_PER_STAGE / SP;
  static_assert(SP >= 1 && SP <= KQ && C::LOADS_PER_STAGE % SP == 0 && (SP == 1 || PL <= C::MFMAS), "refill pieces");
  int cur = 0;
  for (int s = 0; s < nk; ++s) {
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      settle<C>(F[cur]);
      bool loads = false;
      int piece = 0, st = 0;
      if (q + 1 < KQ) {
        read_frags<C>(F[cur ^ 1], stage_a(s), stage_a(s) + C::A_BYTES, wm, wn, (q + 1) * 16, lane);
        // the rest of the stage whose piece 0 went out at the end of stage s - 1
        st = s + C::NSTAGE - 1;
        loads = SP > 1 && q + 1 < SP && s >= 1 && st < nk;
        piece = q + 1;
      } else if (s + 1 < nk) {
        stage_ready<C>(s + 1, nk);
        st = s + C::NSTAGE;
        if (SP == 1) {
          if (st < nk) issue(st);
        } else {
          loads = st < nk;
        }
        read_frags<C>(F[cur ^ 1], stage_a(s + 1), stage_a(s + 1) + C::A_BYTES, wm, wn, 0, lane);
      }
      if constexpr (SP > 1) {
        mfmas_piece<C, PL>(acc, F[cur], piece, A, B, m0, n0, st, loads, lds, wave, lane);
      } else {
        mfmas<C>(acc, F[cur]);
      }
      cur ^= 1;
    }
  }
  __syncthreads();
}

// Interior tiles (every row of both operand tiles exists and K is a whole number of stages)
// take the unchecked loads, through buffer resources when a stage of each operand spans fewer
// than 2^32 bytes.
template <class C>
__device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t K,
                                         char* lds, Acc<C>& acc) {
  const bool interior = m0 + C::BM <= A.rows && n0 + C::BN <= B.rows && K % C::BK == 0 && A.K >= K && B.K >= K;
  const bool fits = stage_span_fits<C::LA, C::BM, C::BK>(A) && stage_span_fits<C::LB, C::BN, C::BK>(B);
  // (the lo plane of a split A has the hi plane's layout, so its stages span the same bytes)
  if (interior && fits) mainloop_t<C, false, true>(A, B, m0, n0, K, lds, acc);
  else if (interior) mainloop_t<C, false, false>(A, B, m0, n0, K, lds, acc);
  else mainloop_t<C, true, false>(A, B, m0, n0, K, lds, acc);
}

// Wait until at most n whole stages of this wave's refill loads (n < NSTAGE) are outstanding.
template <class C>
__device__ __forceinline__ void wait_stages(int n) {
  if (C::NSTAGE > 3 && n >= 3) wait_vm<3 * C::LOADS_PER_STAGE>();
  else if (C::NSTAGE > 2 && n == 2) wait_vm<2 * C::LOADS_PER_STAGE>();
  else if (n == 1) wait_vm<C::LOADS_PER_STAGE>();
  else wait_vm<0>();
}

// Ping-pong schedule of the same product for interior tiles on the buffer path (8 waves, whole
// half-stages of slices). Waves 0-3 and 4-7 form two groups with one wave of each on every SIMD
// (waves go to SIMDs in turn). Every wave runs the same loop over half-stages: read the half's
// fragments (and issue or await its share of a stage refill), barrier, multiply the half from
// registers, barrier. Group 1 passes one extra barrier before the loop and group 0 one after it,
// so the groups run one phase apart: while one group multiplies, the other reads and waits, on
// every SIMD one wave feeds the MFMA pipe while the other waits on memory, and the waits of a
// SIMD's two waves no longer coincide. Counting phases from the first read of group 0 (phase
// -1), group g reads half k in phase 2k - 1 + g and multiplies it in phase 2k + g. While reading
// half 2s it issues its loads of stage s + NSTAGE - 1 (phase 4s - 1 + g), after the last read of
// stage s - 1, whose buffer they fill (phase 4s - 2); while reading half 2s + 1 it awaits stage
// s + 1 (phase 4s + 1 + g), before that stage's first read (phase 4s + 3). With three stages and
// Cfg::PIECES = 2 the refill goes out in two pieces, the second while reading half 2s + 1, which
// spreads the loads of a stage over both read phases (they queue on the CU's load path when
// issued at once). Every accumulator sees the same MFMA sequence as in mainloop_t, so the results
// are the same bits.
template <class C>
__device__ __forceinline__ void mainloop_pp_t(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t K,
                                              char* lds, Acc<C>& acc) {
  static_assert(C::NW == 8 && C::NSTAGE >= 2 && C::NSTAGE <= 4 && (C::BK / 16) % 2 == 0, "ping-pong layout");
  constexpr int HQ = C::BK / 32;  // slices per half-stage
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const bool second = wave >= 4;
  const int nk = (int)(K / C::BK);
  acc.zero();
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int s = 0; s < C::NSTAGE; ++s)
    if (s < nk) issue_buf_range<C, 0, C::LOADS_PER_STAGE>(A, B, m0, n0, s, lds, wave, lane);
  // stage 0 landed: the stages issued after it may stay in flight (loads complete in order)
  wait_stages<C>(min(C::NSTAGE - 1, nk - 1));
  barrier();
  if (second) barrier();
  Frags<C> F[HQ];
  int buf = 0;  // s mod NSTAGE
  for (int s = 0; s < nk; ++s) {
    const char* sa = lds + buf * C::STAGE_BYTES;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int h = 0; h < HQ; ++h) read_frags<C>(F[h], sa, sa + C::A_BYTES, wm, wn, (half * HQ + h) * 16, lane);
      constexpr bool SPLIT = C::NSTAGE >= 3 && C::PIECES == 2;
      constexpr int L0 = SPLIT ? C::LOADS_PER_STAGE / 2 : C::LOADS_PER_STAGE;
      const int st = s + C::NSTAGE - 1;
      if (half == 0) {
        if (s >= 1 && st < nk) issue_buf_range<C, 0, L0>(A, B, m0, n0, st, lds, wave, lane);
      } else {
        if (SPLIT && s >= 1 && st < nk) issue_buf_range<C, L0, C::LOADS_PER_STAGE>(A, B, m0, n0, st, lds, wave, lane);
        // stage s + 1 landed; stages s + 2 .. s + NSTAGE - 1 (those issued) stay in flight
        if (s + 1 < nk) wait_stages<C>(min(s + C::NSTAGE - 1, nk - 1) - (s + 1));
      }
#pragma unroll
      for (int h = 0; h < HQ; ++h) settle<C>(F[h]);
      barrier();
#pragma unroll
      for (int h = 0; h < HQ; ++h) mfmas<C>(acc, F[h]);
      barrier();
    }
    buf = buf + 1 == C::NSTAGE ? 0 : buf + 1;
  }
  if (!second) barrier();
  __syncthreads();
}

// The ping-pong schedule where it applies (interior tiles on the buffer path), else mainloop.
template <class C>
__device__ __forceinline__ void mainloop_pp(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t K,
                                            char* lds, Acc<C>& acc) {
  const bool interior = m0 + C::BM <= A.rows && n0 + C::BN <= B.rows && K % C::BK == 0 && A.K >= K && B.K >= K;
  const bool fits = stage_span_fits<C::LA, C::BM, C::BK>(A) && stage_span_fits<C::LB, C::BN, C::BK>(B);
  if (interior && fits) mainloop_pp_t<C>(A, B, m0, n0, K, lds, acc);
  else mainloop<C>(A, B, m0, n0, K, lds, acc);
}

// Row / column of accumulator v of block (i, j) for this lane, relative to the wave tile.
__device__ __forceinline__ int acc_row(int i, int v, int lane) { return i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int acc_col(int j, int lane) { return j * 32 + (lane & 31); }

}  // namespace gemm
}  // namespace vws
