// gemm.h -- bf16 MFMA tile machinery for gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// A workgroup computes a BM x BN tile of C = A * B^T over the reduction dim K,
// where A is M x K and B is N x K (both indexed (row, k)). Each operand is read
// from global memory in one of two layouts:
//   ROWK : element (r, k) at base[r * ld + k]   (reduction dim contiguous)
//   KROW : element (r, k) at base[k * ld + r]   (row dim contiguous)
// and staged in LDS in that same orientation (padded rows). MFMA fragments are
// read with ds_read_b128 from ROWK tiles and with two ds_read_b64_tr_b16 (the
// gfx950 transposing LDS read) from KROW tiles, so no operand is ever
// transposed in global memory.
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

enum Layout : int { ROWK = 0, KROW = 1 };

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Tile geometry. WM x WN waves; each wave owns a (BM/WM) x (BN/WN) sub-tile made
// of FM x FN MFMA blocks of 32 x 32.
template <int BM_, int BN_, int BK_, int WM_, int WN_, int LA_, int LB_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, LA = LA_, LB = LB_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 32, FN = TN / 32;
  // LDS row strides in bytes: ROWK tiles are [rows][BK] (+16 B keeps 8 lanes of a
  // b128 read on distinct banks), KROW tiles are [BK][rows] (+32 B keeps the four
  // rows of a transposing read on distinct banks).
  static constexpr int SA = LA == ROWK ? BK * 2 + 16 : BM * 2 + 32;
  static constexpr int SB = LB == ROWK ? BK * 2 + 16 : BN * 2 + 32;
  static constexpr int A_BYTES = LA == ROWK ? BM * SA : BK * SA;
  static constexpr int B_BYTES = LB == ROWK ? BN * SB : BK * SB;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // 16-byte chunks per stage, per operand, and per thread
  static constexpr int A_CHUNKS = BM * BK / 8, B_CHUNKS = BN * BK / 8;
  static constexpr int A_PER_T = A_CHUNKS / NT, B_PER_T = B_CHUNKS / NT;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "tile");
  static_assert(BK % 16 == 0 && A_CHUNKS % NT == 0 && B_CHUNKS % NT == 0, "chunks");
};

// Global operand view.
struct Operand {
  const uint16_t* base;
  int64_t ld;    // elements between consecutive rows (ROWK) or consecutive k (KROW)
  int64_t rows;  // valid rows (M or N); rows beyond are clamped on load, masked by the caller
  int64_t K;     // valid reduction length; k beyond reads as 0
};

// One 16-byte chunk of a stage: 8 consecutive elements along the contiguous dim.
// Out-of-range rows are clamped (their results are discarded by the epilogue);
// out-of-range reduction indices read as zero so they add nothing.
template <int L, int R, int BK>
__device__ __forceinline__ u32x4 load_chunk(const Operand& op, int64_t r0, int64_t k0, int c) {
  u32x4 v;
  if constexpr (L == ROWK) {
    constexpr int CPR = BK / 8;  // chunks per row
    const int r = c / CPR, kc = (c % CPR) * 8;
    int64_t row = r0 + r;
    row = row < op.rows ? row : op.rows - 1;
    const int64_t k = k0 + kc;
    const uint16_t* p = op.base + row * op.ld + k;
    if (k + 8 <= op.K) {
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (k + 2 * e < op.K) ? p[2 * e] : 0u;
        const uint32_t hi = (k + 2 * e + 1 < op.K) ? p[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
      }
      v = (u32x4){w[0], w[1], w[2], w[3]};
    }
  } else {
    constexpr int CPK = R / 8;  // chunks per k-row
    const int kk = c / CPK, rc = (c % CPK) * 8;
    const int64_t k = k0 + kk;
    int64_t row = r0 + rc;
    if (k >= op.K) {
      v = (u32x4){0u, 0u, 0u, 0u};
    } else if (row + 8 <= op.rows) {
      v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(op.base + k * op.ld + row));
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r_lo = row + 2 * e < op.rows ? row + 2 * e : op.rows - 1;
        const int64_t r_hi = row + 2 * e + 1 < op.rows ? row + 2 * e + 1 : op.rows - 1;
        w[e] = (uint32_t)op.base[k * op.ld + r_lo] | ((uint32_t)op.base[k * op.ld + r_hi] << 16);
      }
      v = (u32x4){w[0], w[1], w[2], w[3]};
    }
  }
  return v;
}

template <int L, int R, int BK, int S>
__device__ __forceinline__ void store_chunk(char* lds, int c, u32x4 v) {
  int off;
  if constexpr (L == ROWK) {
    constexpr int CPR = BK / 8;
    off = (c / CPR) * S + (c % CPR) * 16;
  } else {
    constexpr int CPK = R / 8;
    off = (c / CPK) * S + (c % CPK) * 16;
  }
  *reinterpret_cast<u32x4*>(lds + off) = v;
}

// MFMA fragment (8 reduction values of one row) for rows r0 + lane % 32, k-slice kk.
template <int L, int S>
__device__ __forceinline__ bf16x8 read_frag(const char* lds, int r0, int kk, int lane) {
  if constexpr (L == ROWK) {
    const int off = (r0 + (lane & 31)) * S + (kk + (lane >> 5) * 8) * 2;
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(lds + off));
  } else {
    // Transposing read: within each 16-lane group, lane 4p + q addresses k-row (k0 + p),
    // rows [4q, 4q + 4) of the group's 16 rows; lane i then holds row i at k0..k0+3.
    const int g = lane >> 4, i = lane & 15, p = i >> 2, q = i & 3;
    const int rbase = r0 + (g & 1) * 16 + 4 * q;
    const int kbase = kk + (g >> 1) * 8 + p;
    const char* a0 = lds + kbase * S + rbase * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a0 + 4 * S));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
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

// C_tile(m0, n0) = A[m0 : m0 + BM, :] * B[n0 : n0 + BN, :]^T over k in [0, K), into acc.
// lds must hold 2 * STAGE_BYTES. All threads of the workgroup must call this.
template <class C>
__device__ __forceinline__ void mainloop(const Operand& A, const Operand& B, int64_t m0, int64_t n0, int64_t K,
                                         char* lds, Acc<C>& acc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int nk = (int)((K + C::BK - 1) / C::BK);
  u32x4 ra[C::A_PER_T], rb[C::B_PER_T];
  acc.zero();

  auto gload = [&](int s) {
    const int64_t k0 = (int64_t)s * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) ra[i] = load_chunk<C::LA, C::BM, C::BK>(A, m0, k0, tid + i * C::NT);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) rb[i] = load_chunk<C::LB, C::BN, C::BK>(B, n0, k0, tid + i * C::NT);
  };
  auto lstore = [&](int buf) {
    char* sa = lds + buf * C::STAGE_BYTES;
    char* sb = sa + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) store_chunk<C::LA, C::BM, C::BK, C::SA>(sa, tid + i * C::NT, ra[i]);
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) store_chunk<C::LB, C::BN, C::BK, C::SB>(sb, tid + i * C::NT, rb[i]);
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) gload(s + 1);
    const char* sa = lds + buf * C::STAGE_BYTES;
    const char* sb = sa + C::A_BYTES;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 16) {
      bf16x8 fa[C::FM], fb[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[i] = read_frag<C::LA, C::SA>(sa, wm * C::TM + i * 32, kk, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) fb[j] = read_frag<C::LB, C::SB>(sb, wn * C::TN + j * 32, kk, lane);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc.c[i][j], 0, 0, 0);
    }
    if (s + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
}

// Row / column of accumulator v of block (i, j) for this lane, relative to the wave tile.
__device__ __forceinline__ int acc_row(int i, int v, int lane) { return i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int acc_col(int j, int lane) { return j * 32 + (lane & 31); }

}  // namespace gemm
}  // namespace vws
