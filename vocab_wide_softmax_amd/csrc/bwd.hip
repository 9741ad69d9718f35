// bwd.hip -- fused backward of logprobs, entropy and KL(A||B).
//
// The probabilities are recomputed in registers from the per-row statistics
// the forward saved, never stored as an fp32 tensor (the JSD PR text pasted
// into PR #8838, "Changes"), p = exp((z - m) - log S) with m and log S kept
// apart, and the gradient is written contiguous in the input dtype (second
// commit message of PR #8838), bf16 by round-to-nearest-even.
//
// Grid: one workgroup per (row, column tile); tiles of a row are consecutive
// workgroups, so the workgroups in flight write one contiguous window of the
// output. Each lane handles UB groups of 8 columns per tile.
//
//   logprobs  dz_j = g (1[j = t] - p_j)            (RL-Kernel PR #208 nitpick)
//   entropy   dz_j = -g p_j (log p_j + H)          (0 where p_j = 0)
//   KL(A||B)  da_j = g p_A,j (log p_A,j - log p_B,j - KL)   (0 where p_A,j = 0)
//             db_j = g (p_B,j - p_A,j)
#include "device.h"
#include "launch.h"

namespace vws {

// Per-row constants of the backward.
struct RowBwd {
  float m, ls, mb, lsb;  // (m, log S) of A, and of B for KL
  float res;             // H or KL
  float gv;
  bool nan_a, nan_b, zero;
  int32_t tg;  // group holding the logprobs target, -1 if none
  int tj;
};

// The row's constants, loaded first so that the tile's loads issued after them stay in
// flight while these are used; derived without branches.
template <int OP>
__device__ __forceinline__ RowBwd row_consts(const BwdArgs& p, int64_t row, int32_t V) {
  RowBwd r;
  r.gv = p.g[row * p.g_stride];
  r.zero = false;
  r.tg = -1;
  r.tj = 0;
  if constexpr (OP == kKL) {
    r.m = p.stats[4 * row + 0];
    r.ls = p.stats[4 * row + 1];
    r.mb = p.stats[4 * row + 2];
    r.lsb = p.stats[4 * row + 3];
    r.res = p.res[row];
    r.nan_a = !(r.res < kInf);  // +inf (support mismatch) or NaN
    r.nan_b = r.res != r.res;
  } else {
    r.m = p.stats[2 * row + 0];
    r.ls = p.stats[2 * row + 1];
    r.mb = r.lsb = 0.0f;
    r.nan_b = false;
    if constexpr (OP == kEntropy) {
      r.res = p.res[row];
      r.nan_a = r.res != r.res;
    } else {
      r.res = 0.0f;
      const int64_t t = load_id(p.ids, row, p.a.n_inner);
      r.zero = t == p.ignore_index;
      r.nan_a = !r.zero && (t < 0 || t >= V);
      const bool ok = !r.zero && !r.nan_a;
      r.tg = ok ? (int32_t)(t >> 3) : -1;
      r.tj = ok ? (int)(t & 7) : 0;
    }
  }
  return r;
}

// Issues the loads of this lane's UB groups (g, g + BLOCK, ...) of one row; groups past the
// row end read as -inf and are not stored.
template <int DT, bool FULL, int BLOCK, int UB>
__device__ __forceinline__ void bwd_load(const char* row, int32_t g, int32_t G, int32_t V, int32_t g_full,
                                         float (&x)[UB][8]) {
#pragma unroll
  for (int u = 0; u < UB; ++u, g += BLOCK) {
    if (FULL) {
      load_group_vec<DT>(row, g, x[u]);
    } else if (g < G) {
      load_group<DT, true>(row, g, V, g_full, x[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[u][j] = -kInf;
    }
  }
}

// The B tile of KL, or (unused) the A tile for the single-input ops.
template <int OP, int UB, int NB>
__device__ __forceinline__ const float (&xb_ref(const float (&xa)[UB][8], const float (&xb)[NB][8]))[UB][8] {
  if constexpr (OP == kKL) return xb;
  else return xa;
}

template <int OP, int DT, bool FULL, int BLOCK, int UB>
__device__ __forceinline__ void bwd_store(const RowBwd& r, const float (&xa)[UB][8], const float (&xb)[UB][8],
                                          char* oa, char* ob, int32_t g, int32_t G, int32_t V, int32_t g_full) {
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int u = 0; u < UB; ++u, g += BLOCK) {
    if (!FULL && g >= G) break;
    if constexpr (OP == kKL) {
      float ya[8], yb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ua = (xa[u][j] - r.m) - r.ls;
        const float ub = (xb[u][j] - r.mb) - r.lsb;
        const PScaled pa = exp_split(ua);
        const PScaled pb = exp_split(ub);
        ya[j] = r.nan_a ? qnan : (mul0(pa.p, (ua - ub) - r.res) * r.gv) * pa.f;
        yb[j] = r.nan_b ? qnan : ((pb.p - pa.p) * r.gv) * pa.f;  // pa and pb share the scale
      }
      if (FULL) {
        if (oa) store_group_vec<DT>(oa, g, ya);
        if (ob) store_group_vec<DT>(ob, g, yb);
      } else {
        if (oa) store_group<DT, true>(oa, g, V, g_full, ya);
        if (ob) store_group<DT, true>(ob, g, V, g_full, yb);
      }
    } else {
      float y[8];
      if constexpr (OP == kEntropy) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float lp = (xa[u][j] - r.m) - r.ls;  // log p_j
          const PScaled pj = exp_split(lp);
          y[j] = r.nan_a ? qnan : (mul0(pj.p, lp + r.res) * (-r.gv)) * pj.f;
        }
      } else {
        float pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const PScaled pj = exp_split((xa[u][j] - r.m) - r.ls);
          pr[j] = pj.p * pj.f;
          y[j] = r.zero ? 0.0f : (r.nan_a ? qnan : (-r.gv * pj.p) * pj.f);
        }
        if (g == r.tg) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j == r.tj) y[j] = r.gv * (1.0f - pr[j]);
        }
      }
      if (FULL) store_group_vec<DT>(oa, g, y);
      else store_group<DT, true>(oa, g, V, g_full, y);
    }
  }
}

// Gradient of one element, the same arithmetic as bwd_store. For logprobs `tgt` marks the
// target's column.
template <int OP>
__device__ __forceinline__ void elem_grad(const RowBwd& r, float xa, float xb, bool tgt, float& ya, float& yb) {
  const float qnan = __builtin_nanf("");
  if constexpr (OP == kKL) {
    const float ua = (xa - r.m) - r.ls;
    const float ub = (xb - r.mb) - r.lsb;
    const PScaled pa = exp_split(ua);
    const PScaled pb = exp_split(ub);
    ya = r.nan_a ? qnan : (mul0(pa.p, (ua - ub) - r.res) * r.gv) * pa.f;
    yb = r.nan_b ? qnan : ((pb.p - pa.p) * r.gv) * pa.f;
  } else if constexpr (OP == kEntropy) {
    const float lp = (xa - r.m) - r.ls;
    const PScaled pj = exp_split(lp);
    ya = r.nan_a ? qnan : (mul0(pj.p, lp + r.res) * (-r.gv)) * pj.f;
  } else {
    const PScaled pj = exp_split((xa - r.m) - r.ls);
    ya = r.zero ? 0.0f : (r.nan_a ? qnan : (-r.gv * pj.p) * pj.f);
    if (tgt) ya = r.gv * (1.0f - pj.p * pj.f);
  }
}

// A whole fp32 tile of NP BLOCK 16-byte pieces (columns [8 g0, 8 g0 + 4 NP BLOCK)): the backward is
// elementwise, so instead of a lane's group of 8 columns (32 bytes, two 16-byte accesses that each
// cover every other 16-byte piece of the wave's span) lane l takes 16-byte pieces l, l + BLOCK, ...:
// every access of the wave covers one contiguous 1 KB.
template <int OP, int BLOCK, int NP>
__device__ __forceinline__ void bwd_tile_f32(const BwdArgs& p, int64_t row, const char* ra, const char* rb, char* oa,
                                             char* ob, int32_t g0, int32_t V) {
  const int64_t q0 = 2 * (int64_t)g0 + threadIdx.x;  // this lane's first piece
  f32x4 xa[NP], xb[OP == kKL ? NP : 1];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    xa[k] = stream_load(reinterpret_cast<const f32x4*>(ra) + q0 + k * BLOCK);
    if constexpr (OP == kKL) xb[k] = stream_load(reinterpret_cast<const f32x4*>(rb) + q0 + k * BLOCK);
  }
  __builtin_amdgcn_sched_barrier(0);
  const RowBwd r = row_consts<OP>(p, row, V);
  const int64_t tcol = r.tg >= 0 ? (int64_t)r.tg * 8 + r.tj : -1;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int64_t c0 = 4 * (q0 + k * BLOCK);
    f32x4 ya, yb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a, b = 0.0f;
      elem_grad<OP>(r, xa[k][e], OP == kKL ? xb[k][e] : 0.0f, c0 + e == tcol, a, b);
      ya[e] = a;
      yb[e] = b;
    }
    if (oa) stream_store(ya, reinterpret_cast<f32x4*>(oa) + q0 + k * BLOCK);
    if constexpr (OP == kKL)
      if (ob) stream_store(yb, reinterpret_cast<f32x4*>(ob) + q0 + k * BLOCK);
  }
}

// TG: groups of 8 columns per tile. The group path covers a tile with UB groups a lane (TG =
// BLOCK UB on 16-bit data); whole fp32 tiles take 2 TG / BLOCK 16-byte pieces a lane.
template <int OP, int DT, bool VEC, int BLOCK, int UB, int TG>
__global__ __launch_bounds__(BLOCK) void bwd_kernel(BwdArgs p) {
  static_assert(TG <= BLOCK * UB && (2 * TG) % BLOCK == 0, "tile");
  constexpr int ES = ElemSize<DT>::value;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = VEC ? V / 8 : 0;  // groups below this use 16-byte loads and stores
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, tpr);
    const int32_t tile = (int32_t)(vb - row * tpr);
    const int32_t g0 = tile * TG;
    const char* ra = row_ptr<DT>(p.a, row);
    const char* rb = OP == kKL ? row_ptr<DT>(p.b, row) : nullptr;
    char* oa = p.da ? p.da + row * (int64_t)V * ES : nullptr;
    char* ob = OP == kKL && p.db ? p.db + row * (int64_t)V * ES : nullptr;
    const int32_t g = g0 + threadIdx.x;
    float xa[UB][8], xb[OP == kKL ? UB : 1][8];
    if constexpr (DT == kF32 && VEC) {
      if (g0 + TG <= g_full) {
        bwd_tile_f32<OP, BLOCK, 2 * TG / BLOCK>(p, row, ra, rb, oa, ob, g0, V);
        continue;
      }
    }
    if (VEC && TG == BLOCK * UB && g0 + TG <= g_full) {
      // the whole tile's loads first, then the row constants: one memory latency per tile
      RawGroup<DT> wa[UB], wb[OP == kKL ? UB : 1];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        load_group_raw<DT>(ra, g + u * BLOCK, wa[u]);
        if constexpr (OP == kKL) load_group_raw<DT>(rb, g + u * BLOCK, wb[u]);
      }
      __builtin_amdgcn_sched_barrier(0);
      const RowBwd r = row_consts<OP>(p, row, V);
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        raw_to_float<DT>(wa[u], xa[u]);
        if constexpr (OP == kKL) raw_to_float<DT>(wb[u], xb[u]);
      }
      bwd_store<OP, DT, true, BLOCK, UB>(r, xa, xb_ref<OP, UB>(xa, xb), oa, ob, g, G, V, g_full);
    } else {
      // groups of this tile only (lanes past a narrower tile's end take none)
      const int32_t gt = min(G, g0 + TG);
      const RowBwd r = row_consts<OP>(p, row, V);
      bwd_load<DT, false, BLOCK, UB>(ra, g, gt, V, g_full, xa);
      if constexpr (OP == kKL) bwd_load<DT, false, BLOCK, UB>(rb, g, gt, V, g_full, xb);
      bwd_store<OP, DT, false, BLOCK, UB>(r, xa, xb_ref<OP, UB>(xa, xb), oa, ob, g, gt, V, g_full);
    }
  }
}

namespace {
constexpr int kBwdBlock = 256;
// Groups of 8 columns per lane per tile, the fastest by measurement: 2 for the single-input ops
// on 16-bit data (4096-column tiles), 1 for KL, which reads two inputs, and for fp32 data
// (2048-column tiles; on fp32 the single-input ops ran 11% slower with 2, KL 7% slower with 2).
constexpr int bwd_ub(int op, int dt) { return op == kKL || dt == kF32 ? 1 : 2; }
// Lanes per workgroup: 256.
constexpr int bwd_block(int, int) { return kBwdBlock; }
// Groups per tile: BLOCK UB, except fp32 KL, whose 1024-column tiles give every lane one 16-byte
// piece per input and gradient, as 16-bit KL tiles do (fp32 KL backward 1.71 -> 1.58 ms on the
// 8192-row causal-shift view against 128-lane workgroups of two pieces a lane; 64 lanes and
// looping over several tiles were slower still). The single-input fp32 ops keep 2048-column
// tiles: with 1024 the logprobs backward ran 25% slower, the entropy backward within 1%.
constexpr int bwd_tile_groups(int op, int dt) { return op == kKL && dt == kF32 ? kBwdBlock / 2 : kBwdBlock * bwd_ub(op, dt); }

template <int OP, int DT, bool VEC>
hipError_t launch_bwd_t(const BwdArgs& p, hipStream_t stream) {
  const int64_t blocks = grid_cap(p.N * p.tiles_per_row);
  hipLaunchKernelGGL((bwd_kernel<OP, DT, VEC, bwd_block(OP, DT), bwd_ub(OP, DT), bwd_tile_groups(OP, DT)>),
                     dim3((uint32_t)blocks), dim3(bwd_block(OP, DT)), 0, stream, p);
  return hipGetLastError();
}

template <int OP>
hipError_t launch_bwd_op(const BwdArgs& p, int dtype, bool vec, hipStream_t stream) {
  return dispatch_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    return vec ? launch_bwd_t<OP, DT, true>(p, stream) : launch_bwd_t<OP, DT, false>(p, stream);
  });
}
}  // namespace

int32_t bwd_tiles_per_row(int op, int dtype, int64_t V) {
  const int64_t G = (V + 7) / 8;
  const int64_t per = bwd_tile_groups(op, dtype);
  return (int32_t)((G + per - 1) / per);
}

hipError_t launch_bwd(int op, const BwdArgs& p, int dtype, bool vec, hipStream_t stream) {
  switch (op) {
    case kLogprobs: return launch_bwd_op<kLogprobs>(p, dtype, vec, stream);
    case kEntropy: return launch_bwd_op<kEntropy>(p, dtype, vec, stream);
    default: return launch_bwd_op<kKL>(p, dtype, vec, stream);
  }
}

}  // namespace vws
