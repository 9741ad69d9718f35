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

template <int OP, int DT, bool FULL>
__device__ __forceinline__ void bwd_groups(const RowBwd& r, const char* ra, const char* rb, char* oa, char* ob,
                                           int32_t g, int32_t stride, int n, int32_t G, int32_t V, int32_t g_full) {
  const float qnan = __builtin_nanf("");
  for (int k = 0; k < n; ++k, g += stride) {
    if (!FULL && g >= G) break;
    if constexpr (OP == kKL) {
      float xa[8], xb[8], ya[8], yb[8];
      if (FULL) {
        load_group_vec<DT>(ra, g, xa);
        load_group_vec<DT>(rb, g, xb);
      } else {
        load_group<DT, true>(ra, g, V, g_full, xa);
        load_group<DT, true>(rb, g, V, g_full, xb);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ua = (xa[j] - r.m) - r.ls;
        const float ub = (xb[j] - r.mb) - r.lsb;
        const float pa = expf_fast(ua);
        const float pb = expf_fast(ub);
        ya[j] = r.nan_a ? qnan : mul0(pa, (ua - ub) - r.res) * r.gv;
        yb[j] = r.nan_b ? qnan : (pb - pa) * r.gv;
      }
      if (FULL) {
        if (oa) store_group_vec<DT>(oa, g, ya);
        if (ob) store_group_vec<DT>(ob, g, yb);
      } else {
        if (oa) store_group<DT, true>(oa, g, V, g_full, ya);
        if (ob) store_group<DT, true>(ob, g, V, g_full, yb);
      }
    } else {
      float x[8], y[8];
      if (FULL) load_group_vec<DT>(ra, g, x);
      else load_group<DT, true>(ra, g, V, g_full, x);
      if constexpr (OP == kEntropy) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float u = (x[j] - r.m) - r.ls;  // log p_j
          const float pj = expf_fast(u);
          y[j] = r.nan_a ? qnan : mul0(pj, u + r.res) * (-r.gv);
        }
      } else {
        float pr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pr[j] = expf_fast((x[j] - r.m) - r.ls);
          y[j] = r.zero ? 0.0f : (r.nan_a ? qnan : -r.gv * pr[j]);
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

template <int OP, int DT, bool VEC, int BLOCK, int UB>
__global__ __launch_bounds__(BLOCK) void bwd_kernel(BwdArgs p) {
  constexpr int ES = ElemSize<DT>::value;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = VEC ? V / 8 : 0;  // groups below this use 16-byte loads and stores
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, tpr);
    const int32_t tile = (int32_t)(vb - row * tpr);
    const int32_t g0 = tile * (BLOCK * UB);
    RowBwd r;
    r.gv = p.g[row * p.g_stride];
    r.zero = false;
    r.tg = -1;
    r.tj = 0;
    const char* ra = row_ptr<DT>(p.a, row);
    const char* rb = nullptr;
    char* oa = p.da ? p.da + row * (int64_t)V * ES : nullptr;
    char* ob = nullptr;
    if constexpr (OP == kKL) {
      rb = row_ptr<DT>(p.b, row);
      ob = p.db ? p.db + row * (int64_t)V * ES : nullptr;
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
        if (!r.zero && !r.nan_a) {
          r.tg = (int32_t)(t >> 3);
          r.tj = (int)(t & 7);
        }
      }
    }
    const int32_t g = g0 + threadIdx.x;
    if (VEC && g0 + BLOCK * UB <= g_full) {
      bwd_groups<OP, DT, true>(r, ra, rb, oa, ob, g, BLOCK, UB, G, V, g_full);
    } else {
      bwd_groups<OP, DT, false>(r, ra, rb, oa, ob, g, BLOCK, UB, G, V, g_full);
    }
  }
}

namespace {
constexpr int kBwdBlock = 256;
constexpr int kBwdUB = 2;

template <int OP, int DT, bool VEC>
hipError_t launch_bwd_t(const BwdArgs& p, hipStream_t stream) {
  const int64_t blocks = grid_cap(p.N * p.tiles_per_row);
  hipLaunchKernelGGL((bwd_kernel<OP, DT, VEC, kBwdBlock, kBwdUB>), dim3((uint32_t)blocks), dim3(kBwdBlock), 0, stream, p);
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

int32_t bwd_tiles_per_row(int64_t V) {
  const int64_t G = (V + 7) / 8;
  return (int32_t)((G + kBwdBlock * kBwdUB - 1) / (kBwdBlock * kBwdUB));
}

hipError_t launch_bwd(int op, const BwdArgs& p, int dtype, bool vec, hipStream_t stream) {
  switch (op) {
    case kLogprobs: return launch_bwd_op<kLogprobs>(p, dtype, vec, stream);
    case kEntropy: return launch_bwd_op<kEntropy>(p, dtype, vec, stream);
    default: return launch_bwd_op<kKL>(p, dtype, vec, stream);
  }
}

}  // namespace vws
