// bwd.hip -- fused backward of logprobs, entropy and KL(A||B).
//
// The probabilities are recomputed in registers from the per-row statistics
// the forward saved (JSD PR text pasted into PR #8838: "Recompute
// probabilities in registers during backward rather than retaining full FP32
// probability tensors"), p = exp((z - m) - log S) with m and log S kept apart,
// and the gradient is written contiguous in the input dtype (second commit
// message: "Gradients are returned contiguous"), bf16 by round-to-nearest-even.
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

template <int OP, int DT, bool VEC, int BLOCK, int UB>
__global__ __launch_bounds__(BLOCK) void bwd_kernel(BwdArgs p) {
  constexpr int ES = ElemSize<DT>::value;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
  const int64_t row = vb / tpr;
  const int32_t tile = (int32_t)(vb - row * tpr);
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = V / 8;
  const int32_t gt0 = tile * (BLOCK * UB) + threadIdx.x;
  const float gv = p.g[row * p.g_stride];
  const float qnan = __builtin_nanf("");
  const char* ra = row_ptr<DT>(p.a, row);

  if constexpr (OP == kKL) {
    const char* rb = row_ptr<DT>(p.b, row);
    char* oa = p.da ? p.da + row * (int64_t)V * ES : nullptr;
    char* ob = p.db ? p.db + row * (int64_t)V * ES : nullptr;
    const float ma = p.stats[4 * row + 0], lsa = p.stats[4 * row + 1];
    const float mb = p.stats[4 * row + 2], lsb = p.stats[4 * row + 3];
    const float kl = p.res[row];
    const bool da_nan = !(kl < kInf);  // +inf (support mismatch) or NaN
    const bool db_nan = kl != kl;
#pragma unroll
    for (int k = 0; k < UB; ++k) {
      const int32_t g = gt0 + k * BLOCK;
      if (g >= G) break;
      float xa[8], xb[8], ya[8], yb[8];
      load_group<DT, VEC>(ra, g, V, g_full, xa);
      load_group<DT, VEC>(rb, g, V, g_full, xb);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float ua = (xa[j] - ma) - lsa;
        const float ub = (xb[j] - mb) - lsb;
        const float pa = expf_fast(ua);
        const float pb = expf_fast(ub);
        ya[j] = da_nan ? qnan : mul0(pa, (ua - ub) - kl) * gv;
        yb[j] = db_nan ? qnan : (pb - pa) * gv;
      }
      if (oa) store_group<DT, VEC>(oa, g, V, g_full, ya);
      if (ob) store_group<DT, VEC>(ob, g, V, g_full, yb);
    }
  } else {
    char* oa = p.da + row * (int64_t)V * ES;
    const float m = p.stats[2 * row + 0], ls = p.stats[2 * row + 1];
    if constexpr (OP == kEntropy) {
      const float H = p.res[row];
      const bool nan_row = H != H;
#pragma unroll
      for (int k = 0; k < UB; ++k) {
        const int32_t g = gt0 + k * BLOCK;
        if (g >= G) break;
        float x[8], y[8];
        load_group<DT, VEC>(ra, g, V, g_full, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float u = (x[j] - m) - ls;  // log p_j
          const float pj = expf_fast(u);
          y[j] = nan_row ? qnan : mul0(pj, u + H) * (-gv);
        }
        store_group<DT, VEC>(oa, g, V, g_full, y);
      }
    } else {
      const int64_t t = load_id(p.ids, row, p.a.n_inner);
      const bool ignored = t == p.ignore_index;
      const bool bad = !ignored && (t < 0 || t >= V);
      const int32_t tg = (ignored || bad) ? -1 : (int32_t)(t >> 3);
      const int tj = (int)(t & 7);
#pragma unroll
      for (int k = 0; k < UB; ++k) {
        const int32_t g = gt0 + k * BLOCK;
        if (g >= G) break;
        float x[8], y[8], pr[8];
        load_group<DT, VEC>(ra, g, V, g_full, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pr[j] = expf_fast((x[j] - m) - ls);
          y[j] = ignored ? 0.0f : (bad ? qnan : -gv * pr[j]);
        }
        if (g == tg) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j == tj) y[j] = gv * (1.0f - pr[j]);
        }
        store_group<DT, VEC>(oa, g, V, g_full, y);
      }
    }
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
  if (dtype == kBF16) return vec ? launch_bwd_t<OP, kBF16, true>(p, stream) : launch_bwd_t<OP, kBF16, false>(p, stream);
  return vec ? launch_bwd_t<OP, kF32, true>(p, stream) : launch_bwd_t<OP, kF32, false>(p, stream);
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
