// jsd.hip -- generalized Jensen-Shannon divergence, 0 < beta < 1.
//
// The JSD pull request pasted into DeepSpeed PR #8838 ("Changes", "Scope and
// limitations") adds jsd(student, teacher, beta): fp32 per token, gradients to
// both inputs, beta = 0 and beta = 1 as explicit forward / reverse KL branches
// (handled by the host through the KL kernels), and for the interior a
// statistics pass followed by a divergence pass, because the nonlinear mixture
// needs the global normalisation first. With S = student, T = teacher and the
// mixture M = (1 - beta) p_S + beta p_T (mixture weight beta on the teacher, as
// in GKD-style distillation):
//
//   K_S = sum p_S (log p_S - log M),   K_T = sum p_T (log p_T - log M)
//   JSD = beta K_T + (1 - beta) K_S                 (the two KL-to-mixture sums)
//   dJSD/ds_j = (1 - beta) p_S,j ((log p_S,j - log M_j) - K_S)
//   dJSD/dt_j = beta p_T,j ((log p_T,j - log M_j) - K_T)
//
// Pass 1 is the KL forward's single read of both inputs, kept for its
// statistics (m, log S) of S and T. Pass 2 (jsd_div_kernel) reads both again and
// accumulates K_S and K_T; with P > 1 vocabulary parts per row the partial sums
// are added in part order by jsd_combine_kernel. The backward recomputes p_S,
// p_T and log M in registers from the saved (m, log S, K_S, K_T) and writes
// contiguous gradients. Masked (-inf) entries have zero weight (the zero-weight
// product); rows where either input is undefined give NaN.
#include "device.h"
#include "launch.h"
#include "span_f32.h"

namespace vws {

namespace {
constexpr int kJsdBlock = 256;
constexpr int kJsdU = 2;   // forward groups per lane per batch
constexpr int kJsdUB = 2;  // backward groups per lane per tile (16-bit data: 4096-column tiles)
// Backward tile of fp32 data, in groups of 8 columns: 2048 columns, two 16-byte pieces a lane per
// input (0.90 -> 0.83 ms at 4096 x 75968 against 4096-column tiles of four pieces a lane).
constexpr int kJsdTileF32 = kJsdBlock;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kFltMin = 1.17549435e-38f;
}  // namespace

// Per-row constants: (m, log S) of both inputs, log S in base 2, beta and 1 - beta.
struct JsdRow {
  float ms, lss, mt, lst;
  float lss2, lst2;  // log S * log2 e
  float wt, ws;
  bool bad;
};

__device__ __forceinline__ JsdRow jsd_row(const float* st4, float beta) {
  JsdRow r;
  r.ms = st4[0];
  r.lss = st4[1];
  r.mt = st4[2];
  r.lst = st4[3];
  r.lss2 = r.lss * kLog2e;
  r.lst2 = r.lst * kLog2e;
  r.wt = beta;
  r.ws = 1.0f - beta;
  // a defined row has a finite max and a finite log S >= 0; an all -inf row has
  // m = -inf, a NaN or +inf entry gives m = +inf or S = NaN
  r.bad = !(__builtin_isfinite(r.ms) && __builtin_isfinite(r.lss) && __builtin_isfinite(r.mt) &&
            __builtin_isfinite(r.lst));
  return r;
}

// Base-2 log-probabilities u = log2 p of one group of 8 columns, the probabilities, and
// l = log2 M of the mixture. log M is taken from the mixture itself while that is a
// normal float; a group holding a smaller mixture (both probabilities tiny, or both
// entries masked) recomputes it as mx + log2((1-b) 2^(us-mx) + b 2^(ut-mx)) with
// mx = max(us, ut), whose argument lies in [min(b, 1-b), 1] (NaN when both are masked,
// where both weights are 0).
// FULL (the backward): ps and pt are kept at the 2^64 scale of exp_split, p = ps fs and p = pt ft,
// so that a gradient whose probability lies below 2^-126 is formed at scale and rounded once
// (device.h); the divergence pass sums its terms against ones near 1 and keeps fs = ft = 1.
struct JsdGroup {
  float us[8], ut[8], ps[8], pt[8], fs[8], ft[8], lm[8];
};

template <bool FULL>
__device__ __forceinline__ void jsd_group(const JsdRow& r, const float (&xs)[8], const float (&xt)[8], JsdGroup& q) {
  bool small = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // (z - m) log2 e - log2 S: the centred difference is exact for entries near the max,
    // and the fma rounds once
    q.us[j] = __builtin_fmaf(xs[j] - r.ms, kLog2e, -r.lss2);
    q.ut[j] = __builtin_fmaf(xt[j] - r.mt, kLog2e, -r.lst2);
    if constexpr (FULL) {
      q.ps[j] = __builtin_amdgcn_exp2f(q.us[j] + kSumScaleLog2);
      q.pt[j] = __builtin_amdgcn_exp2f(q.ut[j] + kSumScaleLog2);
      q.fs[j] = q.ft[j] = kSumUnscale;
    } else {
      q.ps[j] = __builtin_amdgcn_exp2f(q.us[j]);
      q.pt[j] = __builtin_amdgcn_exp2f(q.ut[j]);
      q.fs[j] = q.ft[j] = 1.0f;
    }
    const float mix = __builtin_fmaf(r.wt, q.pt[j] * q.ft[j], r.ws * (q.ps[j] * q.fs[j]));
    q.lm[j] = __builtin_amdgcn_logf(mix);
    small |= !(mix >= kFltMin);
  }
  if (small) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float mx = fmaxf(q.us[j], q.ut[j]);
      const float inner =
          __builtin_fmaf(r.wt, __builtin_amdgcn_exp2f(q.ut[j] - mx), r.ws * __builtin_amdgcn_exp2f(q.us[j] - mx));
      const float mix = __builtin_fmaf(r.wt, q.pt[j] * q.ft[j], r.ws * (q.ps[j] * q.fs[j]));
      if (!(mix >= kFltMin)) q.lm[j] = mx + __builtin_amdgcn_logf(inner);
    }
  }
}

// ---- pass 2: the two KL-to-mixture sums ------------------------------------------------

// Writes the row's outputs from the base-2 sums: JSD, and stats (m_s, log S_s, m_t, log S_t,
// K_S, K_T) with K in natural units.
__device__ void jsd_finalize(const JsdArgs& p, int64_t row, float Ks, float Kt) {
  const float* st4 = p.st4 + 4 * row;
  float* o = p.stats + 6 * row;
  const JsdRow r = jsd_row(st4, p.beta);
  o[0] = r.ms;
  o[1] = r.lss;
  o[2] = r.mt;
  o[3] = r.lst;
  const float qnan = __builtin_nanf("");
  const double ks = (double)Ks * 0.69314718055994530942, kt = (double)Kt * 0.69314718055994530942;
  o[4] = r.bad ? qnan : (float)ks;
  o[5] = r.bad ? qnan : (float)kt;
  p.out[row] = r.bad ? qnan : (float)((double)p.beta * kt + (1.0 - (double)p.beta) * ks);
}


template <int DT, bool VEC>
__global__ __launch_bounds__(kJsdBlock) void jsd_div_kernel(JsdArgs p) {
  constexpr int NW = kJsdBlock / 64;
  constexpr int U = kJsdU;
  __shared__ float red[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t parts = p.parts;
  const int64_t total = p.N * parts;
  const int32_t G = (int32_t)((p.V + 7) / 8);
  const int32_t g_full = VEC ? (int32_t)(p.V / 8) : 0;
  const int32_t V = (int32_t)p.V;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, parts);
    const int32_t part = (int32_t)(vb - row * parts);
    const int32_t g0 = part * p.groups_per_part;
    const int32_t g1 = min(G, g0 + p.groups_per_part);
    const JsdRow r = jsd_row(p.st4 + 4 * row, p.beta);
    const char* rs = row_ptr<DT>(p.s, row);
    const char* rt = row_ptr<DT>(p.t, row);
    float Ks = 0.0f, Kt = 0.0f;  // base-2 sums; scaled by ln 2 once per row
    auto accumulate = [&](const float (&xs)[8], const float (&xt)[8]) {
      JsdGroup q;
      jsd_group<false>(r, xs, xt, q);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Ks += mul0(q.ps[j], q.us[j] - q.lm[j]);
        Kt += mul0(q.pt[j], q.ut[j] - q.lm[j]);
      }
    };
    int32_t gb = g0 + tid;
    // whole vector groups of every lane: no predicates
    const int32_t nfull = VEC ? (min(g1, g_full) - g0) / (kJsdBlock * U) : 0;
    for (int32_t it = 0; it < nfull; ++it, gb += kJsdBlock * U) {
      // all of the batch's loads in flight before any is used
      if constexpr (DT == kF32) {
        F32Span ws_[U], wt_[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          ws_[k] = load_span_f32(rs, gb - lane + k * kJsdBlock, lane);
          wt_[k] = load_span_f32(rt, gb - lane + k * kJsdBlock, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          float xs[8], xt[8];
          span_to_group(ws_[k], lane, xs);
          span_to_group(wt_[k], lane, xt);
          accumulate(xs, xt);
        }
      } else {
        RawGroup<DT> ws_[U], wt_[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          load_group_raw<DT>(rs, gb + k * kJsdBlock, ws_[k]);
          load_group_raw<DT>(rt, gb + k * kJsdBlock, wt_[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          float xs[8], xt[8];
          raw_to_float<DT>(ws_[k], xs);
          raw_to_float<DT>(wt_[k], xt);
          accumulate(xs, xt);
        }
      }
    }
    for (; gb < g1; gb += kJsdBlock * U) {
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int32_t g = gb + k * kJsdBlock;
        if (g < g1) {
          float xs[8], xt[8];
          load_group<DT, VEC>(rs, g, V, g_full, xs);
          load_group<DT, VEC>(rt, g, V, g_full, xt);
          accumulate(xs, xt);
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      Ks += __shfl_xor(Ks, off, 64);
      Kt += __shfl_xor(Kt, off, 64);
    }
    if (lane == 0) {
      red[0][wave] = Ks;
      red[1][wave] = Kt;
    }
    __syncthreads();
    if (tid == 0) {
      float s = red[0][0], t = red[1][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        s += red[0][w];
        t += red[1][w];
      }
      if (parts == 1) {
        jsd_finalize(p, row, s, t);
      } else {
        p.ws2[2 * vb] = s;
        p.ws2[2 * vb + 1] = t;
      }
    }
    __syncthreads();  // red[] is reused by the next row
  }
}

// One thread per row: add the parts' sums in part order, then finalize.
__global__ __launch_bounds__(256) void jsd_combine_kernel(JsdArgs p) {
  for (int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x; row < p.N; row += (int64_t)gridDim.x * 256) {
    const float* w = p.ws2 + 2 * row * p.parts;
    float Ks = 0.0f, Kt = 0.0f;
    for (int i = 0; i < p.parts; ++i) {
      Ks += w[2 * i];
      Kt += w[2 * i + 1];
    }
    jsd_finalize(p, row, Ks, Kt);
  }
}

// ---- backward ---------------------------------------------------------------------------

template <int DT, bool FULL>
__device__ __forceinline__ void jsd_bwd_groups(const JsdRow& r, float Ks, float Kt, float gs, float gt,
                                               const char* rs, const char* rt, char* os, char* ot, int32_t g,
                                               int n, int32_t G, int32_t V, int32_t g_full) {
  const float qnan = __builtin_nanf("");
  for (int u = 0; u < n; ++u, g += kJsdBlock) {
    if (!FULL && g >= G) break;
    float xs[8], xt[8], ys[8], yt[8];
    if (FULL) {
      load_group_vec<DT>(rs, g, xs);
      load_group_vec<DT>(rt, g, xt);
    } else {
      load_group<DT, true>(rs, g, V, g_full, xs);
      load_group<DT, true>(rt, g, V, g_full, xt);
    }
    JsdGroup q;
    jsd_group<true>(r, xs, xt, q);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // (log p - log M) - K in natural units: ln 2 (u - l) - K
      ys[j] = r.bad ? qnan : (mul0(q.ps[j], __builtin_fmaf(kLn2, q.us[j] - q.lm[j], -Ks)) * gs) * q.fs[j];
      yt[j] = r.bad ? qnan : (mul0(q.pt[j], __builtin_fmaf(kLn2, q.ut[j] - q.lm[j], -Kt)) * gt) * q.ft[j];
    }
    if (FULL) {
      if (os) store_group_vec<DT>(os, g, ys);
      if (ot) store_group_vec<DT>(ot, g, yt);
    } else {
      if (os) store_group<DT, true>(os, g, V, g_full, ys);
      if (ot) store_group<DT, true>(ot, g, V, g_full, yt);
    }
  }
}

// A whole fp32 tile (kJsdTileF32 groups): the gradients are elementwise (jsd_group decides its
// recomputed mixtures per element), so lane l takes the tile's 16-byte pieces l, l + 256, ...
// instead of its groups of 8 columns, and every load and store of a wave covers one contiguous
// 1 KB. Two pieces form the 8 values one jsd_group call works on.
__device__ __forceinline__ void jsd_bwd_tile_f32(const JsdRow& r, float Ks, float Kt, float gs, float gt,
                                                 const char* rs, const char* rt, char* os, char* ot, int32_t g0) {
  constexpr int NP = 2 * kJsdTileF32 / kJsdBlock;  // pieces per lane
  static_assert(NP % 2 == 0, "pieces go to jsd_group in pairs");
  const int64_t q0 = 2 * (int64_t)g0 + threadIdx.x;
  const float qnan = __builtin_nanf("");
  f32x4 ps[NP], pt[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    ps[k] = stream_load(reinterpret_cast<const f32x4*>(rs) + q0 + k * kJsdBlock);
    pt[k] = stream_load(reinterpret_cast<const f32x4*>(rt) + q0 + k * kJsdBlock);
  }
#pragma unroll
  for (int k = 0; k < NP; k += 2) {
    float xs[8], xt[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xs[e] = ps[k][e];
      xs[4 + e] = ps[k + 1][e];
      xt[e] = pt[k][e];
      xt[4 + e] = pt[k + 1][e];
    }
    JsdGroup q;
    jsd_group<true>(r, xs, xt, q);
    f32x4 ys[2], yt[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ys[j >> 2][j & 3] = r.bad ? qnan : (mul0(q.ps[j], __builtin_fmaf(kLn2, q.us[j] - q.lm[j], -Ks)) * gs) * q.fs[j];
      yt[j >> 2][j & 3] = r.bad ? qnan : (mul0(q.pt[j], __builtin_fmaf(kLn2, q.ut[j] - q.lm[j], -Kt)) * gt) * q.ft[j];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (os) stream_store(ys[h], reinterpret_cast<f32x4*>(os) + q0 + (k + h) * kJsdBlock);
      if (ot) stream_store(yt[h], reinterpret_cast<f32x4*>(ot) + q0 + (k + h) * kJsdBlock);
    }
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kJsdBlock) void jsd_bwd_kernel(JsdArgs p) {
  constexpr int ES = ElemSize<DT>::value;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = VEC ? V / 8 : 0;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, tpr);
    const int32_t tile = (int32_t)(vb - row * tpr);
    constexpr int TG = DT == kF32 ? kJsdTileF32 : kJsdBlock * kJsdUB;  // groups per tile
    const int32_t g0 = tile * TG;
    const float* st = p.stats + 6 * row;
    JsdRow r = jsd_row(st, p.beta);
    const float Ks = st[4], Kt = st[5];
    r.bad = r.bad || !(Ks == Ks) || !(Kt == Kt);
    const float gv = p.g[row * p.g_stride];
    const float gs = gv * r.ws, gt = gv * r.wt;
    const char* rs = row_ptr<DT>(p.s, row);
    const char* rt = row_ptr<DT>(p.t, row);
    char* os = p.ds ? p.ds + row * (int64_t)V * ES : nullptr;
    char* ot = p.dt ? p.dt + row * (int64_t)V * ES : nullptr;
    const int32_t g = g0 + threadIdx.x;
    if (DT == kF32 && VEC && g0 + TG <= g_full)
      jsd_bwd_tile_f32(r, Ks, Kt, gs, gt, rs, rt, os, ot, g0);
    else if (DT != kF32 && VEC && g0 + TG <= g_full)
      jsd_bwd_groups<DT, true>(r, Ks, Kt, gs, gt, rs, rt, os, ot, g, kJsdUB, G, V, g_full);
    else  // this tile's groups only (fp32 tiles are narrower than kJsdUB groups a lane)
      jsd_bwd_groups<DT, false>(r, Ks, Kt, gs, gt, rs, rt, os, ot, g, kJsdUB, min(G, g0 + TG), V, g_full);
  }
}

// ---- host-side launch -------------------------------------------------------------------

int32_t jsd_tiles_per_row(int64_t V, int dtype) {
  const int64_t G = (V + 7) / 8;
  const int64_t per = dtype == kF32 ? kJsdTileF32 : kJsdBlock * kJsdUB;
  return (int32_t)((G + per - 1) / per);
}

hipError_t launch_jsd_div(const JsdArgs& p, int dtype, bool vec, hipStream_t stream) {
  const dim3 grid((uint32_t)grid_cap(p.N * p.parts)), block(kJsdBlock);
  hipError_t e = dispatch_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (vec) hipLaunchKernelGGL((jsd_div_kernel<DT, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((jsd_div_kernel<DT, false>), grid, block, 0, stream, p);
    return hipGetLastError();
  });
  if (e != hipSuccess || p.parts == 1) return e;
  hipLaunchKernelGGL(jsd_combine_kernel, dim3((uint32_t)grid_cap((p.N + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_jsd_bwd(const JsdArgs& p, int dtype, bool vec, hipStream_t stream) {
  const dim3 grid((uint32_t)grid_cap(p.N * p.tiles_per_row)), block(kJsdBlock);
  return dispatch_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (vec) hipLaunchKernelGGL((jsd_bwd_kernel<DT, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((jsd_bwd_kernel<DT, false>), grid, block, 0, stream, p);
    return hipGetLastError();
  });
}

}  // namespace vws
