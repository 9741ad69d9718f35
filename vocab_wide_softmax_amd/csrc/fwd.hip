// fwd.hip -- single-read forward of logprobs, entropy and KL(A||B).
//
// One workgroup of 512 lanes (large batches in the automatic split) or 256
// streams one row (or one vocabulary part of one row). Each
// lane keeps the running state of device.h over the groups of 8 columns it
// owns: group g of part [g0, g1) belongs to lane (g - g0) mod BLOCK, and a
// lane takes its groups in increasing order, U groups per batch. The element
// to lane map and the order of operations do not depend on the dtype (whole
// fp32 batches are loaded coalesced and handed back to the same lanes,
// span_f32.h), so bf16 and fp32 inputs holding the same values give
// bit-identical results (the review comment on PR #8838 reports the same
// property for its patched kernels). A logprobs row reads its target logits
// (one id, or up to 256 top-k slots) before its stream and writes the
// log-probabilities after the merge.
//
// Per batch the lane takes the batch max first and rescales its state once
// (second commit message of PR #8838: when the max grows, the weighted sum is
// rescaled like the sum-exp), then accumulates e = exp(z - m),
// S += e, W += e (z - m) with the zero-weight product (S and W at the 2^64
// scale of device.h). Lanes are merged by a
// butterfly over the wave, waves through LDS in wave order ("lane
// re-centring", fix commit of the 0 x inf thread).
//
// With P > 1 parts per row the workgroup writes its part's state to the
// workspace and combine_kernel merges the parts in part order and finalizes:
// the pages' MAX / re-centre / SUM across tensor-parallel shards, done inside
// one GPU.
#include "device.h"
#include "launch.h"
#include "span_f32.h"

namespace vws {

// ---- per-batch updates -------------------------------------------------------

template <bool WITH_W, int U>
__device__ __forceinline__ void update1(State1& st, const float (&x)[U][8]) {
  float bm = -kInf;
#pragma unroll
  for (int k = 0; k < U; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) bm = fmaxf(bm, x[k][j]);
  if (bm > st.m) {
    const float d = st.m - bm;  // -inf when the state is empty
    const float s = exp_scaled(d);
    if (WITH_W) st.W = mul0(s, (st.W + d * st.S) * kSumUnscale);
    st.S = s * (st.S * kSumUnscale);
    st.m = bm;
  }
  const float ref = ref_of(st.m);
#pragma unroll
  for (int k = 0; k < U; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = x[k][j] - ref;
      const float e = exp_scaled(d);  // 2^64 e^d
      st.S += e;
      if (WITH_W) st.W += mul0(e, d);
    }
}

template <int U>
__device__ __forceinline__ void update_kl(StateKL& st, const float (&xa)[U][8], const float (&xb)[U][8]) {
  float bma = -kInf, bmb = -kInf, bminb = kInf;
#pragma unroll
  for (int k = 0; k < U; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bma = fmaxf(bma, xa[k][j]);
      bmb = fmaxf(bmb, xb[k][j]);
      bminb = fminf(bminb, xb[k][j]);
    }
  const bool ga = bma > st.ma, gb = bmb > st.mb;
  if (ga || gb) {
    // W holds e_a ((a - ref_a) - (b - ref_b)). Moving the references to the new maxima scales
    // e_a by s = e^(ma - ma') and shifts every bracket by (ref_a - ref_a') - (ref_b - ref_b');
    // both shifts are applied as one difference, so identical inputs (A = B) keep W exactly 0.
    const float nma = ga ? bma : st.ma, nmb = gb ? bmb : st.mb;
    const float sh = (ref_of(st.ma) - ref_of(nma)) - (ref_of(st.mb) - ref_of(nmb));
    if (ga) {
      const float s = exp_scaled(st.ma - nma);  // 0 when the state was empty
      st.W = mul0(s, (st.W + sh * st.Sa) * kSumUnscale);
      st.Sa = s * (st.Sa * kSumUnscale);
    } else {
      st.W += sh * st.Sa;
    }
    if (gb) st.Sb = exp_scaled(st.mb - nmb) * (st.Sb * kSumUnscale);
    st.ma = nma;
    st.mb = nmb;
  }
  if (bminb == -kInf) {  // some B entry is masked: decide the support flag on the logits
    uint32_t f = 0;
#pragma unroll
    for (int k = 0; k < U; ++k)
#pragma unroll
      for (int j = 0; j < 8; ++j) f |= (xa[k][j] > -kInf) & (xb[k][j] == -kInf);
    st.F |= f;
  }
  const float ra = ref_of(st.ma), rb = ref_of(st.mb);
#pragma unroll
  for (int k = 0; k < U; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float da = xa[k][j] - ra;
      const float db = xb[k][j] - rb;
      const float ea = exp_scaled(da);
      const float eb = exp_scaled(db);
      st.Sa += ea;
      st.Sb += eb;
      st.W += mul0(ea, da - db);
    }
}

// ---- finalization of a row from its merged state ----------------------------------

__device__ __forceinline__ double log_d(float S) { return log_unscaled(S); }

// The target of a logprobs row, read before the row's stream and used after its merge: zt is the
// target logit, NaN for an id outside [0, V); ign marks the ignored id.
struct Target {
  float zt;
  bool ign;
};

template <int DT>
__device__ __forceinline__ Target load_target(const FwdArgs& p, const char* ra, int64_t row, int32_t k) {
  const int64_t ro = udiv(row, p.a.n_inner), ri = row - ro * p.a.n_inner;
  const int64_t t = p.ids.data[ro * p.ids.s_outer + ri * p.ids.s_inner + (int64_t)k * p.ids_sk];
  Target r{__builtin_nanf(""), t == p.ignore_index};
  if (!r.ign && t >= 0 && t < p.V) r.zt = load_elem<DT>(ra, t);
  return r;
}

__device__ __forceinline__ float logp_of(const Target& t, float m, double logS) {
  return t.ign ? 0.0f : (float)(((double)t.zt - (double)m) - logS);
}

// Writes the row's statistics and, with one id per row, its log-probability (tgt: the target read
// before the stream, or nullptr to read it here). Returns log S as stored.
template <int DT>
__device__ float finalize1_logprobs(const FwdArgs& p, int64_t row, const State1& st, const Target* tgt = nullptr) {
  const double logS = log_d(st.S);
  p.stats[2 * row + 0] = st.m;
  p.stats[2 * row + 1] = (float)logS;
  if (p.out != nullptr && p.K == 0) {  // else statistics only, or the K slots written after the merge
    const Target t = tgt ? *tgt : load_target<DT>(p, row_ptr<DT>(p.a, row), row, 0);
    p.out[row] = logp_of(t, st.m, logS);
  }
  return (float)logS;
}

__device__ __forceinline__ void finalize1_entropy(const FwdArgs& p, int64_t row, const State1& st) {
  const double logS = log_d(st.S);
  p.stats[2 * row + 0] = st.m;
  p.stats[2 * row + 1] = (float)logS;
  p.out[row] = (float)(logS - (double)st.W / (double)st.S);
}

__device__ __forceinline__ void finalize_kl(const FwdArgs& p, int64_t row, const StateKL& st) {
  const double lsa = log_d(st.Sa), lsb = log_d(st.Sb);
  p.stats[4 * row + 0] = st.ma;
  p.stats[4 * row + 1] = (float)lsa;
  p.stats[4 * row + 2] = st.mb;
  p.stats[4 * row + 3] = (float)lsb;
  if (p.out == nullptr) return;  // statistics only (the JSD statistics pass)
  float out;
  if (!(st.Sa > 0.0f) || st.Sb != st.Sb) {  // A has no live entry, or a NaN / +inf reached S
    out = __builtin_nanf("");
  } else if (st.F) {
    out = kInf;
  } else {
    out = (float)((double)st.W / (double)st.Sa - lsa + lsb);
  }
  p.out[row] = out;
}

// ---- the streaming kernel -----------------------------------------------------------

template <int OP, int DT, bool VEC, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void fwd_kernel(FwdArgs p) {
  constexpr int NW = BLOCK / 64;
  const int32_t parts = p.parts;
  const int64_t total = p.N * parts;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
  const int64_t row = udiv(vb, parts);
  const int32_t part = (int32_t)(vb - row * parts);
  const int32_t G = (int32_t)((p.V + 7) / 8);
  const int32_t g_full = (int32_t)(p.V / 8);
  const int32_t V = (int32_t)p.V;
  const int32_t g0 = part * p.groups_per_part;
  const int32_t g1 = min(G, g0 + p.groups_per_part);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const char* ra = row_ptr<DT>(p.a, row);

  if constexpr (OP == kKL) {
    const char* rb = row_ptr<DT>(p.b, row);
    StateKL st = statekl_init();
    int32_t gb = g0 + tid;
    // batches in which every group of every lane is a full vector group: no predicates
    const int32_t nfull = VEC ? (min(g1, g_full) - g0) / (BLOCK * U) : 0;
    for (int32_t it = 0; it < nfull; ++it, gb += BLOCK * U) {
      // all of the batch's loads in flight before any is used (one latency per batch)
      float xa[U][8], xb[U][8];
      if constexpr (DT == kF32) {
        F32Span wa[U], wb[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          wa[k] = load_span_f32(ra, gb - lane + k * BLOCK, lane);
          wb[k] = load_span_f32(rb, gb - lane + k * BLOCK, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          span_to_group(wa[k], lane, xa[k]);
          span_to_group(wb[k], lane, xb[k]);
        }
      } else {
        RawGroup<DT> wa[U], wb[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          load_group_raw<DT>(ra, gb + k * BLOCK, wa[k]);
          load_group_raw<DT>(rb, gb + k * BLOCK, wb[k]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < U; ++k) {
          raw_to_float<DT>(wa[k], xa[k]);
          raw_to_float<DT>(wb[k], xb[k]);
        }
      }
      update_kl<U>(st, xa, xb);
    }
    // the rest of the part (same batch boundaries), groups predicated
    for (; gb < g1; gb += BLOCK * U) {
      float xa[U][8], xb[U][8];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int32_t g = gb + k * BLOCK;
        if (g < g1) {
          load_group<DT, VEC>(ra, g, V, g_full, xa[k]);
          load_group<DT, VEC>(rb, g, V, g_full, xb[k]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) xa[k][j] = xb[k][j] = -kInf;
        }
      }
      update_kl<U>(st, xa, xb);
    }
    st = wave_reduce_kl(st);
    __shared__ StateKL red[NW];
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0) {
      StateKL s = red[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) s = merge_kl(s, red[w]);
      if (parts == 1) {
        finalize_kl(p, row, s);
      } else {
        float* o = p.ws + vb * 6;
        o[0] = s.ma; o[1] = s.Sa; o[2] = s.mb; o[3] = s.Sb; o[4] = s.W; o[5] = (float)s.F;
      }
    }
  } else {
    constexpr bool WW = OP == kEntropy;
    // logprobs, unsplit: the row's target logits (one, or K slots over the first K lanes) are
    // loaded before the stream, so the row ends without a dependent load
    const int32_t nslot = OP == kLogprobs && parts == 1 && p.out != nullptr ? (p.K > 0 ? p.K : 1) : 0;
    Target tg{0.0f, true};
    if (tid < nslot) tg = load_target<DT>(p, ra, row, tid);
    State1 st = state1_init();
    int32_t gb = g0 + tid;
    const int32_t nfull = VEC ? (min(g1, g_full) - g0) / (BLOCK * U) : 0;
    for (int32_t it = 0; it < nfull; ++it, gb += BLOCK * U) {
      float x[U][8];
      if constexpr (DT == kF32) {
        F32Span w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) w[k] = load_span_f32(ra, gb - lane + k * BLOCK, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < U; ++k) span_to_group(w[k], lane, x[k]);
      } else {
#pragma unroll
        for (int k = 0; k < U; ++k) load_group_vec<DT>(ra, gb + k * BLOCK, x[k]);
      }
      update1<WW, U>(st, x);
    }
    for (; gb < g1; gb += BLOCK * U) {
      float x[U][8];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int32_t g = gb + k * BLOCK;
        if (g < g1) {
          load_group<DT, VEC>(ra, g, V, g_full, x[k]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[k][j] = -kInf;
        }
      }
      update1<WW, U>(st, x);
    }
    st = wave_reduce1<WW>(st);
    __shared__ State1 red[NW];
    __shared__ float row_ml[2];  // (m, log S) of the row for the K-slot outputs
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0) {
      State1 s = red[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) s = merge1<WW>(s, red[w]);
      if (parts == 1) {
        if (OP == kEntropy) {
          finalize1_entropy(p, row, s);
        } else {
          row_ml[1] = finalize1_logprobs<DT>(p, row, s, &tg);
          row_ml[0] = s.m;
        }
      } else {
        float* o = p.ws + vb * 3;
        o[0] = s.m; o[1] = s.S; o[2] = s.W;
      }
    }
    if (OP == kLogprobs && p.K > 0 && nslot > 0) {
      __syncthreads();
      if (tid < nslot) p.out[row * p.K + tid] = logp_of(tg, row_ml[0], (double)row_ml[1]);
    }
  }
  __syncthreads();  // red[] and row_ml[] are reused by the next row
  }
}

// One thread per row: merge the row's parts in part order, then finalize.
template <int OP, int DT>
__global__ __launch_bounds__(256) void combine_kernel(FwdArgs p) {
  for (int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x; row < p.N; row += (int64_t)gridDim.x * 256) {
  if constexpr (OP == kKL) {
    const float* w = p.ws + row * p.parts * 6;
    StateKL s = statekl_init();
    for (int i = 0; i < p.parts; ++i, w += 6) {
      StateKL o{w[0], w[1], w[2], w[3], w[4], w[5] != 0.0f ? 1u : 0u};
      s = merge_kl(s, o);
    }
    finalize_kl(p, row, s);
  } else {
    constexpr bool WW = OP == kEntropy;
    const float* w = p.ws + row * p.parts * 3;
    State1 s = state1_init();
    for (int i = 0; i < p.parts; ++i, w += 3) s = merge1<WW>(s, State1{w[0], w[1], w[2]});
    if (OP == kEntropy) finalize1_entropy(p, row, s);
    else finalize1_logprobs<DT>(p, row, s);
  }
  }
}

// ---- host-side launch -----------------------------------------------------------------

namespace {
// Workgroup widths: 512 lanes (wide) or 256. The lane count fixes the element-to-lane map and so
// a row's rounding; the host picks it (fwd_wide in the ABI layer) from the split mode and N only.
constexpr int kFwdBlockWide = 512, kFwdBlockNarrow = 256;
// Groups of 8 columns per lane per batch: 4 for one input, 2 for KL's two (the same bytes
// in flight per batch; the fastest by measurement).
constexpr int fwd_u(int op) { return op == kKL ? 2 : 4; }

template <int OP, int DT, bool VEC, int BLOCK>
hipError_t launch_fwd_t(const FwdArgs& p, hipStream_t stream) {
  const int64_t blocks = grid_cap(p.N * p.parts);
  hipLaunchKernelGGL((fwd_kernel<OP, DT, VEC, BLOCK, fwd_u(OP)>), dim3((uint32_t)blocks), dim3(BLOCK), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.parts == 1) return e;
  hipLaunchKernelGGL((combine_kernel<OP, DT>), dim3((uint32_t)grid_cap((p.N + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int OP>
hipError_t launch_fwd_op(const FwdArgs& p, int dtype, bool vec, bool wide, hipStream_t stream) {
  return dispatch_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (wide)
      return vec ? launch_fwd_t<OP, DT, true, kFwdBlockWide>(p, stream)
                 : launch_fwd_t<OP, DT, false, kFwdBlockWide>(p, stream);
    return vec ? launch_fwd_t<OP, DT, true, kFwdBlockNarrow>(p, stream)
               : launch_fwd_t<OP, DT, false, kFwdBlockNarrow>(p, stream);
  });
}
}  // namespace

hipError_t launch_fwd(int op, const FwdArgs& p, int dtype, bool vec, bool wide, hipStream_t stream) {
  switch (op) {
    case kLogprobs: return launch_fwd_op<kLogprobs>(p, dtype, vec, wide, stream);
    case kEntropy: return launch_fwd_op<kEntropy>(p, dtype, vec, wide, stream);
    default: return launch_fwd_op<kKL>(p, dtype, vec, wide, stream);
  }
}

}  // namespace vws
