// device.h -- device-side building blocks of libvws (gfx950, wave64).
//
// Running statistics of one row (or one part of a row), after DeepSpeed PR
// #8838 "Add Triton kernels for vocab-parallel logprobs, entropy and KL"
// (second commit message; the review comment proposing a single read):
//   m  running max,  S = sum e^(z - m),  W = sum e^(z - m) (z - m)
// and for KL(A||B) the pair (m_a, S_A), (m_b, S_B) with
//   W = sum e^(a - m_a) ((a - m_a) - (b - m_b))
// plus the support flag F (some column with a > -inf and b = -inf).
//
// When the max grows from m to M, S <- s S and W <- s (W + (m - M) S) with
// s = e^(m - M); parts are merged the same way after taking the larger max.
// Zero-weight rule (the review thread on 0 x inf in the rescaling, and its fix
// commit): a term or a part whose weight is
// exactly 0 contributes nothing, never 0 x inf. It is implemented with
// v_mul_legacy_f32, whose product is 0 whenever either factor is 0 (also
// against inf and NaN).
//
// Conventions of a running state:
// - m is the max of the values seen (NaN ignored); -inf while no value above
//   -inf has been seen.
// - S and W are centred on ref = m, or on 0 while m = -inf (then S = 0 and
//   W = 0 unless a NaN was seen).
// - The logits ops keep S and W multiplied by 2^64: a term e^(z - m) below
//   2^-126 (a column 87.3 to 131.7 nats below the max) is then still a normal
//   number. v_exp_f32 returns 0 for results below 2^-126, and such terms are
//   what H and KL are made of on a row that is one-hot up to a far tail. The
//   scale rides on the exponent argument (exp_scaled: one fma where the
//   unscaled form has one multiply); merges and rescales multiply by the
//   scaled exponential and by 2^-64, which leaves an unscaled state unscaled
//   too; finalization divides the scale out in double precision.
// - A NaN input always reaches S (e^(NaN) = NaN, and 0 * NaN = NaN in the
//   plain products used for S), so S carries "row undefined" to the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vws {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kInf = __builtin_inff();

enum Dtype : int { kF32 = 0, kBF16 = 1, kF16 = 2 };
enum Op : int { kLogprobs = 0, kEntropy = 1, kKL = 2 };

// Cache policy of the streaming accesses: the logits are read once and the
// gradients written once, so both default to non-temporal. (Compile-time
// switches, so launch-shape and policy sweeps can rebuild the same kernels.)
#ifndef VWS_NT_LOAD
#define VWS_NT_LOAD 1
#endif
#ifndef VWS_NT_STORE
#define VWS_NT_STORE 1
#endif

template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
#if VWS_NT_LOAD
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void stream_store(T v, T* p) {
#if VWS_NT_STORE
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

extern "C" __device__ float vws_llvm_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");

// a * b, but exactly 0 when a or b is 0 (even if the other is inf or NaN).
__device__ __forceinline__ float mul0(float a, float b) { return vws_llvm_fmul_legacy(a, b); }

// e^x through the hardware base-2 exponential (v_exp_f32). Results below 2^-126 come out as 0:
// used where such a term is negligible against the sum it joins (the forward statistics).
__device__ __forceinline__ float expf_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

constexpr float kSumScaleLog2 = 64.0f;  // the running sums' scale 2^64, as an exponent
constexpr float kSumUnscale = 0x1p-64f;

// 2^64 e^d for d <= 0: exact for d = 0, a normal number down to d = -131.7 nats.
__device__ __forceinline__ float exp_scaled(float d) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(d, kLog2e, kSumScaleLog2));
}

// log of a running sum S kept at the 2^64 scale: the scale is divided out exactly in double.
__device__ __forceinline__ double log_unscaled(float S) { return log((double)S * 0x1p-64); }

// e^x for gradients as a pair (p, f) with e^x = p f, p = 2^64 e^x and f = 2^-64: a probability
// below 2^-126, where v_exp_f32 returns 0 but bf16 still holds the gradient (down to 2^-133, and
// far above that once multiplied by g and a log-probability), is a normal number at that scale.
// A caller forms its whole product with p and multiplies by f last, so the result is rounded once
// at its own magnitude. The scale rides on the exponent argument (one fma where the unscaled
// form has one multiply): rounding that argument near 64 costs up to 2^-18 ln 2 relative in p,
// far inside the fp32 2e-5 bound, and one multiply by f per gradient. Choosing the scale per
// element instead cost the KL backward 5% and the top-k backward 13%.
struct PScaled {
  float p, f;
};
__device__ __forceinline__ PScaled exp_split(float x) {
  return PScaled{__builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, kSumScaleLog2)), kSumUnscale};
}

template <int DT>
struct ElemSize {
  static constexpr int value = DT == kF32 ? 4 : 2;
};

__device__ __forceinline__ float bf16_bits_to_float(uint32_t hi16) { return __uint_as_float(hi16 << 16); }

// ---- loads of one group of 8 consecutive columns ---------------------------
// Group g of a row covers columns [8g, 8g + 8). The vector form needs the row
// start 16-byte aligned and the whole group inside the row.

// The same load split in two: the raw 16-byte words of a group (issued now), and their
// conversion to fp32 (done later), so that a kernel can put several groups' loads in flight
// before it uses any of them.
template <int DT>
struct RawGroup {
  u32x4 w[DT == kF32 ? 2 : 1];
};

template <int DT>
__device__ __forceinline__ void load_group_raw(const char* __restrict__ row, int32_t g, RawGroup<DT>& r) {
  if constexpr (DT == kF32) {
    const u32x4* p = reinterpret_cast<const u32x4*>(row) + 2 * g;
    r.w[0] = stream_load(p);
    r.w[1] = stream_load(p + 1);
  } else {
    r.w[0] = stream_load(reinterpret_cast<const u32x4*>(row) + g);
  }
}

template <int DT>
__device__ __forceinline__ void raw_to_float(const RawGroup<DT>& r, float (&x)[8]) {
  if constexpr (DT == kF16) {
    const f16x8 h = __builtin_bit_cast(f16x8, r.w[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)h[k];
  } else if constexpr (DT == kBF16) {
    const u32x4 w = r.w[0];
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xffff0000u);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = __uint_as_float(r.w[0][k]);
      x[4 + k] = __uint_as_float(r.w[1][k]);
    }
  }
}

template <int DT>
__device__ __forceinline__ void load_group_vec(const char* __restrict__ row, int32_t g, float (&x)[8]) {
  if constexpr (DT == kF16) {
    const f16x8 h = __builtin_bit_cast(f16x8, stream_load(reinterpret_cast<const u32x4*>(row) + g));
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (float)h[k];
  } else if constexpr (DT == kBF16) {
    u32x4 w = stream_load(reinterpret_cast<const u32x4*>(row) + g);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16);
    x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16);
    x[7] = __uint_as_float(w.w & 0xffff0000u);
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(row) + 2 * g;
    f32x4 a = stream_load(p);
    f32x4 b = stream_load(p + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* __restrict__ row, int64_t col) {
  if constexpr (DT == kF16) {
    return (float)reinterpret_cast<const _Float16*>(row)[col];
  } else if constexpr (DT == kBF16) {
    return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(row)[col]);
  } else {
    return reinterpret_cast<const float*>(row)[col];
  }
}

// Element-wise form: columns at or beyond V read as -inf (zero weight).
template <int DT>
__device__ __forceinline__ void load_group_scalar(const char* __restrict__ row, int32_t g, int32_t V, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int32_t c = 8 * g + k;
    x[k] = c < V ? load_elem<DT>(row, c) : -kInf;
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void load_group(const char* __restrict__ row, int32_t g, int32_t V, int32_t g_full,
                                           float (&x)[8]) {
  if (VEC && g < g_full) {
    load_group_vec<DT>(row, g, x);
  } else {
    load_group_scalar<DT>(row, g, V, x);
  }
}

// ---- stores of one group of 8 gradient values (contiguous output rows) -------

template <int DT>
__device__ __forceinline__ void store_group_vec(char* __restrict__ row, int32_t g, const float (&y)[8]) {
  if constexpr (DT == kF16) {
    u32x4 w;
    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[0], y[1]}, f16x2));
    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[2], y[3]}, f16x2));
    w.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[4], y[5]}, f16x2));
    w.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[6], y[7]}, f16x2));
    stream_store(w, reinterpret_cast<u32x4*>(row) + g);
  } else if constexpr (DT == kBF16) {
    u32x4 w;
    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[0], y[1]}, bf16x2));
    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[2], y[3]}, bf16x2));
    w.z = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[4], y[5]}, bf16x2));
    w.w = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[6], y[7]}, bf16x2));
    stream_store(w, reinterpret_cast<u32x4*>(row) + g);
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(row) + 2 * g;
    stream_store((f32x4){y[0], y[1], y[2], y[3]}, p);
    stream_store((f32x4){y[4], y[5], y[6], y[7]}, p + 1);
  }
}

template <int DT>
__device__ __forceinline__ void store_elem(char* __restrict__ row, int64_t col, float y) {
  if constexpr (DT == kF16) {
    reinterpret_cast<_Float16*>(row)[col] = (_Float16)y;
  } else if constexpr (DT == kBF16) {
    bf16x2 h = __builtin_convertvector((f32x2){y, 0.0f}, bf16x2);
    reinterpret_cast<uint16_t*>(row)[col] = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xffffu);
  } else {
    reinterpret_cast<float*>(row)[col] = y;
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void store_group(char* __restrict__ row, int32_t g, int32_t V, int32_t g_full,
                                            const float (&y)[8]) {
  if (VEC && g < g_full) {
    store_group_vec<DT>(row, g, y);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int32_t c = 8 * g + k;
      if (c < V) store_elem<DT>(row, c, y[k]);
    }
  }
}

// ---- running states ----------------------------------------------------------

// Reference a state's S and W are centred on: m, or 0 while m = -inf.
__device__ __forceinline__ float ref_of(float m) { return m == -kInf ? 0.0f : m; }

struct State1 {  // logprobs (W unused) and entropy
  float m, S, W;
};

struct StateKL {
  float ma, Sa, mb, Sb, W;
  uint32_t F;
};

__device__ __forceinline__ State1 state1_init() { return State1{-kInf, 0.0f, 0.0f}; }
__device__ __forceinline__ StateKL statekl_init() { return StateKL{-kInf, 0.0f, -kInf, 0.0f, 0.0f, 0u}; }

// Merge two single-input states (commutative bit for bit).
template <bool WITH_W>
__device__ __forceinline__ State1 merge1(const State1& x, const State1& y) {
  const float M = fmaxf(x.m, y.m);
  const float R = ref_of(M);
  const float dx = x.m - R, dy = y.m - R;  // -inf for an empty part, or on overflow
  const float sx = exp_scaled(dx), sy = exp_scaled(dy);
  State1 r;
  r.m = M;
  r.S = sx * (x.S * kSumUnscale) + sy * (y.S * kSumUnscale);
  r.W = WITH_W ? mul0(sx, (x.W + dx * x.S) * kSumUnscale) + mul0(sy, (y.W + dy * y.S) * kSumUnscale) : 0.0f;
  return r;
}

// Merge two KL states: both maxima re-centred, S_B on its own, F by OR.
__device__ __forceinline__ StateKL merge_kl(const StateKL& x, const StateKL& y) {
  const float Ma = fmaxf(x.ma, y.ma), Mb = fmaxf(x.mb, y.mb);
  const float Ra = ref_of(Ma), Rb = ref_of(Mb);
  const float dax = x.ma - Ra, day = y.ma - Ra;
  const float sax = exp_scaled(dax), say = exp_scaled(day);
  const float sbx = exp_scaled(x.mb - Rb), sby = exp_scaled(y.mb - Rb);
  // W_i is centred on (ref(m_a,i), ref(m_b,i)); shifting both references:
  // W' = s_a,i (W_i + ((m_a,i - Ra) - (ref(m_b,i) - Rb)) S_A,i)
  const float shx = dax - (ref_of(x.mb) - Rb), shy = day - (ref_of(y.mb) - Rb);
  StateKL r;
  r.ma = Ma;
  r.mb = Mb;
  r.Sa = sax * (x.Sa * kSumUnscale) + say * (y.Sa * kSumUnscale);
  r.Sb = sbx * (x.Sb * kSumUnscale) + sby * (y.Sb * kSumUnscale);
  r.W = mul0(sax, (x.W + shx * x.Sa) * kSumUnscale) + mul0(say, (y.W + shy * y.Sa) * kSumUnscale);
  r.F = x.F | y.F;
  return r;
}

// ---- cross-lane / cross-wave reductions -----------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

template <bool WITH_W>
__device__ __forceinline__ State1 wave_reduce1(State1 s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    State1 o;
    o.m = shfl_xor_f(s.m, off);
    o.S = shfl_xor_f(s.S, off);
    o.W = WITH_W ? shfl_xor_f(s.W, off) : 0.0f;
    s = merge1<WITH_W>(s, o);
  }
  return s;
}

__device__ __forceinline__ StateKL wave_reduce_kl(StateKL s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    StateKL o;
    o.ma = shfl_xor_f(s.ma, off);
    o.Sa = shfl_xor_f(s.Sa, off);
    o.mb = shfl_xor_f(s.mb, off);
    o.Sb = shfl_xor_f(s.Sb, off);
    o.W = shfl_xor_f(s.W, off);
    o.F = (uint32_t)__shfl_xor((int)s.F, off, 64);
    s = merge_kl(s, o);
  }
  return s;
}

// ---- row addressing ---------------------------------------------------------------

struct RowsDev {
  const char* data;
  int64_t n_inner, s_outer, s_inner;  // strides in elements
};

struct IdsDev {
  const int64_t* data;
  int64_t s_outer, s_inner;
};

// a / b for a >= 0 and b >= 1. The callers' operands are almost always wave-uniform and
// below 2^32, where the 32-bit sequence replaces the much longer 64-bit one.
__device__ __forceinline__ int64_t udiv(int64_t a, int64_t b) {
  if (b == 1) return a;
  if (((uint64_t)a | (uint64_t)b) <= 0xffffffffull) return (int64_t)((uint32_t)a / (uint32_t)b);
  return a / b;
}

template <int DT>
__device__ __forceinline__ const char* row_ptr(const RowsDev& r, int64_t row) {
  const int64_t ro = udiv(row, r.n_inner), ri = row - ro * r.n_inner;
  return r.data + (ro * r.s_outer + ri * r.s_inner) * ElemSize<DT>::value;
}

__device__ __forceinline__ int64_t load_id(const IdsDev& t, int64_t row, int64_t n_inner) {
  const int64_t ro = udiv(row, n_inner), ri = row - ro * n_inner;
  return t.data[ro * t.s_outer + ri * t.s_inner];
}

}  // namespace vws
