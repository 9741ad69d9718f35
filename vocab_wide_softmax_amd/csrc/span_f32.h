// span_f32.h -- coalesced loads of whole fp32 batches for the kernels that reduce over
// groups of 8 columns (the forward and the JSD divergence pass).
#pragma once

#include "device.h"

namespace vws {

// fp32 groups of whole batches, loaded coalesced. A group is 32 bytes, so a lane loading its own
// group's two 16-byte pieces makes each load of the wave cover every other piece of its 2 KB span.
// Instead lane l loads pieces l and 64 + l of the span (one contiguous 1 KB per load), and two
// exchanges give every lane its own group back: ds_permute sends piece s to lane s / 2 (even s)
// or 32 + (s - 1) / 2 (odd s), then v_permlane32_swap trades lanes 32-63 of the first result
// with lanes 0-31 of the second. Each lane ends up with the same 8 values as before, in order.
// gw: the wave's first group (its lanes hold groups gw .. gw + 63).
struct F32Span {
  f32x4 a, b;
};

__device__ __forceinline__ F32Span load_span_f32(const char* row, int32_t gw, int lane) {
  const f32x4* p = reinterpret_cast<const f32x4*>(row) + 2 * (int64_t)gw;
  return F32Span{stream_load(p + lane), stream_load(p + 64 + lane)};
}

__device__ __forceinline__ void span_to_group(const F32Span& w, int lane, float (&x)[8]) {
  const int dst = ((lane >> 1) + 32 * (lane & 1)) * 4;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int pa = __builtin_amdgcn_ds_permute(dst, __float_as_int(w.a[c]));
    const int pb = __builtin_amdgcn_ds_permute(dst, __float_as_int(w.b[c]));
    const auto r = __builtin_amdgcn_permlane32_swap(pa, pb, false, false);
    x[c] = __int_as_float((int)r[0]);
    x[4 + c] = __int_as_float((int)r[1]);
  }
}

}  // namespace vws
