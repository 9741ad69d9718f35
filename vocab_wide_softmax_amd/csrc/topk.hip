// topk.hip -- multi-id (top-k) log-probabilities: K target ids per row.
//
// Among the logprobs test cases of DeepSpeed PR #8838 "Add Triton kernels for
// vocab-parallel logprobs, entropy and KL" are repeated ids, ignored ids and
// rows whose ids are all ignored. With ids[n, k] (k < K) and upstream g[n, k]:
//
//   forward    out[n, k] = (z_id - m) - log S          (0 for ignore_index,
//                                                        NaN outside [0, V))
//   backward   dz_j = h_j - G p_j,   h_j = sum of g[n, k] over live slots with
//              ids[n, k] = j (duplicates add), G = sum of g over live slots;
//              a row with every slot ignored gets a zero gradient, a row with
//              any out-of-range live slot a NaN gradient.
//
// The forward is the single-read (m, S) pass of the logprobs forward. When a row
// is one workgroup (unsplit) and K <= 256 that pass writes out[n, k] itself:
// lane k reads slot k's id and logit before the row's stream and forms its output
// after the merge. Otherwise the pass writes the row statistics and the gather
// kernel below (one thread per slot) forms out[n, k]. The backward is one pass over the logits per (row, column tile),
// like the single-id backward. For K <= 64 each wave holds the row's slots one per
// lane and works on them with ballots and lane reads; for larger K each workgroup
// first collects, in slot order, the live ids that fall in its tile into LDS.
// Either way G is summed in a fixed order and the per-column hit sums in slot
// order, the same in every run.
#include "device.h"
#include "launch.h"

namespace vws {

namespace {
constexpr int kTopkBlock = 256;
constexpr int kTopkUB = 4;         // LDS slot kernel: groups of 8 columns per lane per tile (8192-column tiles)
constexpr int kTopkSmallK = 64;    // K up to this: slots in lane registers, one per lane of a wave
constexpr int kTopkSmallUB = 2;    // ... with 4096-column tiles (the fastest by measurement),
// 2048-column tiles on fp32 data, two 16-byte pieces a lane (0.407 -> 0.401 ms at 4096 x 75968, K = 16)
constexpr int topk_small_ub(int dt) { return dt == kF32 ? 1 : kTopkSmallUB; }
constexpr int topk_ub(int32_t K, int dt) { return K <= kTopkSmallK ? topk_small_ub(dt) : kTopkUB; }
}  // namespace

__device__ __forceinline__ int64_t topk_id(const TopkArgs& p, int64_t row, int32_t k) {
  const int64_t ro = udiv(row, p.a.n_inner), ri = row - ro * p.a.n_inner;
  return p.ids[ro * p.ids_so + ri * p.ids_si + (int64_t)k * p.ids_sk];
}

template <int DT>
__global__ __launch_bounds__(256) void topk_gather_kernel(TopkArgs p) {
  const int64_t total = p.N * p.K;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t row = udiv(i, p.K);
    const int32_t k = (int32_t)(i - row * p.K);
    const int64_t t = topk_id(p, row, k);
    float out;
    if (t == p.ignore_index) {
      out = 0.0f;
    } else if (t < 0 || t >= p.V) {
      out = __builtin_nanf("");
    } else {
      const float zt = load_elem<DT>(row_ptr<DT>(p.a, row), t);
      out = (float)(((double)zt - (double)p.stats[2 * row]) - (double)p.stats[2 * row + 1]);
    }
    p.out[i] = out;
  }
}

// Loads this lane's groups of the tile (issued before the slot phase so that their
// latency overlaps it); groups past the row end read as -inf and are not stored.
template <int DT, bool FULL, int UB>
__device__ __forceinline__ void topk_load(const char* ra, int32_t g, int32_t G, int32_t V, int32_t g_full,
                                          float (&x)[UB][8]) {
#pragma unroll
  for (int u = 0; u < UB; ++u, g += kTopkBlock) {
    if (FULL) {
      load_group_vec<DT>(ra, g, x[u]);
    } else if (g < G) {
      load_group<DT, true>(ra, g, V, g_full, x[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[u][j] = -kInf;
    }
  }
}

template <int DT, bool FULL, int UB>
__device__ __forceinline__ void topk_groups(const float (&x)[UB][8], char* oa, int32_t g, int32_t G, int32_t V,
                                            int32_t g_full, int32_t c0, float m, float ls, float Gs, bool nan_row,
                                            bool zero_row, const int32_t* s_col, const float* s_g, int cnt) {
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int u = 0; u < UB; ++u, g += kTopkBlock) {
    if (!FULL && g >= G) break;
    float y[8], h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = 0.0f;
    const int32_t lg = g - (c0 >> 3);  // group index inside the tile
    for (int e = 0; e < cnt; ++e) {
      const int32_t c = s_col[e];
      if ((c >> 3) == lg) {
        const float gk = s_g[e];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j == (c & 7)) h[j] += gk;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const PScaled pj = exp_split((x[u][j] - m) - ls);
      const float d = __builtin_fmaf(-Gs * pj.p, pj.f, h[j]);
      y[j] = zero_row ? 0.0f : (nan_row ? qnan : d);
    }
    if (FULL) store_group_vec<DT>(oa, g, y);
    else store_group<DT, true>(oa, g, V, g_full, y);
  }
}

template <int DT, bool VEC, int UB>
__global__ __launch_bounds__(kTopkBlock) void topk_bwd_kernel(TopkArgs p) {
  constexpr int NW = kTopkBlock / 64;
  constexpr int ES = ElemSize<DT>::value;
  __shared__ int32_t s_col[kTopkMaxK];
  __shared__ float s_g[kTopkMaxK];
  __shared__ float s_red[NW];
  __shared__ int32_t s_cnt[NW];
  __shared__ int32_t s_flags;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = VEC ? V / 8 : 0;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, tpr);
    const int32_t tile = (int32_t)(vb - row * tpr);
    const int32_t g0 = tile * (kTopkBlock * UB);
    // the tile's end column in 64 bits: c0 + 8192 passes INT32_MAX on the last tile of the widest rows
    const int32_t c0 = g0 * 8, c1 = (int32_t)min((int64_t)V, (int64_t)c0 + kTopkBlock * UB * 8);
    const char* ra = row_ptr<DT>(p.a, row);
    const int32_t g = g0 + tid;
    const bool full = VEC && g0 + kTopkBlock * UB <= g_full;
    float x[UB][8];
    if (full) topk_load<DT, true, UB>(ra, g, G, V, g_full, x);
    else topk_load<DT, false, UB>(ra, g, G, V, g_full, x);

    // Slots: G (sum of live g, fixed reduction tree), flags, and the tile's live ids in slot order.
    if (tid == 0) s_flags = 0;
    __syncthreads();
    float gpart = 0.0f;
    int flags = 0;  // bit 0: some slot live, bit 1: some live slot out of range
    int32_t cnt = 0;
    for (int32_t kc = 0; kc < p.K; kc += kTopkBlock) {
      const int32_t k = kc + tid;
      bool hit = false;
      int32_t col = 0;
      float gk = 0.0f;
      if (k < p.K) {
        // the id and its upstream gradient are loaded together (both exist for every slot),
        // so the gradient's latency does not follow the id's
        const int64_t t = topk_id(p, row, k);
        const float gl = p.g[row * p.g_sr + (int64_t)k * p.g_sk];
        if (t != p.ignore_index) {
          flags |= 1;
          if (t < 0 || t >= V) {
            flags |= 2;
          } else {
            gk = gl;
            gpart += gk;
            hit = t >= c0 && t < c1;
            col = (int32_t)(t - c0);
          }
        }
      }
      const uint64_t bal = __ballot(hit);
      const int32_t before = (int32_t)__popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) s_cnt[wave] = (int32_t)__popcll(bal);
      __syncthreads();
      int32_t base = cnt;
      for (int w = 0; w < wave; ++w) base += s_cnt[w];
      if (hit) {
        s_col[base + before] = col;
        s_g[base + before] = gk;
      }
      for (int w = 0; w < NW; ++w) cnt += s_cnt[w];
      __syncthreads();  // s_cnt is rewritten by the next chunk
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gpart += __shfl_xor(gpart, off, 64);
    if (flags) atomicOr(&s_flags, flags);
    if (lane == 0) s_red[wave] = gpart;
    __syncthreads();
    float Gs = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) Gs += s_red[w];
    const int fl = s_flags;

    char* oa = p.dz + row * (int64_t)V * ES;
    const float m = p.stats[2 * row], ls = p.stats[2 * row + 1];
    const bool zero_row = !(fl & 1), nan_row = (fl & 2) != 0;
    if (full)
      topk_groups<DT, true, UB>(x, oa, g, G, V, g_full, c0, m, ls, Gs, nan_row, zero_row, s_col, s_g, cnt);
    else
      topk_groups<DT, false, UB>(x, oa, g, G, V, g_full, c0, m, ls, Gs, nan_row, zero_row, s_col, s_g, cnt);
    __syncthreads();  // LDS is reused by the next tile
  }
}

// Lane k's value (k wave-uniform).
__device__ __forceinline__ float lane_f(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}

// Small K (K <= 64): lane k of every wave loads slot k together with the tile's logits, and
// the slot logic runs on wave-uniform values: ballots give the flags and the live ids that
// fall in the tile, G is a butterfly sum over the wave's lanes (the same value, bit for bit,
// in every lane and every run), and each group of 8 columns adds the hits it owns in slot
// order. No LDS and no barriers: a tile costs about what the single-id backward's does.
// One tile (row, groups g0 .. g0 + TG) of the small-K backward. FULL: every group of the tile is
// a whole 16-byte group (vector loads and stores, no bounds checks); kept as its own instance so
// the interior tile's code has no predicated element loads to merge with.
template <int DT, bool VEC, int UB, bool FULL>
__device__ __forceinline__ void topk_small_tile(const TopkArgs& p, int64_t row, int32_t g0, int tid, int lane) {
  constexpr int ES = ElemSize<DT>::value;
  constexpr int TG = kTopkBlock * UB;  // groups of 8 columns per tile
  const int32_t V = (int32_t)p.V;
  const int32_t G = (V + 7) / 8;
  const int32_t g_full = VEC ? V / 8 : 0;
  const int32_t K = p.K;
  const char* ra = row_ptr<DT>(p.a, row);
  const int32_t g = g0 + tid;
  // The slot and row-constant loads go out first, then the tile's logit loads. Loads complete
  // in issue order, so the slot logic below (ballots, the G butterfly, the hit masks) waits only
  // for the small loads and runs while the tile is in flight: one memory latency per tile.
  int64_t tv = p.ignore_index;
  float gl = 0.0f;
  if (lane < K) {
    tv = topk_id(p, row, lane);
    gl = p.g[row * p.g_sr + (int64_t)lane * p.g_sk];
  }
  const float m = p.stats[2 * row], ls = p.stats[2 * row + 1];
  __builtin_amdgcn_sched_barrier(0);
  RawGroup<DT> w[UB];
  float x[UB][8];
  if constexpr (FULL) {
#pragma unroll
    for (int u = 0; u < UB; ++u) load_group_raw<DT>(ra, g + u * kTopkBlock, w[u]);
  } else {
    topk_load<DT, false, UB>(ra, g, G, V, g_full, x);
  }
  __builtin_amdgcn_sched_barrier(0);

  const bool live = lane < K && tv != p.ignore_index;
  const bool oor = live && (tv < 0 || tv >= V);
  const bool in_tile = live && !oor && (tv >> 3) >= g0 && (tv >> 3) < g0 + TG;
  const bool zero_row = __ballot(live) == 0ull, nan_row = __ballot(oor) != 0ull;
  const uint64_t hits = __ballot(in_tile);
  float Gs = live && !oor ? gl : 0.0f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) Gs += __shfl_xor(Gs, off, 64);

  char* oa = p.dz + row * (int64_t)V * ES;
  const float qnan = __builtin_nanf("");
  if constexpr (FULL) {
#pragma unroll
    for (int u = 0; u < UB; ++u) raw_to_float<DT>(w[u], x[u]);
  }
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    const int32_t gu = g + u * kTopkBlock;
    if (!FULL && gu >= G) break;
    float y[8], hu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) hu[j] = 0.0f;
    for (uint64_t hm = hits; hm; hm &= hm - 1) {  // slot order
      const int k = __builtin_ctzll(hm);
      const int32_t t = __builtin_amdgcn_readlane((int32_t)tv, k);
      const int32_t rel = (t >> 3) - g0;
      if (rel / kTopkBlock != u) continue;
      const float gk = lane_f(gl, k);
      const float add = (rel % kTopkBlock) == tid ? gk : 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j == (t & 7)) hu[j] += add;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const PScaled pj = exp_split((x[u][j] - m) - ls);
      const float d = __builtin_fmaf(-Gs * pj.p, pj.f, hu[j]);
      y[j] = zero_row ? 0.0f : (nan_row ? qnan : d);
    }
    if constexpr (FULL) store_group_vec<DT>(oa, gu, y);
    else store_group<DT, true>(oa, gu, V, g_full, y);
  }
}

// A whole fp32 tile of the small-K backward: the gradient is elementwise (a column adds the hits on
// it in slot order), so lane l takes the tile's 16-byte pieces l, l + 256, ... instead of its
// groups of 8 columns, and every load and store of a wave covers one contiguous 1 KB. Same slot
// logic and arithmetic as topk_small_tile.
template <int UB>
__device__ __forceinline__ void topk_small_tile_f32(const TopkArgs& p, int64_t row, int32_t g0, int tid, int lane) {
  constexpr int TG = kTopkBlock * UB;  // groups of 8 columns per tile
  constexpr int NP = 2 * UB;           // 16-byte pieces per lane
  const int32_t V = (int32_t)p.V;
  const int32_t K = p.K;
  const char* ra = row_ptr<kF32>(p.a, row);
  const int64_t q0 = 2 * (int64_t)g0 + tid;  // this lane's first piece
  int64_t tv = p.ignore_index;
  float gl = 0.0f;
  if (lane < K) {
    tv = topk_id(p, row, lane);
    gl = p.g[row * p.g_sr + (int64_t)lane * p.g_sk];
  }
  const float m = p.stats[2 * row], ls = p.stats[2 * row + 1];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 x[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) x[k] = stream_load(reinterpret_cast<const f32x4*>(ra) + q0 + k * kTopkBlock);
  __builtin_amdgcn_sched_barrier(0);

  const bool live = lane < K && tv != p.ignore_index;
  const bool oor = live && (tv < 0 || tv >= V);
  const bool in_tile = live && !oor && (tv >> 3) >= g0 && (tv >> 3) < g0 + TG;
  const bool zero_row = __ballot(live) == 0ull, nan_row = __ballot(oor) != 0ull;
  const uint64_t hits = __ballot(in_tile);
  float Gs = live && !oor ? gl : 0.0f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) Gs += __shfl_xor(Gs, off, 64);

  float hu[NP][4];
#pragma unroll
  for (int k = 0; k < NP; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) hu[k][e] = 0.0f;
  for (uint64_t hm = hits; hm; hm &= hm - 1) {  // slot order
    const int kk = __builtin_ctzll(hm);
    const int32_t t = __builtin_amdgcn_readlane((int32_t)tv, kk);
    const int32_t rel = (t >> 2) - 2 * g0;  // piece inside the tile
    const float gk = lane_f(gl, kk);
    const float add = (rel % kTopkBlock) == tid ? gk : 0.0f;
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (k == rel / kTopkBlock && e == (t & 3)) hu[k][e] += add;
  }
  char* oa = p.dz + row * (int64_t)V * 4;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const PScaled pj = exp_split((x[k][e] - m) - ls);
      const float d = __builtin_fmaf(-Gs * pj.p, pj.f, hu[k][e]);
      y[e] = zero_row ? 0.0f : (nan_row ? qnan : d);
    }
    stream_store(y, reinterpret_cast<f32x4*>(oa) + q0 + k * kTopkBlock);
  }
}

template <int DT, bool VEC, int UB>
__global__ __launch_bounds__(kTopkBlock) void topk_bwd_small_kernel(TopkArgs p) {
  constexpr int TG = kTopkBlock * UB;  // groups of 8 columns per tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int32_t tpr = p.tiles_per_row;
  const int64_t total = p.N * tpr;
  const int32_t g_full = VEC ? (int32_t)(p.V / 8) : 0;
  for (int64_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
    const int64_t row = udiv(vb, tpr);
    const int32_t tile = (int32_t)(vb - row * tpr);
    const int32_t g0 = tile * TG;
    if (DT == kF32 && VEC && g0 + TG <= g_full) topk_small_tile_f32<UB>(p, row, g0, tid, lane);
    else if (VEC && g0 + TG <= g_full) topk_small_tile<DT, VEC, UB, true>(p, row, g0, tid, lane);
    else topk_small_tile<DT, VEC, UB, false>(p, row, g0, tid, lane);
  }
}

int32_t topk_tiles_per_row(int64_t V, int32_t K, int dtype) {
  const int64_t G = (V + 7) / 8, per = (int64_t)kTopkBlock * topk_ub(K, dtype);
  return (int32_t)((G + per - 1) / per);
}

hipError_t launch_topk_gather(const TopkArgs& p, int dtype, hipStream_t stream) {
  const int64_t blocks = grid_cap((p.N * p.K + 255) / 256);
  return dispatch_dtype(dtype, [&](auto dt) {
    hipLaunchKernelGGL((topk_gather_kernel<decltype(dt)::value>), dim3((uint32_t)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
  });
}

hipError_t launch_topk_bwd(const TopkArgs& p, int dtype, bool vec, hipStream_t stream) {
  const int64_t blocks = grid_cap(p.N * p.tiles_per_row);
  const dim3 grid((uint32_t)blocks), block(kTopkBlock);
  return dispatch_dtype(dtype, [&](auto dt) {
    constexpr int DT = decltype(dt)::value;
    if (p.K <= kTopkSmallK) {
      if (vec) hipLaunchKernelGGL((topk_bwd_small_kernel<DT, true, topk_small_ub(DT)>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((topk_bwd_small_kernel<DT, false, topk_small_ub(DT)>), grid, block, 0, stream, p);
    } else if (vec) {
      hipLaunchKernelGGL((topk_bwd_kernel<DT, true, kTopkUB>), grid, block, 0, stream, p);
    } else {
      hipLaunchKernelGGL((topk_bwd_kernel<DT, false, kTopkUB>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
  });
}

}  // namespace vws
