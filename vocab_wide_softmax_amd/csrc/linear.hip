// linear.hip -- fused linear-logp on MFMA (RL-Kernel PR #208, PR body "Implementation";
// review nitpick on the chunked backward).
//
// Forward: logits z = h W^T (h [N, H] bf16 tokens, W [V, H] bf16 vocabulary rows)
// are computed tile by tile and never stored. lin_fwd_kernel computes a 256-row
// vocabulary tile x 256 tokens with MFMA (A = W rows, B = h rows, fp32
// accumulation); in the accumulator layout each lane holds one token column and
// 16 vocabulary rows per block, so the online (m, S) update of that token is
// mostly in-lane. A workgroup walks one vocabulary chunk for one token tile and
// writes the chunk's (m, S) per token; lin_combine_kernel merges the chunks in
// order (the pages' MAX / rescale / SUM of running max and sum across vocab
// shards, inside one GPU) and forms logp = z_t - lse, with z_t from
// lin_target_kernel (one wave per token, fp32 dot product).
//
// Backward, one vocabulary chunk of 8192 columns at a time (the chunked backward of the review
// nitpick): dz = g (onehot(t) - p) with p = exp((z - m) - log S) recomputed from a second MFMA
// pass (lin_dz_kernel, A = h rows, B = W rows, so a lane's 32 consecutive vocabulary columns
// make coalesced stores of dz [N, chunk]), kept as a bf16 (hi, lo) pair; then dW of the chunk's
// vocabulary rows = dz^T h, and dh += dz W_chunk summed in fp32 over the chunks, by
// gemm_pair_kernel (both planes of dz contracted into one fp32 accumulator; a chunk's dW and dh
// tiles share one grid, gemm_pair2_kernel, when both are wanted), reading the transposed
// operands through gfx950's transposing LDS reads (gemm.h).
#include <algorithm>

#include "device.h"
#include "gemm.h"
#include "launch.h"

namespace vws {

using gemm::Acc;
using gemm::Cfg;
using gemm::KROW;
using gemm::Operand;
using gemm::ROWK;

// Logits tiles, A and B both reduction-contiguous, two stages of BK = 64. The forward runs the
// ping-pong main loop, whose two-stage refill goes out whole in one read phase (PIECES plays no
// part there, nor on the flat path of edge tiles); dz runs the shared loop and refills a stage in
// one burst after its barrier (1% faster there than two pieces; bit-identical either way).
typedef Cfg<256, 256, 64, 2, 4, ROWK, ROWK, 2, 1, 1> CfgNT;   // dz
typedef Cfg<256, 256, 64, 2, 4, ROWK, ROWK, 2, 1, 2> CfgFwd;  // forward
// dh = dz W and dW = dz^T h with dz a bf16 (hi, lo) pair: 3 stages of BK = 32 (48 KB each), wave
// tiles of 64 x 128 so that a k-slice reads 2 + 2 A fragments and 4 B fragments for 16 MFMAs
// (128 x 64 wave tiles: 7-13% slower), run by the ping-pong main loop (a phase is one slice),
// each refill in two pieces, one per half-stage read: 8% faster than the shared loop.
typedef Cfg<256, 256, 32, 4, 2, ROWK, KROW, 3, 2, 2> CfgNN2;  // dh = dz W
typedef Cfg<256, 256, 32, 4, 2, KROW, KROW, 3, 2, 2> CfgTN2;  // dW = dz^T h
// Small batches: dz and dh over 128-token tiles, which doubles their workgroups where the
// 256-token tiles would fill at most half of the 256 CUs (kLinHalfRound tiles or fewer). A token
// row keeps its place in its 32-row MFMA block and every entry its k-sequence, so dz and dh are
// the same bits with either tile height (dh stays batch invariant).
typedef Cfg<128, 256, 64, 2, 4, ROWK, ROWK, 2, 1, 1> CfgNTs;   // dz
typedef Cfg<128, 256, 32, 2, 4, ROWK, KROW, 3, 2, 2> CfgNN2s;  // dh
constexpr int64_t kLinHalfRound = 128;

namespace gemm {
__device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};
}  // namespace gemm


// ---- forward -----------------------------------------------------------------------

// Block -> (token tile, vocabulary chunk). Block b runs on XCD b % 8, and an XCD runs 32
// blocks at a time. Token tiles go in groups of 32, 4 per XCD; an XCD's blocks take its 4
// token tiles fastest, then the chunks, so the 32 it runs at once are 4 token tiles x 8
// chunks: its L2 streams 4 h panels and 8 W tiles per vocabulary step (a one-chunk order
// streams 32 h panels for 1 W tile). Token tiles past the last whole group of 32 follow in
// plain order.
__device__ __forceinline__ void fwd_tile(int64_t b, int64_t ntt, int nchunks, int64_t& tt, int& c) {
  const int64_t ntt_full = (ntt / 32) * 32;
  if (b < ntt_full * nchunks) {
    const int64_t x = b % 8, q = b / 8;
    const int64_t r = q / 4;
    c = (int)(r % nchunks);
    tt = ((r / nchunks) * 8 + x) * 4 + q % 4;
  } else {
    const int64_t r = b - ntt_full * nchunks;
    tt = ntt_full + r / nchunks;
    c = (int)(r % nchunks);
  }
}

template <class C>
__global__ __launch_bounds__(C::NT) void lin_fwd_kernel(LinArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int nchunks = p.chunks;
  int64_t tt;  // token tile
  int c;       // vocabulary chunk
  fwd_tile((int64_t)blockIdx.x, (p.N + C::BN - 1) / C::BN, nchunks, tt, c);
  const int64_t n0 = tt * C::BN;
  const int64_t vt0 = (int64_t)c * p.tiles_per_chunk;
  const int64_t vt1 = min(vt0 + p.tiles_per_chunk, (p.V + C::BM - 1) / C::BM);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  const Operand A{p.W, p.ldw, p.V, p.H};
  const Operand B{p.h, p.ldh, p.N, p.H};
  State1 st[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) st[j] = state1_init();

  Acc<C> acc;
  for (int64_t vt = vt0; vt < vt1; ++vt) {
    const int64_t m0 = vt * C::BM;
    gemm::mainloop_pp<C>(A, B, m0, n0, p.H, lds, acc);  // ping-pong: 3% faster here (dz: no gain)
    if (m0 + C::BM > p.V) {  // the last vocabulary tile: rows past V take no part
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm * C::TM + gemm::acc_row(i, v, lane);
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
            if (row >= p.V) acc.c[i][j][v] = -kInf;
        }
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      float bm = -kInf;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) bm = fmaxf(bm, acc.c[i][j][v]);
      if (bm > st[j].m) {
        const float s = expf_fast(st[j].m - bm);
        st[j].S *= s;
        st[j].m = bm;
      }
      const float ref = ref_of(st[j].m);
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += expf_fast(acc.c[i][j][v] - ref);
      st[j].S += sum;
    }
  }
  // lanes l and l ^ 32 hold the same token column
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    State1 o{__shfl_xor(st[j].m, 32, 64), __shfl_xor(st[j].S, 32, 64), 0.0f};
    st[j] = merge1<false>(st[j], o);
  }
  // waves with the same token columns (different wm) merge through LDS, in wm order
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [WM][BN][2]
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int col = wn * C::TN + j * 32 + lane;
      red[(wm * C::BN + col) * 2 + 0] = st[j].m;
      red[(wm * C::BN + col) * 2 + 1] = st[j].S;
    }
  }
  __syncthreads();
  for (int col = threadIdx.x; col < C::BN; col += C::NT) {
    State1 s = state1_init();
#pragma unroll
    for (int w = 0; w < C::WM; ++w) s = merge1<false>(s, State1{red[(w * C::BN + col) * 2], red[(w * C::BN + col) * 2 + 1], 0.0f});
    const int64_t n = n0 + col;
    if (n < p.N) {
      p.part[(n * nchunks + c) * 2 + 0] = s.m;
      p.part[(n * nchunks + c) * 2 + 1] = s.S;
    }
  }
}

// One wave per token: z_t = sum_k h[n, k] W[t, k] in fp32 (bf16 products are exact).
__global__ __launch_bounds__(256) void lin_target_kernel(LinArgs p) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= p.N) return;
  const int64_t t = p.t[n];
  if (t < 0 || t >= p.V) {
    if (lane == 0) p.zt[n] = 0.0f;
    return;
  }
  const uint16_t* hr = p.h + n * p.ldh;
  const uint16_t* wr = p.W + t * p.ldw;
  float s = 0.0f;
  for (int64_t k = lane; k < p.H; k += 64)
    s = fmaf(bf16_bits_to_float(hr[k]), bf16_bits_to_float(wr[k]), s);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) p.zt[n] = s;
}

// One thread per token: merge the chunk states in chunk order, then logp = z_t - (m + log S).
__global__ __launch_bounds__(256) void lin_combine_kernel(LinArgs p) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= p.N) return;
  State1 s = state1_init();
  for (int c = 0; c < p.chunks; ++c)
    s = merge1<false>(s, State1{p.part[(n * p.chunks + c) * 2], p.part[(n * p.chunks + c) * 2 + 1], 0.0f});
  const double logS = log((double)s.S);
  p.stats[2 * n + 0] = s.m;
  p.stats[2 * n + 1] = (float)logS;
  const int64_t t = p.t[n];
  float out;
  if (t == p.ignore_index) out = 0.0f;
  else if (t < 0 || t >= p.V) out = __builtin_nanf("");
  else out = (float)(((double)p.zt[n] - (double)s.m) - logS);
  p.logp[n] = out;
}

// ---- backward ------------------------------------------------------------------------

// Block -> (token tile, vocabulary tile of the chunk) for the dz pass. Block b runs on XCD b % 8,
// and an XCD runs 32 blocks at a time; those 32 form a patch of 4 token tiles x 8 vocabulary
// tiles, so its L2 streams 4 h panels and 8 W tiles per k-step (one vocabulary tile at a time
// would stream 32 h panels for 1 W tile). The 8 XCDs' patches make a super-tile of 8 token tiles
// x 32 vocabulary tiles (2 x 4 patches), and super-tiles go token fastest, so the chunk's W tiles
// are reused from the MALL by every token group in turn. Tiles outside the whole super-tiles
// follow in plain order.
__device__ __forceinline__ void dz_tile(int64_t b, int64_t ntt, int64_t nvt, int64_t& tt, int64_t& vt) {
  const int64_t ntt8 = (ntt / 8) * 8, nvt32 = (nvt / 32) * 32;
  const int64_t nfull = ntt8 * nvt32;
  if (b < nfull) {
    const int64_t x = b % 8, q = b / 8, s = q / 32, w = q % 32, nst = ntt8 / 8;
    tt = (s % nst) * 8 + (x / 4) * 4 + w % 4;
    vt = (s / nst) * 32 + (x % 4) * 8 + w / 4;
    return;
  }
  const int64_t r = b - nfull, r1 = ntt8 * (nvt - nvt32);
  if (r < r1) {  // whole token groups, vocabulary tiles past the last super-tile
    tt = r % ntt8;
    vt = nvt32 + r / ntt8;
  } else {  // the last ntt - ntt8 token tiles, every vocabulary tile
    const int64_t r2 = r - r1, nt2 = ntt - ntt8;
    tt = ntt8 + r2 % nt2;
    vt = r2 / nt2;
  }
}

// dz = g (1[v = t] - p) of one logit x, the product formed at the 2^64 scale of exp_split so that
// probabilities below 2^-126 keep their bits; c = (m, log S, -g, target column or -1) of its
// token. -g = 0 (ignored token) gives 0 even where p is not finite (v_mul_legacy_f32); the
// target's entry is fma(-g, p, g), rounded once.
__device__ __forceinline__ float dz_of(float x, const f32x4& c, int lc) {
  const PScaled pz = exp_split((x - c.x) - c.y);
  const float gn = c.z;
  return lc == __float_as_int(c.w) ? __builtin_fmaf(gn, pz.p * pz.f, -gn) : mul0(gn, pz.p) * pz.f;
}

// dz of one vocabulary chunk: recompute the logits tile z = h W^T (fp32 accumulation), form
// dz = g (1[v = t] - p) with p = exp((z - m) - log S) in fp32, and store it as the bf16 pair
// hi = rne(dz), lo = rne(dz - hi), which carries dz to about 2^-17 relative into the two
// contractions (a single bf16 dz would cost up to 2^-9 per term of dh and dW).
template <class C>
__global__ __launch_bounds__(C::NT) void lin_dz_kernel(LinArgs p) {
  extern __shared__ __align__(16) char lds[];
  const int64_t ntt = (p.N + C::BM - 1) / C::BM, nvt = (p.cw + C::BN - 1) / C::BN;
  int64_t tt, vt;
  dz_tile((int64_t)blockIdx.x, ntt, nvt, tt, vt);
  const int64_t m0 = tt * C::BM, n0 = vt * C::BN;  // n0: column inside the chunk
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const Operand A{p.h, p.ldh, p.N, p.H};
  const Operand B{p.W + p.v0 * p.ldw, p.ldw, p.cw, p.H};
  // This tile's per-token inputs are loaded before the main loop and used only after it, so
  // their latency hides behind it (deriving anything from them here would wait for them first).
  int64_t t = 0;
  float m = 0.0f, ls = 0.0f, gv = 0.0f;
  if (threadIdx.x < C::BM) {
    const int64_t n = m0 + threadIdx.x < p.N ? m0 + threadIdx.x : p.N - 1;
    t = p.t[n];
    m = p.stats[2 * n];
    ls = p.stats[2 * n + 1];
    gv = p.g[n * p.g_stride];
  }
  Acc<C> acc;
  gemm::mainloop<C>(A, B, m0, n0, p.H, lds, acc);  // ends with a barrier: LDS is free again
  // Row constants in LDS: m, log S, -g (NaN when the target is out of range, which makes the
  // whole row NaN; 0 for an ignored token, whose row is zero) and the target's column inside the
  // tile (-1 when it lies in another tile or the token is ignored).
  f32x4* cst = reinterpret_cast<f32x4*>(lds);
  if (threadIdx.x < C::BM) {
    const bool ignored = t == p.ignore_index, bad = !ignored && (t < 0 || t >= p.V);
    const int64_t c0 = p.v0 + n0;
    const int32_t tc = !ignored && t >= c0 && t < c0 + C::BN ? (int32_t)(t - c0) : -1;
    const float gneg = ignored ? 0.0f : (bad ? __builtin_nanf("") : -gv);
    cst[threadIdx.x] = (f32x4){m, ls, gneg, __int_as_float(tc)};
  }
  __syncthreads();
  uint16_t* th = p.dzh + m0 * p.ldc + n0;
  uint16_t* tl = p.dzl + m0 * p.ldc + n0;
  if (m0 + C::BM <= p.N && n0 + C::BN <= p.cw && p.ldc < (1 << 23)) {
    // Interior tile: no guards, 32-bit byte offsets from the tile's base (below 2^32 for rows of
    // fewer than 2^23 columns, so the stores take a scalar base and a 32-bit offset), and the
    // two rows v, v + 1 of an accumulator pair rounded by one conversion per plane.
    const uint32_t ldb = (uint32_t)p.ldc * 2u;  // row pitch in bytes
    char* thb = reinterpret_cast<char*>(th);
    char* tlb = reinterpret_cast<char*>(tl);
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int r = wm * C::TM + gemm::acc_row(i, v, lane);  // row r + 1 holds accumulator v + 1
        const f32x4 c0 = cst[r], c1 = cst[r + 1];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int lc = wn * C::TN + gemm::acc_col(j, lane);
          const float d0 = dz_of(acc.c[i][j][v], c0, lc), d1 = dz_of(acc.c[i][j][v + 1], c1, lc);
          const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){d0, d1}, bf16x2));
          // exact (Sterbenz), 0 for 0 and NaN
          const float l0 = d0 - __uint_as_float(hb << 16), l1 = d1 - __uint_as_float(hb & 0xffff0000u);
          const uint32_t lb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){l0, l1}, bf16x2));
          const uint32_t o = (uint32_t)r * ldb + (uint32_t)lc * 2u;
          *reinterpret_cast<uint16_t*>(thb + o) = (uint16_t)hb;
          *reinterpret_cast<uint16_t*>(thb + (o + ldb)) = (uint16_t)(hb >> 16);
          *reinterpret_cast<uint16_t*>(tlb + o) = (uint16_t)lb;
          *reinterpret_cast<uint16_t*>(tlb + (o + ldb)) = (uint16_t)(lb >> 16);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * C::TM + gemm::acc_row(i, v, lane);
        const f32x4 c = cst[r];
        const int64_t ro = (int64_t)r * p.ldc;
        const bool row_ok = m0 + r < p.N;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          const int lc = wn * C::TN + gemm::acc_col(j, lane);
          const int64_t col = n0 + lc;
          if (row_ok && col < p.ldc) {
            // columns [cw, ldc) pad the rows with zeros for the dh contraction
            const float d = col < p.cw ? dz_of(acc.c[i][j][v], c, lc) : 0.0f;
            const bf16x2 hb = __builtin_convertvector((f32x2){d, 0.0f}, bf16x2);
            const uint32_t hbits = __builtin_bit_cast(uint32_t, hb) & 0xffffu;
            const float lo = d - __uint_as_float(hbits << 16);
            const bf16x2 lb = __builtin_convertvector((f32x2){lo, 0.0f}, bf16x2);
            th[ro + lc] = (uint16_t)hbits;
            tl[ro + lc] = (uint16_t)(__builtin_bit_cast(uint32_t, lb) & 0xffffu);
          }
        }
      }
  }
}

// Block -> (M tile, N tile) of a contraction with a long reduction (K = 8192 for dh and dW).
// Block b runs on XCD b % 8, and an XCD runs 32 blocks at a time; those form a patch of 4 M tiles
// x 8 N tiles, so per k-step its L2 takes 4 A and 8 B tile slices for 32 tiles (row-major order
// gave an XCD 16 M tiles x 2 N tiles: 18 slices, an L2 hit rate of 61-64%). The 8 XCDs' patches
// cover a super-tile of (32 / ntn) 4 M tiles x ntn N tiles (ntn in {8, 16, 32, 64}), super-tiles
// go along M; other shapes and the M tiles past the last whole super-tile run in row-major order.
__device__ __forceinline__ void pair_tile(int64_t b, int64_t ntm, int64_t ntn, int64_t& tm, int64_t& tn) {
  if (ntn == 8 || ntn == 16 || ntn == 32 || ntn == 64) {
    const int64_t ng = ntn / 8, mg = 8 / ng, sm = mg * 4;  // XCD groups along N and M; super-tile rows
    const int64_t nfull = (ntm / sm) * sm * ntn;
    if (b < nfull) {
      const int64_t x = b % 8, q = b / 8, st = q / 32, w = q % 32;
      tm = st * sm + (x % mg) * 4 + w % 4;
      tn = (x / mg) * 8 + w / 4;
      return;
    }
    const int64_t r = b - nfull;
    tm = ntm / sm * sm + r / ntn;
    tn = r % ntn;
    return;
  }
  tm = b / ntn;
  tn = b - tm * ntn;
}

// C = A B^T over K, A a split (hi, lo) pair, for the tile of block b; dW rows of a chunk (bf16
// stores) and dh of a chunk (stored, or added to the fp32 running sum over the chunks; the last
// chunk rounds the sum to bf16).
template <class C>
__device__ __forceinline__ void pair_block(const GemmArgs& g, int64_t b, char* lds) {
  const int64_t ntm = (g.M + C::BM - 1) / C::BM, ntn = (g.Nc + C::BN - 1) / C::BN;
  int64_t tm, tn;
  pair_tile(b, ntm, ntn, tm, tn);
  const int64_t m0 = tm * C::BM, n0 = tn * C::BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  Acc<C> acc;
  gemm::mainloop_pp<C>(g.A, g.B, m0, n0, g.K, lds, acc);
  const int mode = g.mode;
  if (m0 + C::BM <= g.M && n0 + C::BN <= g.Nc && g.ldc < (1 << 22)) {
    // Interior tile: the mode is tested once, addresses are the wave's scalar tile base plus a
    // 32-bit byte offset (below 2^32: 64 rows of fewer than 2^22 fp32), bf16 results are rounded
    // two rows (accumulators v, v + 1) per conversion, and the running sum is read one 32 x 32
    // block (16 values a lane) at a time before any of it is added: one memory wait per block.
    const int64_t wo = (m0 + wm * C::TM) * g.ldc + n0 + wn * C::TN;
    const uint32_t ld = (uint32_t)g.ldc;
    char* cb = reinterpret_cast<char*>(g.C + wo);
    char* ab = reinterpret_cast<char*>(g.acc + wo);
    auto off = [&](int i, int v, int j) { return (uint32_t)gemm::acc_row(i, v, lane) * ld + (uint32_t)gemm::acc_col(j, lane); };
    auto store_pairs = [&](int i, int j, const float (&y)[16]) {
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){y[v], y[v + 1]}, bf16x2));
        const uint32_t o = off(i, v, j) * 2u;  // row v + 1 is one pitch further
        *reinterpret_cast<uint16_t*>(cb + o) = (uint16_t)hb;
        *reinterpret_cast<uint16_t*>(cb + (o + ld * 2u)) = (uint16_t)(hb >> 16);
      }
    };
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        float y[16];
        if (mode == kDhStore) {
#pragma unroll
          for (int v = 0; v < 16; ++v) y[v] = acc.c[i][j][v];
          store_pairs(i, j, y);
        } else if (mode == kDhFirst) {
#pragma unroll
          for (int v = 0; v < 16; ++v) *reinterpret_cast<float*>(ab + off(i, v, j) * 4u) = acc.c[i][j][v];
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) y[v] = *reinterpret_cast<const float*>(ab + off(i, v, j) * 4u);
#pragma unroll
          for (int v = 0; v < 16; ++v) y[v] = y[v] + acc.c[i][j][v];  // the running sum first: chunk order
          if (mode == kDhAdd) {
#pragma unroll
            for (int v = 0; v < 16; ++v) *reinterpret_cast<float*>(ab + off(i, v, j) * 4u) = y[v];
          } else {
            store_pairs(i, j, y);
          }
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t r = m0 + wm * C::TM + gemm::acc_row(i, v, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int64_t col = n0 + wn * C::TN + gemm::acc_col(j, lane);
        if (r < g.M && col < g.Nc) {
          float x = acc.c[i][j][v];
          const int64_t o = r * g.ldc + col;
          if (mode == kDhFirst) {
            g.acc[o] = x;
            continue;
          }
          if (mode != kDhStore) x = g.acc[o] + x;  // the running sum first: chunk order
          if (mode == kDhAdd) {
            g.acc[o] = x;
            continue;
          }
          const bf16x2 hb = __builtin_convertvector((f32x2){x, 0.0f}, bf16x2);
          g.C[o] = (uint16_t)(__builtin_bit_cast(uint32_t, hb) & 0xffffu);
        }
      }
    }
}

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_pair_kernel(GemmArgs g) {
  extern __shared__ __align__(16) char lds[];
  pair_block<C>(g, (int64_t)blockIdx.x, lds);
}

// A chunk's dW and dh contractions in one launch: blocks [0, nb1) take the tiles of g1 (dW), the
// rest those of g2 (dh). The two read the same dz planes and write disjoint outputs, so running
// them as one grid changes no result; it removes one kernel's last-round tail per chunk (the
// dh tiles start on the CUs the dW tiles leave). nb1 is a multiple of 8, so a block's XCD
// (b mod 8) is the same in either numbering.
template <class C1, class C2>
__global__ __launch_bounds__(C1::NT) void gemm_pair2_kernel(GemmArgs g1, GemmArgs g2, int64_t nb1) {
  static_assert(C1::NT == C2::NT, "one workgroup size");
  extern __shared__ __align__(16) char lds[];
  const int64_t b = (int64_t)blockIdx.x;
  if (b < nb1) pair_block<C1>(g1, b, lds);
  else pair_block<C2>(g2, b - nb1, lds);
}

// ---- host-side launch ---------------------------------------------------------------------

namespace {
template <class C>
size_t lds_bytes() {
  return (size_t)C::LDS_BYTES;
}
}  // namespace

// Vocabulary tiles per forward chunk. Automatic (split_hint 0): the chunking that minimises the
// forward's estimated makespan, rounds x tiles per chunk, where a round is one workgroup on each
// of gfx950's 256 CUs (the kernel's 128 KB of LDS admits one per CU); ties go to fewer rounds
// (workgroups that start together stay in step and share the h panels and W tiles in their
// XCD's L2). At 2048 x 4096 x 151936 that is 32 chunks of 19 tiles in one round instead of 60
// chunks of 10 in two (2.23 -> 2.15 ms); at 8548 x 4096 x 16684, 22 chunks of 3 tiles (1.10 ->
// 1.02 ms); at 512 tokens, 119 chunks of 5 (0.88 -> 0.72 ms). The chunking, and the order in
// which a token's chunk partials merge, then follow the batch. split_hint >= 1 asks for that
// many chunks, and VWS_SPLIT_INVARIANT (-1) fixes chunks of kLinInvariantTiles tiles (1024
// vocabulary columns); both depend on V alone, so a token's logp and statistics are the same
// bits in every batch (each logit is the same MFMA k-sequence whichever tile holds it).
namespace {
constexpr int kLinInvariantTiles = 4;
constexpr int64_t kLinCUs = 256;        // compute units of a gfx950 device (MI350X, MI355X)
constexpr int64_t kLinMaxRounds = 16;   // automatic chunkings considered: up to this many rounds

int64_t lin_auto_tiles_per_chunk(int64_t ntt, int64_t nvt) {
  ntt = std::max<int64_t>(ntt, 1);
  const int64_t cmax = std::max<int64_t>(1, std::min<int64_t>(nvt, kLinCUs * kLinMaxRounds / ntt));
  int64_t best_tpc = nvt, best_cost = -1, best_rounds = 0;
  for (int64_t c = 1; c <= cmax; ++c) {
    const int64_t tpc = (nvt + c - 1) / c, chunks = (nvt + tpc - 1) / tpc;
    const int64_t rounds = (ntt * chunks + kLinCUs - 1) / kLinCUs, cost = rounds * tpc;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && rounds < best_rounds)) {
      best_tpc = tpc;
      best_cost = cost;
      best_rounds = rounds;
    }
  }
  return best_tpc;
}
}  // namespace

int32_t lin_tiles_per_chunk(int64_t N, int64_t V, int split_hint) {
  const int64_t nvt = (V + CfgFwd::BM - 1) / CfgFwd::BM;
  if (split_hint == -1) return kLinInvariantTiles;
  if (split_hint == 0) return (int32_t)lin_auto_tiles_per_chunk((N + CfgFwd::BN - 1) / CfgFwd::BN, nvt);
  const int64_t c = split_hint > nvt ? nvt : split_hint;
  return (int32_t)((nvt + c - 1) / c);
}

int lin_chunks(int64_t N, int64_t V, int split_hint) {
  const int64_t nvt = (V + CfgFwd::BM - 1) / CfgFwd::BM;
  const int64_t tpc = lin_tiles_per_chunk(N, V, split_hint);
  return (int)((nvt + tpc - 1) / tpc);
}

hipError_t launch_lin_fwd(LinArgs p, int split_hint, hipStream_t stream) {
  const int64_t ntt = (p.N + CfgFwd::BN - 1) / CfgFwd::BN;
  p.tiles_per_chunk = lin_tiles_per_chunk(p.N, p.V, split_hint);
  p.chunks = lin_chunks(p.N, p.V, split_hint);
  hipLaunchKernelGGL(lin_target_kernel, dim3((uint32_t)((p.N + 3) / 4)), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((lin_fwd_kernel<CfgFwd>), dim3((uint32_t)(ntt * p.chunks)), dim3(CfgFwd::NT), lds_bytes<CfgFwd>(), stream, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(lin_combine_kernel, dim3((uint32_t)((p.N + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Vocabulary tiles per backward chunk: 32 (8192 columns) unless split_hint >= 1 asks for that
// many chunks. The chunking depends on V alone, so dh is batch invariant.
int32_t lin_bwd_tiles_per_chunk(int64_t V, int split_hint) {
  const int64_t nvt = (V + CfgNT::BN - 1) / CfgNT::BN;
  int64_t tpc = 32;
  if (split_hint >= 1) tpc = (nvt + split_hint - 1) / split_hint;
  tpc = tpc < 1 ? 1 : (tpc > nvt ? nvt : tpc);
  return (int32_t)tpc;
}

hipError_t launch_lin_bwd(LinArgs p, int split_hint, uint16_t* dh, uint16_t* dW, hipStream_t stream) {
  const int64_t C = (int64_t)lin_bwd_tiles_per_chunk(p.V, split_hint) * CfgNT::BN;
  const int64_t nchunks = (p.V + C - 1) / C;
  static_assert(CfgNTs::BN == CfgNT::BN && CfgNN2s::BN == CfgNN2::BN, "small-batch tiles differ in height only");
  const int64_t ntt = (p.N + CfgNT::BM - 1) / CfgNT::BM, nht = (p.H + CfgNN2::BN - 1) / CfgNN2::BN;
  const int64_t ntt_s = (p.N + CfgNTs::BM - 1) / CfgNTs::BM;
  const bool dh_small = ntt * nht <= kLinHalfRound;
  hipError_t e;
  for (int64_t c = 0; c < nchunks; ++c) {
    p.v0 = c * C;
    p.cw = p.V - p.v0 < C ? p.V - p.v0 : C;
    const int64_t nvt = (p.cw + CfgNT::BN - 1) / CfgNT::BN;
    const int64_t kz = (p.cw + 7) / 8 * 8;  // reduction length of dh: the zero-padded chunk width
    if (ntt * nvt <= kLinHalfRound)
      hipLaunchKernelGGL((lin_dz_kernel<CfgNTs>), dim3((uint32_t)(ntt_s * nvt)), dim3(CfgNTs::NT),
                         lds_bytes<CfgNTs>(), stream, p);
    else
      hipLaunchKernelGGL((lin_dz_kernel<CfgNT>), dim3((uint32_t)(ntt * nvt)), dim3(CfgNT::NT), lds_bytes<CfgNT>(),
                         stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t plane = p.dzl - p.dzh;
    // dW[v0 + v, k] = sum_n dz[n, v] h[n, k]: A(v, n) = dz[n, v] (KROW pair; its rows are the
    // zero-padded width kz, so that every 8-row load stays inside the planes), B(k, n) = h[n, k] (KROW)
    const GemmArgs gw{Operand{p.dzh, p.ldc, kz, p.N, plane}, Operand{p.h, p.ldh, p.H, p.N}, dW ? dW + p.v0 * p.H : nullptr, nullptr,
                      p.H, p.cw, p.H, p.N, kDhStore};
    const int64_t nbw = nvt * nht;
    // dh[n, k] += sum_v dz[n, v] W[v0 + v, k]: A = dz (ROWK pair), B(k, v) = W[v0 + v, k] (KROW)
    const int32_t mode = nchunks == 1 ? kDhStore : (c == 0 ? kDhFirst : (c + 1 < nchunks ? kDhAdd : kDhLast));
    GemmArgs gh{Operand{p.dzh, p.ldc, p.N, kz, plane}, Operand{p.W + p.v0 * p.ldw, p.ldw, p.H, p.cw}, dh, p.dh_acc,
                p.H, p.N, p.H, kz, mode};
    if (mode == kDhFirst || mode == kDhAdd) gh.ldc = p.H;
    if (dW && dh && !dh_small && nbw % 8 == 0) {
      static_assert(CfgTN2::LDS_BYTES == CfgNN2::LDS_BYTES, "one LDS size");
      hipLaunchKernelGGL((gemm_pair2_kernel<CfgTN2, CfgNN2>), dim3((uint32_t)(nbw + ntt * nht)), dim3(CfgTN2::NT),
                         lds_bytes<CfgTN2>(), stream, gw, gh, nbw);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      continue;
    }
    if (dW) {
      hipLaunchKernelGGL((gemm_pair_kernel<CfgTN2>), dim3((uint32_t)nbw), dim3(CfgTN2::NT), lds_bytes<CfgTN2>(),
                         stream, gw);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (dh) {
      if (dh_small)
        hipLaunchKernelGGL((gemm_pair_kernel<CfgNN2s>), dim3((uint32_t)(ntt_s * nht)), dim3(CfgNN2s::NT),
                           lds_bytes<CfgNN2s>(), stream, gh);
      else
        hipLaunchKernelGGL((gemm_pair_kernel<CfgNN2>), dim3((uint32_t)(ntt * nht)), dim3(CfgNN2::NT),
                           lds_bytes<CfgNN2>(), stream, gh);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

size_t lin_fwd_lds_bytes() { return lds_bytes<CfgFwd>(); }

}  // namespace vws
