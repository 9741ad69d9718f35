// launch.h -- kernel argument blocks and launchers shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "gemm.h"

namespace vws {

template <int DT>
struct DtypeTag {
  static constexpr int value = DT;
};

// Calls f(DtypeTag<DT>{}) for the logits dtype code (kF32, kBF16 or kF16).
template <class F>
hipError_t dispatch_dtype(int dtype, F&& f) {
  switch (dtype) {
    case kBF16: return f(DtypeTag<kBF16>{});
    case kF16: return f(DtypeTag<kF16>{});
    default: return f(DtypeTag<kF32>{});
  }
}

struct FwdArgs {
  RowsDev a, b;  // b used by KL only
  IdsDev ids;    // logprobs only
  int64_t N, V, ignore_index;
  int32_t parts, groups_per_part;  // vocabulary split: part p covers groups [p*gpp, (p+1)*gpp)
  float* out;                      // [N]
  float* stats;                    // [N, 2] or [N, 4]
  float* ws;                       // [N, parts, 3 or 6] partial states when parts > 1
  // multi-id logprobs in the unsplit forward: K ids per row (1 <= K <= 256) at
  // ids[r_o * s_outer + r_i * s_inner + k * ids_sk], out [N, K]; K = 0 for one id (or none)
  int64_t ids_sk;
  int32_t K;
};

struct BwdArgs {
  RowsDev a, b;
  IdsDev ids;
  int64_t N, V, ignore_index;
  int32_t tiles_per_row;
  const float* stats;  // [N, 2] or [N, 4]
  const float* res;    // H or KL [N]; unused for logprobs
  const float* g;
  int64_t g_stride;
  char* da;  // dz for logprobs / entropy
  char* db;
};

// Multi-id (top-k) logprobs: ids[n, k] at ids[r_o * ids_so + r_i * ids_si + k * ids_sk] with the
// logits' row decomposition; upstream g[n, k] at g[n * g_sr + k * g_sk].
constexpr int kTopkMaxK = 2048;

struct TopkArgs {
  RowsDev a;
  const int64_t* ids;
  int64_t ids_so, ids_si, ids_sk;
  int32_t K;
  int32_t tiles_per_row;
  int64_t N, V, ignore_index;
  const float* stats;  // [N, 2] (m, log S)
  float* out;          // [N, K] contiguous (forward)
  const float* g;      // backward
  int64_t g_sr, g_sk;
  char* dz;  // [N, V] contiguous, dtype of the logits
};

int32_t topk_tiles_per_row(int64_t V, int32_t K, int dtype);
hipError_t launch_topk_gather(const TopkArgs& p, int dtype, hipStream_t stream);
hipError_t launch_topk_bwd(const TopkArgs& p, int dtype, bool vec, hipStream_t stream);

// Generalized JSD (0 < beta < 1) of student s and teacher t.
struct JsdArgs {
  RowsDev s, t;
  int64_t N, V;
  float beta;
  int32_t parts, groups_per_part, tiles_per_row;
  const float* st4;  // [N, 4] (m_s, log S_s, m_t, log S_t) from the statistics pass (forward)
  float* ws2;        // [N, parts, 2] partial (K_S, K_T) when parts > 1
  float* out;        // [N] JSD
  float* stats;      // [N, 6] (m_s, log S_s, m_t, log S_t, K_S, K_T); read by the backward
  const float* g;
  int64_t g_stride;
  char* ds;  // [N, V] contiguous, may be null
  char* dt;  // [N, V] contiguous, may be null
};

int32_t jsd_tiles_per_row(int64_t V, int dtype);
hipError_t launch_jsd_div(const JsdArgs& p, int dtype, bool vec, hipStream_t stream);
hipError_t launch_jsd_bwd(const JsdArgs& p, int dtype, bool vec, hipStream_t stream);

// Fused linear-logp: h [N, H] and W [V, H] bf16 (row strides ldh, ldw), targets t [N].
struct LinArgs {
  const uint16_t* h;
  const uint16_t* W;
  int64_t ldh, ldw, N, H, V;
  const int64_t* t;
  int64_t ignore_index;
  // forward
  float* logp;   // [N]
  float* stats;  // [N, 2] (m, log S); read by the backward
  float* part;   // workspace [N, chunks, 2]
  float* zt;     // workspace [N]
  int32_t chunks, tiles_per_chunk;
  // backward, one vocabulary chunk [v0, v0 + cw) at a time
  const float* g;
  int64_t g_stride;
  uint16_t* dzh;  // workspace [N, ldc] bf16: hi part of the chunk's dz
  uint16_t* dzl;  // workspace [N, ldc] bf16: lo part, dz - hi rounded
  int64_t ldc;    // row pitch of the dz planes (columns [cw, ldc) hold zeros)
  int64_t v0, cw;
  float* dh_acc;  // workspace [N, H] fp32: dh summed over the chunks so far (more than one chunk)
};

// Epilogue of the dh contraction of one chunk.
enum DhMode : int { kDhStore = 0, kDhFirst = 1, kDhAdd = 2, kDhLast = 3 };

struct GemmArgs {
  gemm::Operand A, B;
  uint16_t* C;     // bf16 output, row pitch ldc
  float* acc;      // fp32 running sum (dh over chunks), row pitch ldc
  int64_t ldc, M, Nc, K;
  int32_t mode;    // DhMode for dh; kDhStore for dW
};

// Forward vocabulary chunking; split_hint as for the logits ops (0 automatic, >= 1 that many
// chunks, -1 fixed 1024-column chunks).
int32_t lin_tiles_per_chunk(int64_t N, int64_t V, int split_hint);
int lin_chunks(int64_t N, int64_t V, int split_hint);
hipError_t launch_lin_fwd(LinArgs p, int split_hint, hipStream_t stream);
// Backward vocabulary chunking: tiles of 256 columns per chunk (split_hint 0 or -1: 32 tiles, a
// function of nothing; k >= 1: k chunks), and the workspace layout built on it.
int32_t lin_bwd_tiles_per_chunk(int64_t V, int split_hint);
hipError_t launch_lin_bwd(LinArgs p, int split_hint, uint16_t* dh, uint16_t* dW, hipStream_t stream);

// Workgroups per launch: kernels loop over virtual blocks beyond this, which
// keeps grid size x workgroup size below the 2^32 work-item limit.
inline int64_t grid_cap(int64_t blocks) { return blocks < (1 << 20) ? (blocks > 0 ? blocks : 1) : (1 << 20); }

// wide: 512-lane workgroups instead of 256 (a different element-to-lane map, so other rounding).
hipError_t launch_fwd(int op, const FwdArgs& p, int dtype, bool vec, bool wide, hipStream_t stream);
hipError_t launch_bwd(int op, const BwdArgs& p, int dtype, bool vec, hipStream_t stream);
int32_t bwd_tiles_per_row(int op, int dtype, int64_t V);

}  // namespace vws
