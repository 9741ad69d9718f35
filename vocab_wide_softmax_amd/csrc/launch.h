// launch.h -- kernel argument blocks and launchers shared by the host API and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace vws {

struct FwdArgs {
  RowsDev a, b;  // b used by KL only
  IdsDev ids;    // logprobs only
  int64_t N, V, ignore_index;
  int32_t parts, groups_per_part;  // vocabulary split: part p covers groups [p*gpp, (p+1)*gpp)
  float* out;                      // [N]
  float* stats;                    // [N, 2] or [N, 4]
  float* ws;                       // [N, parts, 3 or 6] partial states when parts > 1
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

// Workgroups per launch: kernels loop over virtual blocks beyond this, which
// keeps grid size x workgroup size below the 2^32 work-item limit.
inline int64_t grid_cap(int64_t blocks) { return blocks < (1 << 20) ? (blocks > 0 ? blocks : 1) : (1 << 20); }

hipError_t launch_fwd(int op, const FwdArgs& p, int dtype, bool vec, hipStream_t stream);
hipError_t launch_bwd(int op, const BwdArgs& p, int dtype, bool vec, hipStream_t stream);
int32_t bwd_tiles_per_row(int64_t V);

}  // namespace vws
