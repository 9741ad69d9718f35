// api.hip -- the C ABI of libvws (declared in include/vws.h): argument and
// layout validation on the host, then asynchronous launches on the caller's
// stream. Nothing here allocates or synchronises; the only state is the static
// scratch buffer of vws_kl_fwd_noalloc and its per-device address.
#include <limits.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "launch.h"
#include "vws.h"

// Scratch of vws_kl_fwd_noalloc: the split path's partial states go here instead of into a
// caller-supplied workspace. Each GPU the library runs on holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory: host code uses only
// the device address that hipGetSymbolAddress returns for it (kept per device below).
static __device__ __align__(256) float scratch[VWS_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, resolved once per device with that device
// current (the calling thread's current device is the one the caller launches on).
int scratch_addr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VWS_EHIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VWS_EHIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return VWS_OK;
}

using vws::BwdArgs;
using vws::FwdArgs;

int elem_size(int dtype) { return dtype == VWS_F32 ? 4 : 2; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Validates one logits descriptor; on success *N is its row count.
int check_rows(const vws_rows* r, int64_t* N) {
  if (!r) return VWS_EINVAL;
  if (r->dtype != VWS_F32 && r->dtype != VWS_BF16 && r->dtype != VWS_F16) return VWS_EDTYPE;
  if (r->n_outer < 0 || r->n_inner < 0 || r->V < 1) return VWS_EINVAL;
  if (r->V > (int64_t)INT32_MAX - 4096) return VWS_EINVAL;  // column and group indexes are 32-bit
  if (r->col_stride != 1) return VWS_ELAYOUT;
  if (r->s_outer < 0 || r->s_inner < 0) return VWS_ELAYOUT;
  int64_t n;
  if (!mul_ok(r->n_outer, r->n_inner, &n)) return VWS_EINVAL;
  if (n > ((int64_t)1 << 40)) return VWS_EINVAL;
  *N = n;
  if (n == 0) return VWS_OK;
  if (!r->data) return VWS_EINVAL;
  const int es = elem_size(r->dtype);
  if (!aligned(r->data, (uintptr_t)es)) return VWS_ELAYOUT;
  // last element touched: (n_outer-1) s_outer + (n_inner-1) s_inner + V - 1, in bytes
  int64_t o1, o2, last;
  if (!mul_ok(r->n_outer - 1, r->s_outer, &o1) || !mul_ok(r->n_inner - 1, r->s_inner, &o2)) return VWS_ELAYOUT;
  if (o1 > INT64_MAX - o2) return VWS_ELAYOUT;
  last = o1 + o2;
  if (last > INT64_MAX - r->V) return VWS_ELAYOUT;
  last += r->V;
  if (last > INT64_MAX / es) return VWS_ELAYOUT;
  return VWS_OK;
}

int check_ids(const vws_ids* t) {
  if (!t || !t->data) return VWS_EINVAL;
  if (t->s_outer < 0 || t->s_inner < 0) return VWS_ELAYOUT;
  if (!aligned(t->data, 8)) return VWS_ELAYOUT;
  return VWS_OK;
}

// 16-byte vector loads are legal for every row of r.
bool rows_vec_ok(const vws_rows* r) {
  const int es = elem_size(r->dtype);
  if (!aligned(r->data, 16)) return false;
  if (r->n_outer > 1 && (r->s_outer * es) % 16 != 0) return false;
  if (r->n_inner > 1 && (r->s_inner * es) % 16 != 0) return false;
  return true;
}

bool out_vec_ok(const void* out, int64_t N, int64_t V, int es) {
  if (!out) return true;
  if (!aligned(out, 16)) return false;
  return N <= 1 || (V * es) % 16 == 0;
}

vws::RowsDev rows_dev(const vws_rows* r) {
  return vws::RowsDev{static_cast<const char*>(r->data), r->n_inner > 0 ? r->n_inner : 1, r->s_outer, r->s_inner};
}

vws::IdsDev ids_dev(const vws_ids* t) { return vws::IdsDev{t ? t->data : nullptr, t ? t->s_outer : 0, t ? t->s_inner : 0}; }

int state_floats(int op) { return op == VWS_OP_KL ? 6 : 3; }

// Segment length (in groups of 8 columns) of the batch-invariant split: 32768 columns.
constexpr int64_t kInvariantGroups = 4096;

// Most slots the unsplit forward writes itself (one per lane of its first 256 lanes).
constexpr int64_t kFwdTopkMaxK = 256;

// Forward workgroup width: 512 lanes in the automatic split from kFwdWideRows rows up (rows are
// then never split), 256 otherwise. Measured at V = 75968 bf16 (one-card A/Bs, Infinity Cache
// flushed before each launch, us, 256 -> 512 lanes): 2048 rows logprobs / entropy / KL 57.3 /
// 64.3 / 111.1 -> 54.9 / 56.5 / 104.7, 8192 rows 195 / 196 / 382 -> 193 / 192 / 371, and the
// four-op step 3.50-3.53 -> 3.48-3.49 ms on three cards; at 1024 rows 32.7 / 34.8 / 57.8 ->
// 34.2 / 33.9 / 59.4, so small batches keep 256, and so do the fixed splits, whose 32768-column
// segments leave a 512-lane workgroup two batches a lane (the invariant step 3.56 -> 3.80 ms).
// The width sets a row's element-to-lane map: a fixed split (VWS_SPLIT_INVARIANT, split_hint >= 1)
// always takes 256 lanes, so its bits still depend on V alone.
constexpr int64_t kFwdWideRows = 2048;
bool fwd_wide(int64_t N, int split_hint) { return split_hint == 0 && N >= kFwdWideRows; }

// Vocabulary parts per row for the forward (see vws_split_parts in vws.h).
int parts_for(int op, int64_t N, int64_t V, int hint) {
  const int64_t G = (V + 7) / 8;
  int64_t P;
  if (hint == VWS_SPLIT_INVARIANT) {
    // fixed vocabulary segments of kInvariantGroups groups: the part count, and so
    // every row's reduction order, depends on V alone (batch invariant)
    P = (G + kInvariantGroups - 1) / kInvariantGroups;
  } else if (hint == 1) {
    P = 1;
  } else if (hint > 1) {
    P = hint < G ? hint : G;
  } else {
    // About 768 workgroups (three per CU), keeping every part at least 512 groups
    // (4096 columns) long. Measured at V = 75968 bf16 with the Infinity Cache
    // flushed, a part's fixed cost (the cross-wave merge, the partial state and
    // the combine launch) outweighs more parallelism beyond that: 1024 rows run
    // fastest unsplit (entropy 34.7 us against 47.4 us with 8 parts), 256 rows
    // with 3 parts (17.2 us against 21.2 unsplit and 28.0 with 32 parts).
    const int64_t want = N >= 768 ? 1 : (768 + N - 1) / (N > 0 ? N : 1);
    const int64_t cap = G / 512 > 1 ? G / 512 : 1;
    P = want < cap ? want : cap;
  }
  if (P > 1024) P = 1024;
  if (P < 1) P = 1;
  // no empty parts
  const int64_t gpp = (G + P - 1) / P;
  P = (G + gpp - 1) / gpp;
  (void)op;
  return (int)P;
}

// stats_only (logprobs): write the row statistics but no per-row output, for the multi-id forward.
// static_ws: take the workspace from the library's static scratch (vws_kl_fwd_noalloc) instead of
// ws / ws_bytes.
// topk: multi-id logprobs written by the unsplit forward itself (out [N, K], 1 <= K <= kFwdTopkMaxK;
// the caller checks that the launch is unsplit).
int fwd_common(int op, const vws_rows* a, const vws_rows* b, const vws_ids* t, int64_t ignore_index, float* out,
               float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream, bool stats_only = false,
               bool static_ws = false, const vws_ids_k* topk = nullptr) {
  int64_t N, Nb;
  int rc = check_rows(a, &N);
  if (rc) return rc;
  if (op == VWS_OP_KL) {
    if ((rc = check_rows(b, &Nb))) return rc;
    if (b->dtype != a->dtype) return VWS_EDTYPE;
    if (Nb != N || b->V != a->V || b->n_inner != a->n_inner) return VWS_EINVAL;
  }
  if (split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if (op == VWS_OP_LOGPROBS && !stats_only && !topk && (rc = check_ids(t))) return rc;
  if ((!out && !stats_only) || !stats) return VWS_EINVAL;
  if (!aligned(out, 4) || !aligned(stats, 4)) return VWS_ELAYOUT;
  const int P = parts_for(op, N, a->V, split_hint);
  if (N * (int64_t)P > (int64_t)INT32_MAX) return VWS_EINVAL;
  const size_t need = P > 1 ? (size_t)N * (size_t)P * (size_t)state_floats(op) * sizeof(float) : 0;
  if (static_ws) {
    if (need > (size_t)VWS_NOALLOC_SCRATCH_BYTES) return VWS_ESCRATCH;
    ws = nullptr;
    ws_bytes = 0;
    if (need > 0) {
      if ((rc = scratch_addr(&ws))) return rc;
      ws_bytes = (size_t)VWS_NOALLOC_SCRATCH_BYTES;
    }
  }
  if (need > 0 && (!ws || ws_bytes < need)) return VWS_EWORKSPACE;
  if (need > 0 && !aligned(ws, 4)) return VWS_ELAYOUT;

  FwdArgs p{};
  p.a = rows_dev(a);
  if (op == VWS_OP_KL) p.b = rows_dev(b);
  p.ids = ids_dev(op == VWS_OP_LOGPROBS && !stats_only ? t : nullptr);
  if (topk) {
    p.ids = vws::IdsDev{topk->data, topk->s_outer, topk->s_inner};
    p.ids_sk = topk->s_k;
    p.K = (int32_t)topk->K;
  }
  p.N = N;
  p.V = a->V;
  p.ignore_index = ignore_index;
  p.parts = P;
  const int64_t G = (a->V + 7) / 8;
  p.groups_per_part = (int32_t)((G + P - 1) / P);
  p.out = stats_only ? nullptr : out;
  p.stats = stats;
  p.ws = static_cast<float*>(ws);
  const bool vec = rows_vec_ok(a) && (op != VWS_OP_KL || rows_vec_ok(b));
  hipError_t e = vws::launch_fwd(op, p, a->dtype, vec, fwd_wide(N, split_hint), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

int bwd_common(int op, const vws_rows* a, const vws_rows* b, const vws_ids* t, int64_t ignore_index,
               const float* stats, const float* res, const float* g, int64_t g_stride, void* da, void* db,
               void* stream) {
  int64_t N, Nb;
  int rc = check_rows(a, &N);
  if (rc) return rc;
  if (op == VWS_OP_KL) {
    if ((rc = check_rows(b, &Nb))) return rc;
    if (b->dtype != a->dtype) return VWS_EDTYPE;
    if (Nb != N || b->V != a->V || b->n_inner != a->n_inner) return VWS_EINVAL;
  }
  if (g_stride < 0) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if (op == VWS_OP_LOGPROBS && (rc = check_ids(t))) return rc;
  if (!stats || !g || (op != VWS_OP_LOGPROBS && !res)) return VWS_EINVAL;
  if (op != VWS_OP_KL && !da) return VWS_EINVAL;
  if (op == VWS_OP_KL && !da && !db) return VWS_OK;
  if (!aligned(stats, 4) || !aligned(g, 4) || (res && !aligned(res, 4))) return VWS_ELAYOUT;
  const int es = elem_size(a->dtype);
  if (!aligned(da, es) || !aligned(db, es)) return VWS_ELAYOUT;
  int64_t nv, bytes;
  if (!mul_ok(N, a->V, &nv) || !mul_ok(nv, es, &bytes)) return VWS_EINVAL;
  const int32_t tpr = vws::bwd_tiles_per_row(op, a->dtype, a->V);
  if (N * (int64_t)tpr > (int64_t)INT32_MAX) return VWS_EINVAL;

  BwdArgs p{};
  p.a = rows_dev(a);
  if (op == VWS_OP_KL) p.b = rows_dev(b);
  p.ids = ids_dev(op == VWS_OP_LOGPROBS ? t : nullptr);
  p.N = N;
  p.V = a->V;
  p.ignore_index = ignore_index;
  p.tiles_per_row = tpr;
  p.stats = stats;
  p.res = res;
  p.g = g;
  p.g_stride = g_stride;
  p.da = static_cast<char*>(da);
  p.db = static_cast<char*>(db);
  const bool vec = rows_vec_ok(a) && (op != VWS_OP_KL || rows_vec_ok(b)) && out_vec_ok(da, N, a->V, es) &&
                   out_vec_ok(db, N, a->V, es);
  hipError_t e = vws::launch_bwd(op, p, a->dtype, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

int check_ids_k(const vws_ids_k* t) {
  if (!t || !t->data) return VWS_EINVAL;
  if (t->K < 1 || t->K > vws::kTopkMaxK) return VWS_EINVAL;
  if (t->s_outer < 0 || t->s_inner < 0 || t->s_k < 0) return VWS_ELAYOUT;
  if (!aligned(t->data, 8)) return VWS_ELAYOUT;
  return VWS_OK;
}

vws::TopkArgs topk_args(const vws_rows* z, const vws_ids_k* t, int64_t N, int64_t ignore_index) {
  vws::TopkArgs p{};
  p.a = rows_dev(z);
  p.ids = t->data;
  p.ids_so = t->s_outer;
  p.ids_si = t->s_inner;
  p.ids_sk = t->s_k;
  p.K = (int32_t)t->K;
  p.N = N;
  p.V = z->V;
  p.ignore_index = ignore_index;
  return p;
}

// JSD forward workspace: statistics [N, 4], then the statistics pass's partial states
// [N, P, 6] and the divergence pass's partial sums [N, P, 2] when P > 1.
size_t jsd_ws_bytes(int64_t N, int P) {
  return (size_t)N * 4 * sizeof(float) + (P > 1 ? (size_t)N * (size_t)P * 8 * sizeof(float) : 0);
}

// Shared checks of the two JSD inputs; *N is the row count.
int jsd_check_pair(const vws_rows* s, const vws_rows* t, int64_t* N) {
  int64_t Nt;
  int rc = check_rows(s, N);
  if (rc) return rc;
  if ((rc = check_rows(t, &Nt))) return rc;
  if (t->dtype != s->dtype) return VWS_EDTYPE;
  if (Nt != *N || t->V != s->V || t->n_inner != s->n_inner) return VWS_EINVAL;
  return VWS_OK;
}

int64_t round_up8(int64_t x) { return (x + 7) / 8 * 8; }

constexpr int64_t kLinMaxBlocks = (int64_t)1 << 23;  // 512-thread workgroups per linear-logp launch

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Backward vocabulary chunk: width in columns and pitch of the dz planes.
int64_t lin_bwd_chunk(int64_t V, int split_hint) { return (int64_t)vws::lin_bwd_tiles_per_chunk(V, split_hint) * 256; }
int64_t lin_bwd_ldc(int64_t V, int split_hint) {
  const int64_t c = lin_bwd_chunk(V, split_hint);
  return c < round_up8(V) ? c : round_up8(V);
}

// Workspace layout of the fused linear-logp.
//   forward:  part [N, chunks, 2] fp32, then zt [N] fp32
//   backward: the chunk's dz as a bf16 pair, hi [N, ldc] then lo [N, ldc] (each 256-byte
//             aligned), then, with more than one chunk, the fp32 running sum of dh [N, H]
size_t lin_ws_bytes(int pass, int64_t N, int64_t H, int64_t V, int split_hint) {
  if (pass == 0) {
    const size_t part = (size_t)N * (size_t)vws::lin_chunks(N, V, split_hint) * 2 * sizeof(float);
    return align256(part) + (size_t)N * sizeof(float);
  }
  const size_t plane = align256((size_t)N * (size_t)lin_bwd_ldc(V, split_hint) * 2);
  const bool multi = lin_bwd_chunk(V, split_hint) < V;
  return 2 * plane + (multi ? (size_t)N * (size_t)H * sizeof(float) : 0);
}

int lin_check(const void* h, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t N, int64_t H, int64_t V,
              const int64_t* t) {
  if (dtype != VWS_BF16) return VWS_EDTYPE;
  if (N < 0 || H < 1 || V < 1) return VWS_EINVAL;
  if (V > (int64_t)INT32_MAX || H > (int64_t)INT32_MAX || N > ((int64_t)1 << 31)) return VWS_EINVAL;
  if (ldh < H || ldw < H || ldh % 8 || ldw % 8 || H % 8) return VWS_ELAYOUT;
  if (N == 0) return VWS_OK;
  if (!h || !W || !t) return VWS_EINVAL;
  if (!aligned(h, 16) || !aligned(W, 16) || !aligned(t, 8)) return VWS_ELAYOUT;
  int64_t x;
  if (!mul_ok(N, ldh, &x) || !mul_ok(V, ldw, &x) || !mul_ok(N, round_up8(V), &x)) return VWS_EINVAL;
  // every launch has one 512-thread workgroup per 256 x 256 tile and a launch holds fewer than
  // 2^32 work-items: (token, vocabulary) tiles for dz, (token, hidden) for dh, (vocabulary,
  // hidden) for dW, and (token tile, chunk) pairs for the forward (at most the first)
  const int64_t ntt = (N + 255) / 256, nvt = (V + 255) / 256, nht = (H + 255) / 256;
  if (ntt * nvt >= kLinMaxBlocks || ntt * nht >= kLinMaxBlocks || nvt * nht >= kLinMaxBlocks) return VWS_EINVAL;
  return VWS_OK;
}

}  // namespace

extern "C" {

VWS_API size_t vws_linear_workspace_bytes(int pass, int64_t N, int64_t H, int64_t V, int split_hint) {
  if ((pass != 0 && pass != 1) || N < 0 || H < 1 || V < 1 || split_hint < VWS_SPLIT_INVARIANT) return (size_t)-1;
  if (N == 0) return 0;
  return lin_ws_bytes(pass, N, H, V, split_hint);
}

VWS_API int vws_linear_logp_fwd(const void* h, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t N,
                                int64_t H, int64_t V, const int64_t* t, int64_t ignore_index, float* logp,
                                float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream) {
  if (split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  int rc = lin_check(h, ldh, W, ldw, dtype, N, H, V, t);
  if (rc) return rc;
  if (N == 0) return VWS_OK;
  if (!logp || !stats) return VWS_EINVAL;
  if (!aligned(logp, 4) || !aligned(stats, 4)) return VWS_ELAYOUT;
  const size_t need = lin_ws_bytes(0, N, H, V, split_hint);
  if (!ws || ws_bytes < need) return VWS_EWORKSPACE;
  if (!aligned(ws, 16)) return VWS_ELAYOUT;
  vws::LinArgs p{};
  p.h = static_cast<const uint16_t*>(h);
  p.W = static_cast<const uint16_t*>(W);
  p.ldh = ldh;
  p.ldw = ldw;
  p.N = N;
  p.H = H;
  p.V = V;
  p.t = t;
  p.ignore_index = ignore_index;
  p.logp = logp;
  p.stats = stats;
  const size_t part = (size_t)N * (size_t)vws::lin_chunks(N, V, split_hint) * 2 * sizeof(float);
  p.part = static_cast<float*>(ws);
  p.zt = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(part));
  hipError_t e = vws::launch_lin_fwd(p, split_hint, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

VWS_API int vws_linear_logp_bwd(const void* h, int64_t ldh, const void* W, int64_t ldw, int dtype, int64_t N,
                                int64_t H, int64_t V, const int64_t* t, int64_t ignore_index, const float* stats,
                                const float* g, int64_t g_stride, void* dh, void* dW, void* ws, size_t ws_bytes,
                                int split_hint, void* stream) {
  int rc = lin_check(h, ldh, W, ldw, dtype, N, H, V, t);
  if (rc) return rc;
  if (g_stride < 0 || split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  if (N == 0 || (!dh && !dW)) return VWS_OK;
  if (!stats || !g) return VWS_EINVAL;
  if (!aligned(stats, 4) || !aligned(g, 4) || !aligned(dh, 16) || !aligned(dW, 16)) return VWS_ELAYOUT;
  const size_t need = lin_ws_bytes(1, N, H, V, split_hint);
  if (!ws || ws_bytes < need) return VWS_EWORKSPACE;
  if (!aligned(ws, 256)) return VWS_ELAYOUT;
  vws::LinArgs p{};
  p.h = static_cast<const uint16_t*>(h);
  p.W = static_cast<const uint16_t*>(W);
  p.ldh = ldh;
  p.ldw = ldw;
  p.N = N;
  p.H = H;
  p.V = V;
  p.t = t;
  p.ignore_index = ignore_index;
  p.stats = const_cast<float*>(stats);
  p.g = g;
  p.g_stride = g_stride;
  const int64_t ldc = lin_bwd_ldc(V, split_hint);
  const size_t plane = align256((size_t)N * (size_t)ldc * 2);
  p.dzh = static_cast<uint16_t*>(ws);
  p.dzl = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + plane);
  p.ldc = ldc;
  p.dh_acc = lin_bwd_chunk(V, split_hint) < V ? reinterpret_cast<float*>(static_cast<char*>(ws) + 2 * plane) : nullptr;
  hipError_t e = vws::launch_lin_bwd(p, split_hint, static_cast<uint16_t*>(dh), static_cast<uint16_t*>(dW),
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}


VWS_API size_t vws_workspace_bytes(int op, int64_t N, int64_t V, int split_hint) {
  if (op < VWS_OP_LOGPROBS || op > VWS_OP_JSD || N < 0 || V < 1 || split_hint < VWS_SPLIT_INVARIANT) return (size_t)-1;
  if (N == 0) return 0;
  const int P = parts_for(op, N, V, split_hint);
  if (op == VWS_OP_JSD) return jsd_ws_bytes(N, P);
  return P > 1 ? (size_t)N * (size_t)P * (size_t)state_floats(op) * sizeof(float) : 0;
}

VWS_API int vws_split_parts(int op, int64_t N, int64_t V, int split_hint) {
  if (op < VWS_OP_LOGPROBS || op > VWS_OP_JSD || N < 0 || V < 1 || split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  return parts_for(op, N, V, split_hint);
}

VWS_API int vws_logprobs_fwd(const vws_rows* z, const vws_ids* t, int64_t ignore_index, float* logp, float* stats,
                             void* ws, size_t ws_bytes, int split_hint, void* stream) {
  return fwd_common(VWS_OP_LOGPROBS, z, nullptr, t, ignore_index, logp, stats, ws, ws_bytes, split_hint, stream);
}

VWS_API int vws_logprobs_bwd(const vws_rows* z, const vws_ids* t, int64_t ignore_index, const float* stats,
                             const float* g, int64_t g_stride, void* dz, void* stream) {
  return bwd_common(VWS_OP_LOGPROBS, z, nullptr, t, ignore_index, stats, nullptr, g, g_stride, dz, nullptr, stream);
}

VWS_API int vws_entropy_fwd(const vws_rows* z, float* H, float* stats, void* ws, size_t ws_bytes, int split_hint,
                            void* stream) {
  return fwd_common(VWS_OP_ENTROPY, z, nullptr, nullptr, 0, H, stats, ws, ws_bytes, split_hint, stream);
}

VWS_API int vws_entropy_bwd(const vws_rows* z, const float* stats, const float* H, const float* g, int64_t g_stride,
                            void* dz, void* stream) {
  return bwd_common(VWS_OP_ENTROPY, z, nullptr, nullptr, 0, stats, H, g, g_stride, dz, nullptr, stream);
}

VWS_API int vws_kl_fwd(const vws_rows* a, const vws_rows* b, float* kl, float* stats, void* ws, size_t ws_bytes,
                       int split_hint, void* stream) {
  return fwd_common(VWS_OP_KL, a, b, nullptr, 0, kl, stats, ws, ws_bytes, split_hint, stream);
}

VWS_API int vws_kl_fwd_noalloc(const vws_rows* a, const vws_rows* b, float* kl, float* stats, int split_hint,
                               void* stream) {
  return fwd_common(VWS_OP_KL, a, b, nullptr, 0, kl, stats, nullptr, 0, split_hint, stream, false, true);
}

VWS_API int vws_kl_bwd(const vws_rows* a, const vws_rows* b, const float* stats, const float* kl, const float* g,
                       int64_t g_stride, void* da, void* db, void* stream) {
  return bwd_common(VWS_OP_KL, a, b, nullptr, 0, stats, kl, g, g_stride, da, db, stream);
}

VWS_API int vws_logprobs_topk_fwd(const vws_rows* z, const vws_ids_k* ids, int64_t ignore_index, float* logp,
                                  float* stats, void* ws, size_t ws_bytes, int split_hint, void* stream) {
  int64_t N;
  int rc = check_rows(z, &N);
  if (rc) return rc;
  if (split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if ((rc = check_ids_k(ids))) return rc;
  if (!logp || !stats) return VWS_EINVAL;
  if (!aligned(logp, 4)) return VWS_ELAYOUT;
  int64_t nk;
  if (!mul_ok(N, ids->K, &nk)) return VWS_EINVAL;
  // Unsplit rows with up to 256 slots: the forward writes the slots itself (their logits read
  // before the row's stream); otherwise the statistics pass, then one gather launch.
  const bool fused = parts_for(VWS_OP_LOGPROBS, N, z->V, split_hint) == 1 && ids->K <= kFwdTopkMaxK;
  rc = fwd_common(VWS_OP_LOGPROBS, z, nullptr, nullptr, ignore_index, fused ? logp : nullptr, stats, ws, ws_bytes,
                  split_hint, stream, !fused, false, fused ? ids : nullptr);
  if (rc || fused) return rc;
  vws::TopkArgs p = topk_args(z, ids, N, ignore_index);
  p.stats = stats;
  p.out = logp;
  hipError_t e = vws::launch_topk_gather(p, z->dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

VWS_API int vws_logprobs_topk_bwd(const vws_rows* z, const vws_ids_k* ids, int64_t ignore_index, const float* stats,
                                  const float* g, int64_t g_s_row, int64_t g_s_k, void* dz, void* stream) {
  int64_t N;
  int rc = check_rows(z, &N);
  if (rc) return rc;
  if (g_s_row < 0 || g_s_k < 0) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if ((rc = check_ids_k(ids))) return rc;
  if (!stats || !g || !dz) return VWS_EINVAL;
  const int es = elem_size(z->dtype);
  if (!aligned(stats, 4) || !aligned(g, 4) || !aligned(dz, es)) return VWS_ELAYOUT;
  int64_t nv, bytes;
  if (!mul_ok(N, z->V, &nv) || !mul_ok(nv, es, &bytes)) return VWS_EINVAL;
  const int32_t tpr = vws::topk_tiles_per_row(z->V, (int32_t)ids->K, z->dtype);
  if (N * (int64_t)tpr > (int64_t)INT32_MAX) return VWS_EINVAL;
  vws::TopkArgs p = topk_args(z, ids, N, ignore_index);
  p.tiles_per_row = tpr;
  p.stats = stats;
  p.g = g;
  p.g_sr = g_s_row;
  p.g_sk = g_s_k;
  p.dz = static_cast<char*>(dz);
  const bool vec = rows_vec_ok(z) && out_vec_ok(dz, N, z->V, es);
  hipError_t e = vws::launch_topk_bwd(p, z->dtype, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

VWS_API int vws_jsd_fwd(const vws_rows* s, const vws_rows* t, float beta, float* jsd, float* stats, void* ws,
                        size_t ws_bytes, int split_hint, void* stream) {
  if (!(beta >= 0.0f && beta <= 1.0f)) return VWS_EINVAL;
  // endpoint branches: forward KL(T||S) and reverse KL(S||T)
  if (beta == 0.0f) return fwd_common(VWS_OP_KL, t, s, nullptr, 0, jsd, stats, ws, ws_bytes, split_hint, stream);
  if (beta == 1.0f) return fwd_common(VWS_OP_KL, s, t, nullptr, 0, jsd, stats, ws, ws_bytes, split_hint, stream);
  int64_t N;
  int rc = jsd_check_pair(s, t, &N);
  if (rc) return rc;
  if (split_hint < VWS_SPLIT_INVARIANT) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if (!jsd || !stats) return VWS_EINVAL;
  if (!aligned(jsd, 4) || !aligned(stats, 4)) return VWS_ELAYOUT;
  const int P = parts_for(VWS_OP_JSD, N, s->V, split_hint);
  if (N * (int64_t)P > (int64_t)INT32_MAX) return VWS_EINVAL;
  if (!ws || ws_bytes < jsd_ws_bytes(N, P)) return VWS_EWORKSPACE;
  if (!aligned(ws, 4)) return VWS_ELAYOUT;
  float* st4 = static_cast<float*>(ws);
  float* part1 = st4 + 4 * N;
  float* part2 = part1 + (P > 1 ? N * (int64_t)P * 6 : 0);
  // pass 1: (m, log S) of both inputs in one read (the KL forward, statistics only)
  rc = fwd_common(VWS_OP_KL, s, t, nullptr, 0, nullptr, st4, part1, P > 1 ? (size_t)N * P * 6 * sizeof(float) : 0,
                  split_hint, stream, true);
  if (rc) return rc;
  // pass 2: K_S and K_T, then JSD = beta K_T + (1 - beta) K_S
  vws::JsdArgs p{};
  p.s = rows_dev(s);
  p.t = rows_dev(t);
  p.N = N;
  p.V = s->V;
  p.beta = beta;
  p.parts = P;
  const int64_t G = (s->V + 7) / 8;
  p.groups_per_part = (int32_t)((G + P - 1) / P);
  p.st4 = st4;
  p.ws2 = part2;
  p.out = jsd;
  p.stats = stats;
  const bool vec = rows_vec_ok(s) && rows_vec_ok(t);
  hipError_t e = vws::launch_jsd_div(p, s->dtype, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

VWS_API int vws_jsd_bwd(const vws_rows* s, const vws_rows* t, float beta, const float* stats, const float* jsd,
                        const float* g, int64_t g_stride, void* ds, void* dt, void* stream) {
  if (!(beta >= 0.0f && beta <= 1.0f)) return VWS_EINVAL;
  if (beta == 0.0f) return bwd_common(VWS_OP_KL, t, s, nullptr, 0, stats, jsd, g, g_stride, dt, ds, stream);
  if (beta == 1.0f) return bwd_common(VWS_OP_KL, s, t, nullptr, 0, stats, jsd, g, g_stride, ds, dt, stream);
  int64_t N;
  int rc = jsd_check_pair(s, t, &N);
  if (rc) return rc;
  if (g_stride < 0) return VWS_EINVAL;
  if (N == 0) return VWS_OK;
  if (!stats || !jsd || !g) return VWS_EINVAL;
  if (!ds && !dt) return VWS_OK;
  const int es = elem_size(s->dtype);
  if (!aligned(stats, 4) || !aligned(g, 4) || !aligned(ds, es) || !aligned(dt, es)) return VWS_ELAYOUT;
  int64_t nv, bytes;
  if (!mul_ok(N, s->V, &nv) || !mul_ok(nv, es, &bytes)) return VWS_EINVAL;
  const int32_t tpr = vws::jsd_tiles_per_row(s->V, s->dtype);
  if (N * (int64_t)tpr > (int64_t)INT32_MAX) return VWS_EINVAL;
  vws::JsdArgs p{};
  p.s = rows_dev(s);
  p.t = rows_dev(t);
  p.N = N;
  p.V = s->V;
  p.beta = beta;
  p.tiles_per_row = tpr;
  p.stats = const_cast<float*>(stats);
  p.g = g;
  p.g_stride = g_stride;
  p.ds = static_cast<char*>(ds);
  p.dt = static_cast<char*>(dt);
  const bool vec = rows_vec_ok(s) && rows_vec_ok(t) && out_vec_ok(ds, N, s->V, es) && out_vec_ok(dt, N, s->V, es);
  hipError_t e = vws::launch_jsd_bwd(p, s->dtype, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VWS_OK : VWS_EHIP;
}

VWS_API const char* vws_strerror(int status) {
  switch (status) {
    case VWS_OK: return "ok";
    case VWS_EINVAL: return "invalid argument (null pointer, negative or inconsistent size)";
    case VWS_EDTYPE: return "unsupported or mismatched dtype";
    case VWS_ELAYOUT: return "unsupported layout (col_stride != 1, negative stride, misaligned pointer or address overflow)";
    case VWS_EWORKSPACE: return "workspace too small";
    case VWS_EHIP: return "HIP launch failed";
    case VWS_ESCRATCH: return "the split needs more than the library's static scratch (VWS_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

VWS_API int vws_version(void) { return 103; }

}  // extern "C"
