// C ABI of the library: argument checks, workspace carving and the order of
// kernel launches on the caller's stream.  Declarations and the contract of
// every entry point are in include/vsa.h.
#include "vsa.h"
#include "vsa_launch.h"

#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

using namespace vsa;

namespace {

constexpr size_t kAlign = 256;
// (batch, head, cube) units at most: kernels with one 256-thread workgroup
// per unit launch 1-D grids (rounded up to a multiple of 8 workgroups)
// whose work-item count must stay below 2^32.
constexpr int64_t kMaxCubeUnits = (int64_t(1) << 24) - 8;
constexpr size_t kDsTileBytes = 64 * 64 * 2;  // one bf16 dS tile (64 queries x 64 keys)
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

struct Shape {
  int B, heads, D, T, H, W, dtype;
  int64_t N, nc;
  size_t elt;
};

// Shape checks shared by every entry point; fills `s` on success.
int check_shape(int B, int heads, int D, int T, int H, int W, int dtype, Shape* s) {
  if (B < 1 || heads < 1 || T < 4 || H < 4 || W < 4) return VSA_ERR_INVALID_ARG;
  if (T % 4 || H % 4 || W % 4) return VSA_ERR_INVALID_ARG;  // whole 4x4x4 cubes only
  if (dtype != VSA_F32 && dtype != VSA_BF16) return VSA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return VSA_ERR_UNSUPPORTED;
  const int64_t N = (int64_t)T * H * W;
  const int64_t nc = N / 64;
  if ((int64_t)B * heads > 65535) return VSA_ERR_UNSUPPORTED;  // grid y dimension
  if (N > INT_MAX / 2 || (int64_t)B * heads * nc > kMaxCubeUnits || (int64_t)B * N * heads > INT_MAX)
    return VSA_ERR_UNSUPPORTED;
  if (nc > coarse_max_cubes(D)) return VSA_ERR_UNSUPPORTED;
  *s = Shape{B, heads, D, T, H, W, dtype, N, nc, dtype == VSA_BF16 ? 2u : 4u};
  return VSA_OK;
}

struct FwdWorkspace {
  int32_t* check;  // 2 ints: list validation counts (VSA_VALIDATE)
  void *kp, *vp;
  float *qc, *kc, *vc, *oc, *lse_c;
  int32_t* order;  // processing order of the fine stage's query cubes
};

size_t fwd_ws_layout(const Shape& s, char* base, FwdWorkspace* w) {
  const size_t tile_bytes = align_up((size_t)s.B * s.heads * s.N * s.D * s.elt);
  const size_t pooled = align_up((size_t)s.B * s.heads * s.nc * s.D * sizeof(float));
  // pooled K and V may be held in the packed layouts (keys padded)
  const size_t pooled_kv = align_up((size_t)s.B * s.heads * packed_keys((int)s.nc) * s.D * sizeof(float));
  const size_t lse = align_up((size_t)s.B * s.heads * s.nc * sizeof(float));
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += bytes; return (void*)p; };
  FwdWorkspace t;
  t.check = (int32_t*)take(kAlign);
  t.kp = take(tile_bytes); t.vp = take(tile_bytes);
  t.qc = (float*)take(pooled); t.kc = (float*)take(pooled_kv); t.vc = (float*)take(pooled_kv);
  t.oc = (float*)take(pooled); t.lse_c = (float*)take(lse);
  t.order = (int32_t*)take(align_up((size_t)s.B * s.heads * s.nc * sizeof(int32_t)));
  if (w) *w = t;
  return off;
}

// Forward -> backward state.  Besides the forward's outputs that the
// backward needs (coarse output and log-sum-exp, fine log-sum-exp and fine
// output), the forward leaves its K and V cube tiles and the plain fp32
// cube means of Q, K and V here, so that the backward's permute only has
// to make Q tiles.
struct Saved {
  float *oc, *lse_c, *lse_f, *of;
  void *kp, *vp;
  float *qc, *kc, *vc;
};

size_t saved_layout(const Shape& s, char* base, Saved* sv) {
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += align_up(bytes); return (void*)p; };
  const size_t pooled = (size_t)s.B * s.heads * s.nc * s.D * sizeof(float);
  const size_t tile = (size_t)s.B * s.heads * s.N * s.D * s.elt;
  Saved t;
  t.oc = (float*)take(pooled);
  t.lse_c = (float*)take((size_t)s.B * s.heads * s.nc * sizeof(float));
  t.lse_f = (float*)take((size_t)s.B * s.heads * s.N * sizeof(float));
  t.of = (float*)take((size_t)s.B * s.heads * s.N * s.D * sizeof(float));
  t.kp = take(tile);
  t.vp = take(tile);
  t.qc = (float*)take(pooled);
  t.kc = (float*)take(pooled);
  t.vc = (float*)take(pooled);
  if (sv) *sv = t;
  return off;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_HIP; }

// VSA_VALIDATE=1 in the environment (read at every call): entry points
// that take caller-made key lists check them on the GPU first, wait for the
// answer and return VSA_ERR_INVALID_ARG, queueing nothing more, if any
// precondition fails.  Off by default: the check reads the lists once and
// synchronizes the stream.
bool validate_mode() {
  const char* e = std::getenv("VSA_VALIDATE");
  return e && *e && std::strcmp(e, "0") != 0;
}

// Runs the list check into `slot` (2 ints of device scratch) and waits for
// it.  VSA_OK when the lists are well formed.
int validate_now(const int32_t* offs, const int32_t* ids, int topk, int64_t n_ids, int64_t n_rows,
                 int nc, int32_t* slot, hipStream_t st) {
  if (nc > validate_max_cubes() || n_rows > INT_MAX) return VSA_ERR_UNSUPPORTED;
  if (launch_validate_lists(offs, ids, topk, n_ids, (int)n_rows, nc, slot, st) != hipSuccess)
    return VSA_ERR_HIP;
  int32_t counts[2] = {0, 0};
  if (hipMemcpyAsync(counts, slot, sizeof(counts), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return VSA_ERR_HIP;
  return counts[0] == 0 && counts[1] == 0 ? VSA_OK : VSA_ERR_INVALID_ARG;
}

// Mass-rule selection inside a forward: the coarse stage writes per-row
// lengths and padded lists into the workspace, then they are packed into
// the caller's CSR buffers, which the fine stage reads.
struct MassRule {
  float mass;
  int k_min, k_max;
  int32_t *offsets, *ids;  // caller's CSR output
};

// Workspace beyond the forward's own for the mass rule: counts and padded
// lists.
size_t mass_ws_bytes(const Shape& s, int k_max) {
  const size_t rows = (size_t)s.B * s.heads * s.nc;
  return align_up(rows * sizeof(int32_t)) + align_up(rows * (size_t)k_max * sizeof(int32_t));
}

// Shared body of vsa_forward, block_sparse_attn_varlen and vsa_forward_mass.
int forward_impl(const void* q, const void* k, const void* v, const void* gc, const void* gf,
                 const Shape& s, int topk, const int32_t* offs, const int32_t* ids, int64_t n_ids,
                 int32_t* sel, void* out, void* saved, void* ws, size_t ws_bytes,
                 hipStream_t st, const MassRule* mr = nullptr) {
  FwdWorkspace w;
  const size_t fwd_bytes = fwd_ws_layout(s, nullptr, nullptr);
  if (ws_bytes < fwd_bytes + (mr ? mass_ws_bytes(s, mr->k_max) : 0)) return VSA_ERR_WORKSPACE;
  fwd_ws_layout(s, (char*)ws, &w);
  if (offs && validate_mode()) {  // caller-made lists
    const int vs = validate_now(offs, ids, 0, n_ids, (int64_t)s.B * s.heads * s.nc, (int)s.nc,
                                w.check, st);
    if (vs != VSA_OK) return vs;
  }
  const bool bf = s.dtype == VSA_BF16;
  float *oc = w.oc, *lse_c = w.lse_c, *lse_f = nullptr, *of = nullptr;
  void *kp = w.kp, *vp = w.vp;
  float *qc = w.qc, *kc = w.kc, *vc = w.vc;
  float *plain_k = nullptr, *plain_v = nullptr;
  if (saved) {  // tiles and means go where the backward will read them
    Saved sv;
    saved_layout(s, (char*)saved, &sv);
    oc = sv.oc; lse_c = sv.lse_c; lse_f = sv.lse_f; of = sv.of;
    kp = sv.kp; vp = sv.vp; qc = sv.qc;
    if (bf) { plain_k = sv.kc; plain_v = sv.vc; }  // the coarse stage reads the packed copies
    else { kc = sv.kc; vc = sv.vc; }
  }
  // The fine stage reads Q in place; K and V are copied into cube tiles.
  // bf16: pooled K and V go straight into the coarse kernel's operand order.
  PermutePoolArgs pa{{{q, k, v}, {nullptr, kp, vp}, {qc, kc, vc}, {nullptr, plain_k, plain_v}},
                     s.B, s.heads, s.D, s.T, s.H, s.W, bf};
  pa.packed_kv = bf;
  hipError_t e = launch_permute_pool(pa, st);
  if (e != hipSuccess) return VSA_ERR_HIP;
  CoarseArgs ca{qc, kc, vc, s.B, s.heads, s.D, (int)s.nc, offs ? 0 : topk, oc, lse_c, sel, bf};
  ca.packed = bf;
  const int rows = (int)((int64_t)s.B * s.heads * s.nc);
  int32_t* counts = nullptr;
  int32_t* padded = nullptr;
  if (mr) {
    counts = (int32_t*)((char*)ws + fwd_bytes);
    padded = (int32_t*)((char*)counts + align_up((size_t)rows * sizeof(int32_t)));
    ca.topk = 0;
    ca.sel = padded;
    ca.mass = mr->mass; ca.k_min = mr->k_min; ca.k_max = mr->k_max; ca.counts = counts;
  }
  e = launch_coarse_topk(ca, st);
  if (e != hipSuccess) return VSA_ERR_HIP;
  if (mr) {
    e = launch_pack_lists(counts, padded, rows, mr->k_max, mr->offsets, mr->ids, st);
    if (e != hipSuccess) return VSA_ERR_HIP;
    offs = mr->offsets;
    ids = mr->ids;
    n_ids = (int64_t)rows * mr->k_max;  // capacity; the packed lists end at offsets[rows]
  }
  if (!offs) n_ids = (int64_t)rows * topk;
  FineArgs fa{q, kp, vp, oc, gc, gf, s.B, s.heads, s.D, s.T, s.H, s.W,
              offs, offs ? ids : sel, topk, n_ids, bf, out, lse_f, of};
  if (bf) {  // the MFMA kernel runs the query cubes sorted by where their lists lie
    e = launch_fine_order(fa.offs, fa.ids, topk, n_ids, s.B * s.heads, (int)s.nc, w.order, st);
    if (e != hipSuccess) return VSA_ERR_HIP;
    fa.order = w.order;
  }
  return hip_status(launch_fine_forward(fa, st));
}

struct BwdWorkspace {
  int32_t* check;  // 2 ints: list validation counts (VSA_VALIDATE)
  void *qp, *dofp;
  float *delta, *doc, *deltac, *S, *dP, *dqc, *dkc, *dvc;
  int32_t *tr_offs, *tr_order, *tr_ids, *tr_tmp, *tr_pos, *tr_tmp_pos;
  void* ds;  // bf16: the dS tile of every (query cube, selected key cube) entry
};

size_t bwd_ws_layout(const Shape& s, int64_t n_entries, char* base, BwdWorkspace* w) {
  const size_t tile = align_up((size_t)s.B * s.heads * s.N * s.D * s.elt);
  const size_t pooled = align_up((size_t)s.B * s.heads * s.nc * s.D * sizeof(float));
  const size_t per_tok = align_up((size_t)s.B * s.heads * s.N * sizeof(float));
  const size_t per_cube = align_up((size_t)s.B * s.heads * s.nc * sizeof(float));
  const size_t sq = align_up((size_t)s.B * s.heads * s.nc * s.nc * sizeof(float));
  size_t off = 0;
  auto take = [&](size_t bytes) { char* p = base ? base + off : nullptr; off += bytes; return (void*)p; };
  BwdWorkspace t;
  t.check = (int32_t*)take(kAlign);
  t.qp = take(tile); t.dofp = take(tile);
  t.delta = (float*)take(per_tok);
  t.doc = (float*)take(pooled); t.deltac = (float*)take(per_cube);
  t.S = (float*)take(sq); t.dP = (float*)take(sq);
  t.dqc = (float*)take(pooled); t.dkc = (float*)take(pooled); t.dvc = (float*)take(pooled);
  t.tr_offs = (int32_t*)take(align_up(((size_t)s.B * s.heads * s.nc + 1) * sizeof(int32_t)));
  t.tr_order = (int32_t*)take(align_up((size_t)s.B * s.heads * s.nc * sizeof(int32_t)));
  const size_t per_entry = align_up((size_t)(n_entries > 0 ? n_entries : 1) * sizeof(int32_t));
  t.tr_ids = (int32_t*)take(per_entry);
  t.tr_tmp = (int32_t*)take(per_entry);
  t.tr_pos = t.tr_tmp_pos = nullptr;
  t.ds = nullptr;
  if (s.dtype == VSA_BF16) {
    t.tr_pos = (int32_t*)take(per_entry);
    t.tr_tmp_pos = (int32_t*)take(per_entry);
    t.ds = take(align_up((size_t)(n_entries > 0 ? n_entries : 1) * kDsTileBytes));
  }
  if (w) *w = t;
  return off;
}

int backward_impl(const void* q, const void* k, const void* v, const void* gc, const void* gf,
                  const void* dout, const int32_t* offs, const int32_t* ids, int topk,
                  int64_t n_entries, const void* saved, const Shape& s,
                  void* dq, void* dk, void* dv, void* dgc, void* dgf,
                  void* ws, size_t ws_bytes, hipStream_t st) {
  if (!q || !k || !v || !gc || !gf || !dout || !saved || !ws) return VSA_ERR_INVALID_ARG;
  if (!dq || !dk || !dv || !dgc || !dgf) return VSA_ERR_INVALID_ARG;
  if (ws_bytes < bwd_ws_layout(s, n_entries, nullptr, nullptr)) return VSA_ERR_WORKSPACE;
  BwdWorkspace w;
  bwd_ws_layout(s, n_entries, (char*)ws, &w);
  if (validate_mode()) {  // the lists always come from the caller here
    const int vs = validate_now(offs, ids, topk, n_entries, (int64_t)s.B * s.heads * s.nc,
                                (int)s.nc, w.check, st);
    if (vs != VSA_OK) return vs;
  }
  Saved sv;
  saved_layout(s, (char*)const_cast<void*>(saved), &sv);
  const bool bf = s.dtype == VSA_BF16;
  // Q tiles only: the K and V tiles and all three cube means are the
  // forward's, kept in `saved`.
  PermutePoolArgs pa{{{q, nullptr, nullptr}, {w.qp, nullptr, nullptr}, {nullptr, nullptr, nullptr}},
                     s.B, s.heads, s.D, s.T, s.H, s.W, bf};
  pa.n_tensors = 1;
  if (launch_permute_pool(pa, st) != hipSuccess) return VSA_ERR_HIP;
  BackwardArgs ba;
  ba.B = s.B; ba.heads = s.heads; ba.D = s.D; ba.T = s.T; ba.H = s.H; ba.W = s.W;
  ba.bf16 = bf;
  ba.dout = dout; ba.gc = gc; ba.gf = gf;
  ba.qp = w.qp; ba.kp = sv.kp; ba.vp = sv.vp;
  ba.qc = sv.qc; ba.kc = sv.kc; ba.vc = sv.vc;
  ba.oc = sv.oc; ba.lse_c = sv.lse_c; ba.lse_f = sv.lse_f; ba.of = sv.of;
  ba.offs = offs; ba.ids = ids; ba.topk = topk; ba.n_ids = n_entries;
  ba.delta = w.delta; ba.dofp = w.dofp;
  ba.doc = w.doc; ba.deltac = w.deltac; ba.S = w.S; ba.dP = w.dP;
  ba.dqc = w.dqc; ba.dkc = w.dkc; ba.dvc = w.dvc;
  ba.tr_offs = w.tr_offs; ba.tr_order = w.tr_order; ba.tr_ids = w.tr_ids; ba.tr_tmp = w.tr_tmp;
  ba.tr_pos = w.tr_pos; ba.tr_tmp_pos = w.tr_tmp_pos; ba.ds = w.ds;
  ba.dq = dq; ba.dk = dk; ba.dv = dv; ba.dgc = dgc; ba.dgf = dgf;
  return hip_status(launch_backward(ba, st));
}

// ------------------------------------------------ fixed device scratch
// vsa_forward_noalloc runs the forward with its workspace in this array
// instead of a caller's buffer.  Every GPU the library is loaded on holds
// its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address of each
// GPU's copy is looked up once per device (with that device current) and
// kept in scratch_ptr, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// The copy on the GPU that `st` runs on (the current device for the null
// stream); its address is looked up with that device current.
int device_scratch(hipStream_t st, void** ptr) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return VSA_ERR_HIP;
  if (st) {
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return VSA_ERR_HIP;
  } else {
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxDevices) return VSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return VSA_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return VSA_ERR_HIP;
    if (e != hipSuccess || !p) return VSA_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

const char* vsa_status_string(int status) {
  switch (status) {
    case VSA_OK: return "ok";
    case VSA_ERR_INVALID_ARG: return "invalid argument";
    case VSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case VSA_ERR_WORKSPACE: return "workspace too small";
    case VSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t vsa_forward_workspace_bytes(int B, int heads, int head_dim, int T, int H, int W, int dtype) {
  Shape s;
  if (check_shape(B, heads, head_dim, T, H, W, dtype, &s) != VSA_OK) return 0;
  return fwd_ws_layout(s, nullptr, nullptr);
}

size_t vsa_saved_bytes(int B, int heads, int head_dim, int T, int H, int W, int dtype) {
  Shape s;
  if (check_shape(B, heads, head_dim, T, H, W, dtype, &s) != VSA_OK) return 0;
  return saved_layout(s, nullptr, nullptr);
}

int vsa_forward(const void* q, const void* k, const void* v, const void* gate_c, const void* gate_f,
                int B, int heads, int head_dim, int T, int H, int W, int topk, int dtype,
                void* out, int32_t* sel_idx, void* saved, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !gate_c || !gate_f || !out || !sel_idx || !workspace) return VSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > s.nc) return VSA_ERR_INVALID_ARG;
  if ((int64_t)B * heads * s.nc * topk > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return forward_impl(q, k, v, gate_c, gate_f, s, topk, nullptr, nullptr, 0, sel_idx, out, saved,
                      workspace, workspace_bytes, stream);
}

int vsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gate_c,
                        const void* gate_f, int B, int heads, int head_dim, int T, int H, int W,
                        int topk, int dtype, void* out, int32_t* sel_idx, void* saved,
                        hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !gate_c || !gate_f || !out || !sel_idx) return VSA_ERR_INVALID_ARG;
  if (topk < 1 || topk > s.nc) return VSA_ERR_INVALID_ARG;
  if ((int64_t)B * heads * s.nc * topk > INT_MAX) return VSA_ERR_UNSUPPORTED;
  if (fwd_ws_layout(s, nullptr, nullptr) > kNoAllocScratchBytes) return VSA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = device_scratch(stream, &ws);
  if (st != VSA_OK) return st;
  // Nothing in the forward's workspace has to start at zero: every stage
  // writes what the next one reads.
  return forward_impl(q, k, v, gate_c, gate_f, s, topk, nullptr, nullptr, 0, sel_idx, out, saved, ws,
                      kNoAllocScratchBytes, stream);
}

int block_sparse_attn_varlen(const void* q, const void* k, const void* v,
                             const void* gate_c, const void* gate_f,
                             int B, int heads, int head_dim, int T, int H, int W,
                             const int32_t* kv_offsets, const int32_t* kv_ids,
                             int64_t n_list_entries, int dtype, void* out, void* saved,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !gate_c || !gate_f || !out || !kv_offsets || !workspace) return VSA_ERR_INVALID_ARG;
  if (n_list_entries < 0 || n_list_entries > (int64_t)B * heads * s.nc * s.nc) return VSA_ERR_INVALID_ARG;
  if (n_list_entries > 0 && !kv_ids) return VSA_ERR_INVALID_ARG;
  if (n_list_entries > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return forward_impl(q, k, v, gate_c, gate_f, s, 0, kv_offsets, kv_ids, n_list_entries, nullptr,
                      out, saved, workspace, workspace_bytes, stream);
}

// Argument checks of the mass rule shared by its entry points.
static int check_mass(float mass, int k_min, int k_max, int64_t nc, int64_t rows) {
  if (!(mass > 0.f && mass <= 1.f)) return VSA_ERR_INVALID_ARG;  // also rejects NaN
  if (k_min < 1 || k_min > k_max || k_max > nc) return VSA_ERR_INVALID_ARG;
  if (rows * k_max > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return VSA_OK;
}

size_t vsa_forward_mass_workspace_bytes(int B, int heads, int head_dim, int T, int H, int W,
                                        int dtype, int k_max) {
  Shape s;
  if (check_shape(B, heads, head_dim, T, H, W, dtype, &s) != VSA_OK) return 0;
  if (k_max < 1 || k_max > s.nc || (int64_t)B * heads * s.nc * k_max > INT_MAX) return 0;
  return fwd_ws_layout(s, nullptr, nullptr) + mass_ws_bytes(s, k_max);
}

int vsa_forward_mass(const void* q, const void* k, const void* v, const void* gate_c,
                     const void* gate_f, int B, int heads, int head_dim, int T, int H, int W,
                     float mass, int k_min, int k_max, int dtype, void* out,
                     int32_t* kv_offsets, int32_t* kv_ids, void* saved, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !gate_c || !gate_f || !out || !kv_offsets || !kv_ids || !workspace)
    return VSA_ERR_INVALID_ARG;
  st = check_mass(mass, k_min, k_max, s.nc, (int64_t)B * heads * s.nc);
  if (st != VSA_OK) return st;
  const MassRule mr{mass, k_min, k_max, kv_offsets, kv_ids};
  return forward_impl(q, k, v, gate_c, gate_f, s, 0, nullptr, nullptr, 0, nullptr, out, saved,
                      workspace, workspace_bytes, stream, &mr);
}

int vsa_coarse_select_mass(const float* qc, const float* kc, const float* vc, int B, int heads,
                           int head_dim, int n_cubes, float mass, int k_min, int k_max, int dtype,
                           float* oc, float* lse_c, int32_t* counts, int32_t* ids,
                           hipStream_t stream) {
  if (dtype != VSA_F32 && dtype != VSA_BF16) return VSA_ERR_INVALID_ARG;
  if (B < 1 || heads < 1 || n_cubes < 1) return VSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return VSA_ERR_UNSUPPORTED;
  if (n_cubes > coarse_max_cubes(head_dim) || (int64_t)B * heads > 65535) return VSA_ERR_UNSUPPORTED;
  if (!qc || !kc || !vc || !oc || !lse_c || !counts || !ids) return VSA_ERR_INVALID_ARG;
  if ((int64_t)B * heads * n_cubes > kMaxCubeUnits) return VSA_ERR_UNSUPPORTED;
  const int st = check_mass(mass, k_min, k_max, n_cubes, (int64_t)B * heads * n_cubes);
  if (st != VSA_OK) return st;
  CoarseArgs ca{qc, kc, vc, B, heads, head_dim, n_cubes, 0, oc, lse_c, ids, dtype == VSA_BF16};
  ca.mass = mass; ca.k_min = k_min; ca.k_max = k_max; ca.counts = counts;
  return hip_status(launch_coarse_topk(ca, stream));
}

int vsa_pack_lists(const int32_t* counts, const int32_t* ids_padded, int n_rows, int k_max,
                   int32_t* kv_offsets, int32_t* kv_ids, hipStream_t stream) {
  if (n_rows < 0 || k_max < 1) return VSA_ERR_INVALID_ARG;
  if (!kv_offsets || (n_rows > 0 && (!counts || !ids_padded || !kv_ids))) return VSA_ERR_INVALID_ARG;
  if ((int64_t)n_rows * k_max > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return hip_status(launch_pack_lists(counts, ids_padded, n_rows, k_max, kv_offsets, kv_ids, stream));
}

int vsa_cube_permute_pool(const void* q, const void* k, const void* v,
                          int B, int heads, int head_dim, int T, int H, int W, int dtype,
                          void* qp, void* kp, void* vp, float* qc, float* kc, float* vc,
                          hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !kp || !vp || !qc || !kc || !vc) return VSA_ERR_INVALID_ARG;
  PermutePoolArgs pa{{{q, k, v}, {qp, kp, vp}, {qc, kc, vc}},
                     B, heads, head_dim, T, H, W, dtype == VSA_BF16};
  return hip_status(launch_permute_pool(pa, stream));
}

int vsa_cube_max_pool(const void* q, const void* k, const void* v, int B, int heads, int head_dim,
                      int T, int H, int W, int dtype, float* qc, float* kc, float* vc,
                      hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !k || !v || !qc || !kc || !vc) return VSA_ERR_INVALID_ARG;
  PermutePoolArgs pa{{{q, k, v}, {nullptr, nullptr, nullptr}, {qc, kc, vc}},
                     B, heads, head_dim, T, H, W, dtype == VSA_BF16};
  pa.max_pool = true;
  return hip_status(launch_permute_pool(pa, stream));
}

int vsa_coarse_topk(const float* qc, const float* kc, const float* vc,
                    int B, int heads, int head_dim, int n_cubes, int topk, int dtype,
                    float* oc, float* lse_c, int32_t* sel_idx, hipStream_t stream) {
  if (dtype != VSA_F32 && dtype != VSA_BF16) return VSA_ERR_INVALID_ARG;
  if (B < 1 || heads < 1 || n_cubes < 1) return VSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return VSA_ERR_UNSUPPORTED;
  if (n_cubes > coarse_max_cubes(head_dim) || (int64_t)B * heads > 65535) return VSA_ERR_UNSUPPORTED;
  if (topk < 0 || topk > n_cubes) return VSA_ERR_INVALID_ARG;
  if (!qc || !kc || !vc || !oc || !lse_c || (topk > 0 && !sel_idx)) return VSA_ERR_INVALID_ARG;
  if ((int64_t)B * heads * n_cubes > kMaxCubeUnits || (int64_t)B * heads * n_cubes * topk > INT_MAX)
    return VSA_ERR_UNSUPPORTED;
  CoarseArgs ca{qc, kc, vc, B, heads, head_dim, n_cubes, topk, oc, lse_c, sel_idx, dtype == VSA_BF16};
  return hip_status(launch_coarse_topk(ca, stream));
}

int vsa_fine_forward(const void* q, const void* kp, const void* vp, const float* oc,
                     const void* gate_c, const void* gate_f,
                     int B, int heads, int head_dim, int T, int H, int W,
                     const int32_t* kv_offsets, const int32_t* kv_ids, int64_t n_list_entries,
                     int topk, int dtype, void* out, float* lse_f, float* o_fine,
                     const int32_t* order, hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!q || !kp || !vp || !oc || !gate_c || !gate_f || !out) return VSA_ERR_INVALID_ARG;
  if ((lse_f == nullptr) != (o_fine == nullptr)) return VSA_ERR_INVALID_ARG;
  if (!kv_offsets) {
    if (topk < 1 || topk > s.nc || !kv_ids) return VSA_ERR_INVALID_ARG;
    if ((int64_t)B * heads * s.nc * topk > INT_MAX) return VSA_ERR_UNSUPPORTED;
    n_list_entries = (int64_t)B * heads * s.nc * topk;
  } else {
    if (n_list_entries < 0 || n_list_entries > (int64_t)B * heads * s.nc * s.nc) return VSA_ERR_INVALID_ARG;
    if (n_list_entries > 0 && !kv_ids) return VSA_ERR_INVALID_ARG;
    if (n_list_entries > INT_MAX) return VSA_ERR_UNSUPPORTED;
  }
  FineArgs fa{q, kp, vp, oc, gate_c, gate_f, B, heads, head_dim, T, H, W,
              kv_offsets, kv_ids, topk, n_list_entries, dtype == VSA_BF16, out, lse_f, o_fine};
  fa.order = order;
  return hip_status(launch_fine_forward(fa, stream));
}

int vsa_fine_order(const int32_t* kv_offsets, const int32_t* kv_ids, int64_t n_list_entries,
                   int topk, int B, int heads, int n_cubes, int32_t* order, hipStream_t stream) {
  if (B < 1 || heads < 1 || n_cubes < 1 || !order) return VSA_ERR_INVALID_ARG;
  if (n_cubes > order_max_cubes() || (int64_t)B * heads > 65535) return VSA_ERR_UNSUPPORTED;
  if ((int64_t)B * heads * n_cubes > kMaxCubeUnits) return VSA_ERR_UNSUPPORTED;
  if (!kv_offsets) {
    if (topk < 1 || topk > n_cubes || !kv_ids) return VSA_ERR_INVALID_ARG;
    if ((int64_t)B * heads * n_cubes * topk > INT_MAX) return VSA_ERR_UNSUPPORTED;
    n_list_entries = (int64_t)B * heads * n_cubes * topk;
  } else {
    if (n_list_entries < 0 || n_list_entries > (int64_t)B * heads * n_cubes * n_cubes)
      return VSA_ERR_INVALID_ARG;
    if (n_list_entries > 0 && !kv_ids) return VSA_ERR_INVALID_ARG;
    if (n_list_entries > INT_MAX) return VSA_ERR_UNSUPPORTED;
  }
  return hip_status(launch_fine_order(kv_offsets, kv_ids, topk, n_list_entries, B * heads, n_cubes,
                                      order, stream));
}

int vsa_validate_lists(const int32_t* kv_offsets, const int32_t* kv_ids, int64_t n_list_entries,
                       int topk, int n_rows, int n_cubes, int32_t* result, hipStream_t stream) {
  if (n_rows < 0 || n_cubes < 1 || !result) return VSA_ERR_INVALID_ARG;
  if (n_cubes > validate_max_cubes()) return VSA_ERR_UNSUPPORTED;
  if (n_list_entries < 0 || n_list_entries > INT_MAX) return VSA_ERR_INVALID_ARG;
  if (kv_offsets) {
    if (n_list_entries > 0 && !kv_ids) return VSA_ERR_INVALID_ARG;
  } else {
    if (topk < 1 || !kv_ids || (int64_t)n_rows * topk != n_list_entries) return VSA_ERR_INVALID_ARG;
  }
  return hip_status(launch_validate_lists(kv_offsets, kv_ids, topk, n_list_entries, n_rows, n_cubes,
                                          result, stream));
}

size_t vsa_backward_workspace_bytes(int B, int heads, int head_dim, int T, int H, int W, int dtype,
                                    int64_t n_list_entries) {
  Shape s;
  if (check_shape(B, heads, head_dim, T, H, W, dtype, &s) != VSA_OK || n_list_entries < 0) return 0;
  return bwd_ws_layout(s, n_list_entries, nullptr, nullptr);
}

int vsa_backward(const void* q, const void* k, const void* v, const void* gate_c, const void* gate_f,
                 const void* dout, const int32_t* sel_idx, const void* saved,
                 int B, int heads, int head_dim, int T, int H, int W, int topk, int dtype,
                 void* dq, void* dk, void* dv, void* dgate_c, void* dgate_f,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (topk < 1 || topk > s.nc || !sel_idx) return VSA_ERR_INVALID_ARG;
  if ((int64_t)B * heads * s.nc * topk > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return backward_impl(q, k, v, gate_c, gate_f, dout, nullptr, sel_idx, topk,
                       (int64_t)B * heads * s.nc * topk, saved, s, dq, dk, dv, dgate_c, dgate_f,
                       workspace, workspace_bytes, stream);
}

int block_sparse_attn_varlen_backward(const void* q, const void* k, const void* v,
                                      const void* gate_c, const void* gate_f, const void* dout,
                                      const int32_t* kv_offsets, const int32_t* kv_ids,
                                      int64_t n_list_entries, const void* saved,
                                      int B, int heads, int head_dim, int T, int H, int W, int dtype,
                                      void* dq, void* dk, void* dv, void* dgate_c, void* dgate_f,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Shape s;
  int st = check_shape(B, heads, head_dim, T, H, W, dtype, &s);
  if (st != VSA_OK) return st;
  if (!kv_offsets) return VSA_ERR_INVALID_ARG;
  if (n_list_entries < 0 || n_list_entries > (int64_t)B * heads * s.nc * s.nc) return VSA_ERR_INVALID_ARG;
  if (n_list_entries > 0 && !kv_ids) return VSA_ERR_INVALID_ARG;
  if (n_list_entries > INT_MAX) return VSA_ERR_UNSUPPORTED;
  return backward_impl(q, k, v, gate_c, gate_f, dout, kv_offsets, kv_ids, 0, n_list_entries, saved, s,
                       dq, dk, dv, dgate_c, dgate_f, workspace, workspace_bytes, stream);
}

}  // extern "C"
