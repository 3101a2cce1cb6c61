// Host-only build of the C ABI's argument checks and workspace carving,
// compiled with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_abi_sanitize.py builds and runs it; no GPU is involved).
//
// The library's launch layer (vsa_launch.h) is replaced by stubs that, for
// every launch, read each input range and overwrite each output range the
// real kernels would touch, computed from the launch arguments.  Device
// buffers are stood in for by host allocations of exactly the sizes the
// size queries report, so an entry point that carves a workspace wrongly,
// or hands a kernel a pointer past its buffer, is caught by ASan; integer
// overflow in the size arithmetic is caught by UBSan.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "vsa.h"
#include "vsa_launch.h"

namespace {

int g_launches = 0;
int g_validate_faults = 0;  // what the stub validation kernel reports
volatile unsigned g_sink = 0;

void touch_read(const void* p, size_t bytes) {
  if (!p || !bytes) return;
  const unsigned char* c = static_cast<const unsigned char*>(p);
  unsigned s = 0;
  for (size_t i = 0; i < bytes; i += 61) s += c[i];
  s += c[bytes - 1];
  g_sink += s;
}

void touch_write(void* p, size_t bytes) {
  if (p && bytes) std::memset(p, 0x5A, bytes);
}

int failures = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

}  // namespace

// ------------------------------------------------------------ launch stubs
namespace vsa {

int coarse_max_cubes(int) { return 3584; }
int order_max_cubes() { return 4096; }
int validate_max_cubes() { return 4096; }

hipError_t launch_permute_pool(const PermutePoolArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t N = (int64_t)a.T * a.H * a.W, nc = N / 64, BH = (int64_t)a.B * a.heads;
  const size_t elt = a.bf16 ? 2 : 4;
  for (int t = 0; t < 3; ++t) {
    touch_read(a.p.src[t], (size_t)(a.B * N * a.heads * a.D) * elt);
    if (a.p.nat[t] && !a.max_pool) touch_write(a.p.nat[t], (size_t)(BH * N * a.D) * elt);
    const int64_t keys = (a.packed_kv && t > 0) ? packed_keys((int)nc) : nc;
    touch_write(a.p.pooled[t], (size_t)(BH * keys * a.D) * 4);
  }
  return hipSuccess;
}

hipError_t launch_coarse_topk(const CoarseArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t BH = (int64_t)a.B * a.heads, rows = BH * a.nc;
  const int64_t keys = a.packed ? packed_keys(a.nc) : a.nc;
  touch_read(a.qc, (size_t)(rows * a.D) * 4);
  touch_read(a.kc, (size_t)(BH * keys * a.D) * 4);
  touch_read(a.vc, (size_t)(BH * keys * a.D) * 4);
  touch_write(a.oc, (size_t)(rows * a.D) * 4);
  touch_write(a.lse, (size_t)rows * 4);
  if (a.counts) {
    touch_write(a.counts, (size_t)rows * 4);
    touch_write(a.sel, (size_t)(rows * a.k_max) * 4);
  } else if (a.topk > 0) {
    touch_write(a.sel, (size_t)(rows * a.topk) * 4);
  }
  return hipSuccess;
}

hipError_t launch_pack_lists(const int32_t* counts, const int32_t* padded, int n_rows, int k_max,
                             int32_t* offsets, int32_t* ids, hipStream_t) {
  ++g_launches;
  touch_read(counts, (size_t)n_rows * 4);
  touch_read(padded, (size_t)n_rows * k_max * 4);
  touch_write(offsets, (size_t)(n_rows + 1) * 4);
  touch_write(ids, (size_t)n_rows * k_max * 4);
  return hipSuccess;
}

hipError_t launch_fine_forward(const FineArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t N = (int64_t)a.T * a.H * a.W, nc = N / 64, BH = (int64_t)a.B * a.heads;
  const size_t elt = a.bf16 ? 2 : 4;
  touch_read(a.q, (size_t)(a.B * N * a.heads * a.D) * elt);
  touch_read(a.kp, (size_t)(BH * N * a.D) * elt);
  touch_read(a.vp, (size_t)(BH * N * a.D) * elt);
  touch_read(a.oc, (size_t)(BH * nc * a.D) * 4);
  touch_read(a.gc, (size_t)(a.B * N * a.heads) * elt);
  touch_read(a.gf, (size_t)(a.B * N * a.heads) * elt);
  if (a.offs) touch_read(a.offs, (size_t)(BH * nc + 1) * 4);
  touch_read(a.ids, (size_t)a.n_ids * 4);
  if (a.order) touch_read(a.order, (size_t)(BH * nc) * 4);
  touch_write(a.out, (size_t)(a.B * N * a.heads * a.D) * elt);
  touch_write(a.lse_f, (size_t)(BH * N) * 4);
  touch_write(a.o_fine, (size_t)(BH * N * a.D) * 4);
  return hipSuccess;
}

hipError_t launch_fine_order(const int32_t* offs, const int32_t* ids, int, int64_t n_ids, int n_bh,
                             int nc, int32_t* order, hipStream_t) {
  ++g_launches;
  if (offs) touch_read(offs, (size_t)((int64_t)n_bh * nc + 1) * 4);
  touch_read(ids, (size_t)n_ids * 4);
  touch_write(order, (size_t)((int64_t)n_bh * nc) * 4);
  return hipSuccess;
}

hipError_t launch_validate_lists(const int32_t* offs, const int32_t* ids, int, int64_t n_ids,
                                 int n_rows, int, int32_t* result, hipStream_t) {
  ++g_launches;
  if (offs) touch_read(offs, (size_t)(n_rows + 1) * 4);
  touch_read(ids, (size_t)n_ids * 4);
  result[0] = 0;
  result[1] = g_validate_faults;
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t) {
  ++g_launches;
  const int64_t N = (int64_t)a.T * a.H * a.W, nc = N / 64, BH = (int64_t)a.B * a.heads;
  const size_t elt = a.bf16 ? 2 : 4;
  const size_t raster = (size_t)(a.B * N * a.heads * a.D) * elt, tiles = (size_t)(BH * N * a.D) * elt;
  const size_t pooled = (size_t)(BH * nc * a.D) * 4;
  touch_read(a.dout, raster);
  touch_read(a.gc, (size_t)(a.B * N * a.heads) * elt);
  touch_read(a.gf, (size_t)(a.B * N * a.heads) * elt);
  touch_read(a.qp, tiles); touch_read(a.kp, tiles); touch_read(a.vp, tiles);
  touch_read(a.qc, pooled); touch_read(a.kc, pooled); touch_read(a.vc, pooled);
  touch_read(a.oc, pooled);
  touch_read(a.lse_c, (size_t)(BH * nc) * 4);
  touch_read(a.lse_f, (size_t)(BH * N) * 4);
  touch_read(a.of, (size_t)(BH * N * a.D) * 4);
  if (a.offs) touch_read(a.offs, (size_t)(BH * nc + 1) * 4);
  touch_read(a.ids, (size_t)a.n_ids * 4);
  touch_write(a.delta, (size_t)(BH * N) * 4);
  touch_write(a.dofp, tiles);
  touch_write(a.doc, pooled);
  touch_write(a.deltac, (size_t)(BH * nc) * 4);
  touch_write(a.S, (size_t)(BH * nc * nc) * 4);
  touch_write(a.dP, (size_t)(BH * nc * nc) * 4);
  touch_write(a.dqc, pooled); touch_write(a.dkc, pooled); touch_write(a.dvc, pooled);
  touch_write(a.tr_offs, (size_t)(BH * nc + 1) * 4);
  touch_write(a.tr_order, (size_t)(BH * nc) * 4);
  touch_write(a.tr_ids, (size_t)a.n_ids * 4);
  touch_write(a.tr_tmp, (size_t)a.n_ids * 4);
  touch_write(a.dq, raster); touch_write(a.dk, raster); touch_write(a.dv, raster);
  touch_write(a.dgc, (size_t)(a.B * N * a.heads) * 4);
  touch_write(a.dgf, (size_t)(a.B * N * a.heads) * 4);
  return hipSuccess;
}

}  // namespace vsa

// Device-to-host copy and stream wait of the VSA_VALIDATE path: the
// "device" memory is host memory here.
extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
// The fixed scratch of the allocation-free entry point: in this host build
// the "device address" of the array is the host array itself, so the stub
// launches' writes into it are bounds-checked by ASan against its size.
extern "C" hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipSetDevice(int dev) { return dev == 0 ? hipSuccess : hipErrorInvalidDevice; }
extern "C" hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* dev) {
  *dev = 0;
  return hipSuccess;
}
extern "C" hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  return hipSuccess;
}

// ------------------------------------------------------------------ driver
namespace {

struct Buf {
  std::vector<unsigned char*> owned;
  ~Buf() { for (auto* p : owned) std::free(p); }
  void* get(size_t bytes) {
    auto* p = static_cast<unsigned char*>(std::malloc(bytes ? bytes : 1));
    std::memset(p, 0, bytes ? bytes : 1);
    owned.push_back(p);
    return p;
  }
};

// CSR lists over n_rows rows of a head with nc cubes: row r lists
// (r % 3) cubes, distinct and ascending.
void make_csr(Buf& m, int64_t n_rows, int nc, int32_t** offs, int32_t** ids, int64_t* n) {
  *offs = static_cast<int32_t*>(m.get((size_t)(n_rows + 1) * 4));
  std::vector<int32_t> all;
  (*offs)[0] = 0;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int len = (int)(r % 3) < nc ? (int)(r % 3) : nc;
    for (int i = 0; i < len; ++i) all.push_back((int32_t)((r + 2 * i) % nc));
    (*offs)[r + 1] = (int32_t)all.size();
  }
  *n = (int64_t)all.size();
  *ids = static_cast<int32_t*>(m.get(all.size() * 4));
  if (!all.empty()) std::memcpy(*ids, all.data(), all.size() * 4);
}

void run_shape(int B, int heads, int D, int T, int H, int W, int dtype, int topk) {
  Buf m;
  const int64_t N = (int64_t)T * H * W, nc = N / 64, rows = (int64_t)B * heads * nc;
  const size_t elt = dtype == VSA_BF16 ? 2 : 4;
  const size_t raster = (size_t)(B * N * heads * D) * elt, gates = (size_t)(B * N * heads) * elt;
  void *q = m.get(raster), *k = m.get(raster), *v = m.get(raster), *dout = m.get(raster);
  void *gc = m.get(gates), *gf = m.get(gates), *out = m.get(raster);
  const size_t svb = vsa_saved_bytes(B, heads, D, T, H, W, dtype);
  const size_t fwb = vsa_forward_workspace_bytes(B, heads, D, T, H, W, dtype);
  EXPECT(svb > 0 && fwb > 0);
  void *saved = m.get(svb), *ws = m.get(fwb);
  auto* sel = static_cast<int32_t*>(m.get((size_t)(rows * topk) * 4));
  EXPECT(vsa_forward(q, k, v, gc, gf, B, heads, D, T, H, W, topk, dtype, out, sel, saved, ws, fwb,
                     nullptr) == VSA_OK);
  EXPECT(vsa_forward(q, k, v, gc, gf, B, heads, D, T, H, W, topk, dtype, out, sel, nullptr, ws, fwb,
                     nullptr) == VSA_OK);
  EXPECT(vsa_forward(q, k, v, gc, gf, B, heads, D, T, H, W, topk, dtype, out, sel, saved, ws, fwb - 1,
                     nullptr) == VSA_ERR_WORKSPACE);
  int32_t *offs, *ids;
  int64_t n_ids;
  make_csr(m, rows, (int)nc, &offs, &ids, &n_ids);
  EXPECT(block_sparse_attn_varlen(q, k, v, gc, gf, B, heads, D, T, H, W, offs, ids, n_ids, dtype, out,
                                  saved, ws, fwb, nullptr) == VSA_OK);
  const int k_max = (int)(nc < 5 ? nc : 5);
  const size_t mwb = vsa_forward_mass_workspace_bytes(B, heads, D, T, H, W, dtype, k_max);
  void* mws = m.get(mwb);
  auto* moffs = static_cast<int32_t*>(m.get((size_t)(rows + 1) * 4));
  auto* mids = static_cast<int32_t*>(m.get((size_t)(rows * k_max) * 4));
  EXPECT(vsa_forward_mass(q, k, v, gc, gf, B, heads, D, T, H, W, 0.5f, 1, k_max, dtype, out, moffs,
                          mids, saved, mws, mwb, nullptr) == VSA_OK);
  EXPECT(vsa_forward_mass(q, k, v, gc, gf, B, heads, D, T, H, W, 0.5f, 1, k_max, dtype, out, moffs,
                          mids, saved, mws, mwb - 1, nullptr) == VSA_ERR_WORKSPACE);
  // backward, both list forms
  const size_t bwb = vsa_backward_workspace_bytes(B, heads, D, T, H, W, dtype, rows * topk);
  void* bws = m.get(bwb);
  void *dq = m.get(raster), *dk = m.get(raster), *dv = m.get(raster);
  void *dgc = m.get((size_t)(B * N * heads) * 4), *dgf = m.get((size_t)(B * N * heads) * 4);
  EXPECT(vsa_backward(q, k, v, gc, gf, dout, sel, saved, B, heads, D, T, H, W, topk, dtype, dq, dk, dv,
                      dgc, dgf, bws, bwb, nullptr) == VSA_OK);
  EXPECT(vsa_backward(q, k, v, gc, gf, dout, sel, saved, B, heads, D, T, H, W, topk, dtype, dq, dk, dv,
                      dgc, dgf, bws, bwb - 1, nullptr) == VSA_ERR_WORKSPACE);
  const size_t vbwb = vsa_backward_workspace_bytes(B, heads, D, T, H, W, dtype, n_ids);
  void* vbws = m.get(vbwb);
  EXPECT(block_sparse_attn_varlen_backward(q, k, v, gc, gf, dout, offs, ids, n_ids, saved, B, heads, D,
                                           T, H, W, dtype, dq, dk, dv, dgc, dgf, vbws, vbwb,
                                           nullptr) == VSA_OK);
  // stage calls on their own buffers
  const size_t tiles = (size_t)(rows * 64 * D) * elt, pooled = (size_t)(rows * D) * 4;
  void *qp = m.get(tiles), *kp = m.get(tiles), *vp = m.get(tiles);
  auto *qc = static_cast<float*>(m.get(pooled)), *kc = static_cast<float*>(m.get(pooled)),
       *vc = static_cast<float*>(m.get(pooled)), *oc = static_cast<float*>(m.get(pooled));
  auto* lse = static_cast<float*>(m.get((size_t)rows * 4));
  EXPECT(vsa_cube_permute_pool(q, k, v, B, heads, D, T, H, W, dtype, qp, kp, vp, qc, kc, vc, nullptr) ==
         VSA_OK);
  EXPECT(vsa_cube_max_pool(q, k, v, B, heads, D, T, H, W, dtype, qc, kc, vc, nullptr) == VSA_OK);
  EXPECT(vsa_coarse_topk(qc, kc, vc, B, heads, D, (int)nc, topk, dtype, oc, lse, sel, nullptr) == VSA_OK);
  auto* counts = static_cast<int32_t*>(m.get((size_t)rows * 4));
  auto* padded = static_cast<int32_t*>(m.get((size_t)(rows * k_max) * 4));
  EXPECT(vsa_coarse_select_mass(qc, kc, vc, B, heads, D, (int)nc, 0.3f, 1, k_max, dtype, oc, lse, counts,
                                padded, nullptr) == VSA_OK);
  EXPECT(vsa_pack_lists(counts, padded, (int)rows, k_max, moffs, mids, nullptr) == VSA_OK);
  auto* order = static_cast<int32_t*>(m.get((size_t)rows * 4));
  auto* lse_f = static_cast<float*>(m.get((size_t)(B * heads * N) * 4));
  auto* o_fine = static_cast<float*>(m.get((size_t)(B * heads * N * D) * 4));
  EXPECT(vsa_fine_order(nullptr, sel, 0, topk, B, heads, (int)nc, order, nullptr) == VSA_OK);
  EXPECT(vsa_fine_order(offs, ids, n_ids, 0, B, heads, (int)nc, order, nullptr) == VSA_OK);
  EXPECT(vsa_fine_forward(q, kp, vp, oc, gc, gf, B, heads, D, T, H, W, nullptr, sel, 0, topk, dtype, out,
                          lse_f, o_fine, order, nullptr) == VSA_OK);
  EXPECT(vsa_fine_forward(q, kp, vp, oc, gc, gf, B, heads, D, T, H, W, offs, ids, n_ids, 0, dtype, out,
                          nullptr, nullptr, nullptr, nullptr) == VSA_OK);
  auto* result = static_cast<int32_t*>(m.get(8));
  EXPECT(vsa_validate_lists(offs, ids, n_ids, 0, (int)rows, (int)nc, result, nullptr) == VSA_OK);
  EXPECT(vsa_validate_lists(nullptr, sel, rows * topk, topk, (int)rows, (int)nc, result, nullptr) == VSA_OK);

  // VSA_VALIDATE: checked lists pass, a reported fault refuses the call
  setenv("VSA_VALIDATE", "1", 1);
  g_validate_faults = 0;
  EXPECT(block_sparse_attn_varlen(q, k, v, gc, gf, B, heads, D, T, H, W, offs, ids, n_ids, dtype, out,
                                  saved, ws, fwb, nullptr) == VSA_OK);
  g_validate_faults = 1;
  const int before = g_launches;
  EXPECT(block_sparse_attn_varlen(q, k, v, gc, gf, B, heads, D, T, H, W, offs, ids, n_ids, dtype, out,
                                  saved, ws, fwb, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(g_launches == before + 1);  // only the check itself was queued
  EXPECT(vsa_backward(q, k, v, gc, gf, dout, sel, saved, B, heads, D, T, H, W, topk, dtype, dq, dk, dv,
                      dgc, dgf, bws, bwb, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(block_sparse_attn_varlen_backward(q, k, v, gc, gf, dout, offs, ids, n_ids, saved, B, heads, D,
                                           T, H, W, dtype, dq, dk, dv, dgc, dgf, vbws, vbwb,
                                           nullptr) == VSA_ERR_INVALID_ARG);
  g_validate_faults = 0;
  unsetenv("VSA_VALIDATE");

  // the allocation-free forward: same launches into the fixed scratch,
  // refused (nothing queued) where the workspace would not fit in it
  const int launches = g_launches;
  const int st = vsa_forward_noalloc(q, k, v, gc, gf, B, heads, D, T, H, W, topk, dtype, out, sel, saved,
                                     nullptr);
  if (fwb <= (size_t(128) << 20)) {
    EXPECT(st == VSA_OK);
    EXPECT(g_launches > launches);
  } else {
    EXPECT(st == VSA_ERR_WORKSPACE);
    EXPECT(g_launches == launches);
  }
}

void argument_checks() {
  void* F = reinterpret_cast<void*>(0x1000);  // never dereferenced by failing calls
  auto* I = static_cast<int32_t*>(F);
  const size_t big = (size_t)1 << 40;
  // grid not made of cubes, empty sides, bad topk, head_dim, dtype, nulls
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 6, 8, 8, 2, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 8, 0, 8, 2, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 0, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 9, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 96, 8, 8, 8, 2, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 2, 7, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 2, VSA_BF16, nullptr, I, nullptr, F, big, nullptr) ==
         VSA_ERR_INVALID_ARG);
  // sizes that would overflow 32-bit indexing or the grid limits
  EXPECT(vsa_forward(F, F, F, F, F, 256, 256, 64, 8, 8, 8, 2, VSA_BF16, F, I, nullptr, F, big, nullptr) ==
         VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_forward(F, F, F, F, F, 1, 1, 128, 4, 4, 4 * 3585, 2, VSA_BF16, F, I, nullptr, F, big,
                     nullptr) == VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_forward(F, F, F, F, F, 65535, 1, 128, 4, 4, 4 * 3584, 2, VSA_BF16, F, I, nullptr, F, big,
                     nullptr) == VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_forward_workspace_bytes(1 << 20, 1 << 10, 128, 1 << 10, 1 << 10, 1 << 10, VSA_BF16) == 0);
  EXPECT(vsa_backward_workspace_bytes(1, 1, 64, 8, 8, 8, VSA_BF16, -1) == 0);
  // varlen and backward
  EXPECT(block_sparse_attn_varlen(F, F, F, F, F, 1, 2, 64, 8, 8, 8, nullptr, I, 4, VSA_BF16, F, nullptr,
                                  F, big, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(block_sparse_attn_varlen(F, F, F, F, F, 1, 2, 64, 8, 8, 8, I, I, -1, VSA_BF16, F, nullptr, F,
                                  big, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(block_sparse_attn_varlen(F, F, F, F, F, 1, 2, 64, 8, 8, 8, I, I, 129, VSA_BF16, F, nullptr, F,
                                  big, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_backward(F, F, F, F, F, F, I, nullptr, 1, 2, 64, 8, 8, 8, 2, VSA_BF16, F, F, F, F, F, F, big,
                      nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_backward(F, F, F, F, F, F, I, F, 1, 2, 64, 8, 8, 8, 2, 7, F, F, F, F, F, F, big, nullptr) ==
         VSA_ERR_UNSUPPORTED);
  // mass rule, stage calls, validation
  EXPECT(vsa_forward_mass(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 0.f, 1, 4, VSA_BF16, F, I, I, nullptr, F,
                          big, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward_mass(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 0.5f, 1, 9, VSA_BF16, F, I, I, nullptr, F,
                          big, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_pack_lists(I, I, 1 << 20, 1 << 12, I, I, nullptr) == VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_coarse_topk(static_cast<float*>(F), static_cast<float*>(F), static_cast<float*>(F), 1, 1, 64,
                         100000, 2, VSA_BF16, static_cast<float*>(F), static_cast<float*>(F), I,
                         nullptr) == VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_fine_order(I, I, 65, 0, 1, 1, 8, I, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_validate_lists(I, I, 10, 0, 4, 5000, I, nullptr) == VSA_ERR_UNSUPPORTED);
  EXPECT(vsa_validate_lists(nullptr, I, 10, 3, 4, 8, I, nullptr) == VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward_noalloc(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 9, VSA_BF16, F, I, nullptr, nullptr) ==
         VSA_ERR_INVALID_ARG);
  EXPECT(vsa_forward_noalloc(F, F, F, F, F, 1, 2, 64, 8, 8, 8, 2, VSA_BF16, F, nullptr, nullptr, nullptr) ==
         VSA_ERR_INVALID_ARG);
  // the 16384-token training shape with B = 2 needs about 215 MB of workspace
  EXPECT(vsa_forward_noalloc(F, F, F, F, F, 2, 12, 128, 16, 32, 32, 32, VSA_BF16, F, I, nullptr, nullptr) ==
         VSA_ERR_WORKSPACE);
  EXPECT(g_launches == 0);  // no failing call queued anything
}

}  // namespace

int main() {
  argument_checks();
  const int shapes[][8] = {
      // B, heads, D, T, H, W, dtype, topk
      {1, 2, 64, 8, 8, 8, VSA_F32, 2},   {1, 2, 64, 8, 8, 8, VSA_BF16, 3},
      {2, 3, 128, 4, 8, 12, VSA_BF16, 6}, {2, 1, 128, 4, 4, 4, VSA_F32, 1},
      {1, 2, 128, 12, 8, 16, VSA_F32, 24}, {1, 1, 64, 4, 8, 20, VSA_BF16, 10},
      {1, 12, 128, 16, 32, 32, VSA_BF16, 32},  // the largest workload the fixed scratch holds
  };
  for (const auto& s : shapes) run_shape(s[0], s[1], s[2], s[3], s[4], s[5], s[6], s[7]);
  if (failures) {
    std::fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  std::printf("host ABI checks passed (%d stub launches)\n", g_launches);
  return 0;
}
