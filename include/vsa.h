/*
 * vsa.h - C ABI of the MI355X (gfx950) library for hierarchical video sparse
 * attention: VSA, plus the variable-length key lists of VSA2.
 *
 * Sources, cited by page title and section:
 *   [VSA-abs]  "VSA: Faster Video Diffusion with Trainable Sparse Attention",
 *              Abstract (arXiv).
 *   [VSA-sum]  "Faster Video Diffusion with Trainable Sparse Attention"
 *              (AI-extracted summary page): Approach, Key results,
 *              Limitations.
 *   [VSA2-abs] "Improving Video Sparse Attention with Fine-grained Router and
 *              Sparse Rebasing", Abstract (arXiv).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer unless marked "host".
 *    Buffers are dense and row-major.  The caller owns all memory; the
 *    library allocates nothing and keeps no state between calls.
 *  - Work is queued on `stream` (0 = the null stream).  No call waits for
 *    the GPU; results are ready when the stream has drained.
 *  - Arguments are checked before anything is queued.  On any error the
 *    call returns a non-zero vsa_status and queues nothing.  VSA_ERR_HIP
 *    reports a failed kernel launch (hipGetLastError after queueing).
 *  - dtype: VSA_F32 or VSA_BF16 for q, k, v, gates, out and gradients.
 *    Arithmetic: bf16 operands feed MFMA with fp32 accumulation; softmax,
 *    pooling and the coarse stage run in fp32; each output is rounded once
 *    (round to nearest even).  VSA_F32 uses fp32 arithmetic throughout.
 *  - Shapes: B batch, `heads` heads, head_dim D in {64, 128}; a latent grid
 *    of T x H x W tokens, N = T*H*W, each of T, H, W a positive multiple of
 *    4 ([VSA-sum, Limitations]).  Nc = N / 64 cubes, at most 3584 per
 *    (batch, head) (VSA_ERR_UNSUPPORTED beyond: the coarse stage keeps
 *    blocks of logit rows in LDS and the row it ranks in registers);
 *    B*heads at most 65535, and B*heads*Nc at most 2^24 - 8 (one
 *    workgroup of 256 threads per (batch, head, cube) in 1-D grids; about
 *    275 GB per bf16 tensor at D = 128, so beyond one GPU's memory anyway).
 *  - Token order is raster, token (t, y, x) at (t*H + y)*W + x.
 *    q, k, v, out, dout, dq, dk, dv: [B, N, heads, D].
 *    gate_c, gate_f: [B, N, heads] (one scalar per token and head,
 *    broadcast over D).  dgate_c, dgate_f: [B, N, heads], always fp32: they
 *    are D-long dot products whose magnitude (~10 at unit-scale inputs)
 *    puts bf16 rounding above the accuracy the method is checked to.
 *  - Cubes ([VSA-sum, Approach]): token (t, y, x) lies in cube
 *    ((t/4)*(H/4) + y/4)*(W/4) + x/4, at slot ((t%4)*4 + y%4)*4 + x%4.
 *  - Softmax scale is 1/sqrt(D) in both stages.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARG = 1, /* bad shape, null pointer, topk out of range  */
  VSA_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, dtype, size  */
  VSA_ERR_WORKSPACE = 3,   /* workspace_bytes below the required size     */
  VSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed  */
} vsa_status;

typedef enum { VSA_F32 = 0, VSA_BF16 = 1 } vsa_dtype;

/* Human-readable text for a status code (static storage, never NULL). */
const char* vsa_status_string(int status);

/* ------------------------------------------------------------------ sizes
 * Bytes of device scratch each call needs.  0 means the shape is invalid.
 * n_list_entries: total number of (query cube, key cube) pairs, i.e.
 * B*heads*Nc*topk for the fixed top-K path, kv_offsets[B*heads*Nc] for
 * the variable-length path.  Host functions, no GPU work.
 */
size_t vsa_forward_workspace_bytes(int B, int heads, int head_dim,
                                   int T, int H, int W, int dtype);
size_t vsa_backward_workspace_bytes(int B, int heads, int head_dim,
                                    int T, int H, int W, int dtype,
                                    int64_t n_list_entries);
/* Size of the forward->backward state ("saved") for element type dtype:
 * fp32 coarse output [B,heads,Nc,D], coarse log-sum-exp [B,heads,Nc], fine
 * log-sum-exp [B,heads,N] and fine output [B,heads,N,D] (cube-major token
 * order), the forward's K and V cube tiles [B,heads,Nc,64,D] (dtype) and
 * the fp32 cube means of Q, K and V [B,heads,Nc,D].  The backward reads K
 * and V only from here.  Opaque to the caller; 0 for an invalid shape. */
size_t vsa_saved_bytes(int B, int heads, int head_dim, int T, int H, int W, int dtype);

/* ---------------------------------------------------------------- forward
 * vsa_forward: the whole operator ([VSA-sum, Approach]; [VSA-abs]).
 *  1. permute tokens into cube-major order and mean-pool Q, K, V per cube;
 *  2. dense cube-to-cube attention on the pooled tensors -> coarse output
 *     Oc per cube (broadcast to the cube's 64 tokens);
 *  3. per query cube, the topk key cubes with the largest coarse logits,
 *     ties to the lower cube index, written ascending to
 *     sel_idx [B, heads, Nc, topk] (int32);
 *  4. fine attention of every query token over the 64*topk tokens of its
 *     cube's selection (online softmax);
 *  5. out = gate_c * Oc + gate_f * O_fine.
 * topk in [1, Nc].  `saved` (vsa_saved_bytes) may be NULL for inference;
 * pass it to vsa_backward.  workspace: vsa_forward_workspace_bytes.
 */
int vsa_forward(const void* q, const void* k, const void* v,
                const void* gate_c, const void* gate_f,
                int B, int heads, int head_dim, int T, int H, int W,
                int topk, int dtype,
                void* out, int32_t* sel_idx, void* saved,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* vsa_forward_noalloc: vsa_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * vsa_forward without the workspace: the workspace lives in a fixed
 * 128 MiB device array inside the library (one per GPU, held until the
 * process ends; enough for B*heads = 12 at 16384 tokens, head_dim 128,
 * bf16).  A shape whose forward workspace (vsa_forward_workspace_bytes)
 * exceeds 128 MiB returns VSA_ERR_WORKSPACE and queues nothing.  The call
 * allocates nothing; its first call on a device looks up that device's
 * copy of the array (the device `stream` runs on, or the current device
 * for the null stream).  All calls on one GPU share the array, so calls that
 * overlap in time on one GPU (on different streams, or from different
 * threads) race and must be serialized by the caller.
 */
int vsa_forward_noalloc(const void* q, const void* k, const void* v,
                        const void* gate_c, const void* gate_f,
                        int B, int heads, int head_dim, int T, int H, int W,
                        int topk, int dtype,
                        void* out, int32_t* sel_idx, void* saved, hipStream_t stream);

/* block_sparse_attn_varlen: as vsa_forward, but step 3 is replaced by a
 * caller-given list of key cubes per query cube ([VSA2-abs]: each query
 * attends a variable number of key-value pairs; the router that would make
 * the lists is not defined on the pages and is not implemented).
 * kv_offsets [B*heads*Nc + 1] (int32, non-decreasing, kv_offsets[0] = 0)
 * indexes kv_ids, lists ordered by (b, h, query cube).  n_list_entries
 * (host) equals kv_offsets[B*heads*Nc].  Ids must lie in [0, Nc) and be
 * distinct within a list; any order.  An empty list gives O_fine = 0.
 * Lists are not checked unless asked for (vsa_validate_lists, or
 * VSA_VALIDATE=1 in the environment, below).  Malformed lists give
 * unspecified outputs but never a memory access outside the buffers:
 * every kernel clamps list ranges to [0, n_list_entries) and skips any id
 * outside [0, Nc); an id listed twice counts twice, consistently in the
 * forward and the backward.
 */
int block_sparse_attn_varlen(const void* q, const void* k, const void* v,
                             const void* gate_c, const void* gate_f,
                             int B, int heads, int head_dim, int T, int H, int W,
                             const int32_t* kv_offsets, const int32_t* kv_ids,
                             int64_t n_list_entries, int dtype,
                             void* out, void* saved,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------- variable-length selection
 * A stand-in rule for variable-length key lists.  [VSA2-abs] lets each
 * query attend a variable number of key-value pairs but does not define
 * how VSA2 picks them (its router is not given); this rule is an
 * assumption of this library, not the method:
 *   per query cube, rank the key cubes as the top-K step does (coarse logit
 *   descending, lower cube index first on ties) and take the shortest
 *   prefix of that ranking whose coarse softmax probability mass reaches
 *   `mass` ([VSA-sum, Approach]: the coarse scores mark the critical
 *   cubes); clamp its length to [k_min, k_max]; report it ascending.
 * The mass is summed in fp32 on the GPU: where a prefix's mass lies within
 * rounding of `mass`, the length may differ by one from an exact-arithmetic
 * evaluation.
 * mass in (0, 1]; 1 <= k_min <= k_max <= Nc; B*heads*Nc*k_max <= INT_MAX
 * (else VSA_ERR_UNSUPPORTED); anything else VSA_ERR_INVALID_ARG.
 *
 * vsa_forward_mass: vsa_forward with step 3 replaced by this rule.  The
 * lists it used are written as CSR, ordered by (b, h, query cube):
 * kv_offsets [B*heads*Nc + 1] and kv_ids (capacity B*heads*Nc*k_max;
 * kv_offsets[B*heads*Nc] entries are written), ready for
 * block_sparse_attn_varlen_backward with the same `saved`.  workspace:
 * vsa_forward_mass_workspace_bytes (0 for an invalid shape or k_max).
 */
size_t vsa_forward_mass_workspace_bytes(int B, int heads, int head_dim,
                                        int T, int H, int W, int dtype, int k_max);
int vsa_forward_mass(const void* q, const void* k, const void* v,
                     const void* gate_c, const void* gate_f,
                     int B, int heads, int head_dim, int T, int H, int W,
                     float mass, int k_min, int k_max, int dtype,
                     void* out, int32_t* kv_offsets, int32_t* kv_ids, void* saved,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------------- backward
 * Gradients of sum(dout * out) for a forward run with `saved` non-NULL
 * ([VSA-abs]: one operator trained end-to-end).  The selection is held
 * fixed (no gradient through the discrete choice); the coarse stage carries
 * gradient to the pooled tensors, which spread it evenly over each cube's
 * 64 tokens.  sel_idx / kv lists must be the ones the forward used, and
 * q and `saved` must come from that same forward: K and V enter only
 * through the tiles and means the forward left in `saved` (k and v must
 * still be non-NULL, and are not read).
 * Outputs dq, dk, dv [B,N,heads,D] (dtype) and dgate_c, dgate_f [B,N,heads]
 * (fp32) are overwritten.  VSA_BF16 runs the products on the bf16 matrix
 * cores with fp32 accumulation; VSA_F32 uses fp32 arithmetic throughout
 * (plain vector code, for accuracy rather than speed).  workspace:
 * vsa_backward_workspace_bytes with n_list_entries = B*heads*Nc*topk
 * (resp. the varlen total); for bf16 it includes one 8 KB dS tile per list
 * entry (the dK/dV pass stores dS for the dQ pass), e.g. 1.6 GB at B = 2,
 * 12 heads, 16384 tokens, top-K 32.  With VSA_VALIDATE=1 the key lists
 * (sel_idx included) are checked first as in vsa_validate_lists.
 */
int vsa_backward(const void* q, const void* k, const void* v,
                 const void* gate_c, const void* gate_f, const void* dout,
                 const int32_t* sel_idx, const void* saved,
                 int B, int heads, int head_dim, int T, int H, int W,
                 int topk, int dtype,
                 void* dq, void* dk, void* dv, void* dgate_c, void* dgate_f,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

int block_sparse_attn_varlen_backward(
    const void* q, const void* k, const void* v,
    const void* gate_c, const void* gate_f, const void* dout,
    const int32_t* kv_offsets, const int32_t* kv_ids, int64_t n_list_entries,
    const void* saved,
    int B, int heads, int head_dim, int T, int H, int W, int dtype,
    void* dq, void* dk, void* dv, void* dgate_c, void* dgate_f,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------ stage calls
 * The forward's steps one at a time, for per-stage checks and timing.
 * Internal layouts (written by vsa_cube_permute_pool):
 *   qp, kp, vp: [B, heads, Nc, 64, D], token slot-major inside each cube
 *           (qp is optional: pass NULL to skip it; the forward does, since
 *           the fine stage reads Q in place);
 *   qc, kc, vc: fp32 [B, heads, Nc, D] cube means.
 * Element type of qp/kp/vp is `dtype`.
 */
int vsa_cube_permute_pool(const void* q, const void* k, const void* v,
                          int B, int heads, int head_dim, int T, int H, int W,
                          int dtype, void* qp, void* kp, void* vp,
                          float* qc, float* kc, float* vc, hipStream_t stream);

/* Pooling ablation: the per-channel maximum of each cube's 64 tokens
 * instead of the mean, for Q, K and V, as fp32 [B, heads, Nc, D] (exact).
 * The pages found mean pooling better than max pooling ([VSA-sum,
 * Surprising findings]); the operator entry points always mean-pool.  This
 * call feeds vsa_coarse_topk to compare the two selections. */
int vsa_cube_max_pool(const void* q, const void* k, const void* v,
                      int B, int heads, int head_dim, int T, int H, int W, int dtype,
                      float* qc, float* kc, float* vc, hipStream_t stream);

/* Coarse stage: Oc [B,heads,Nc,D] fp32, lse_c [B,heads,Nc] fp32 and, when
 * topk > 0, sel_idx [B,heads,Nc,topk]; topk == 0 skips the selection.
 * dtype is the element type of the attention inputs and sets the precision
 * of the two products (logits, P * Vc), which accumulate in fp32 either way:
 * VSA_F32 multiplies in fp32; VSA_BF16 splits every fp32 operand into bf16
 * hi + lo and takes hi*hi + hi*lo + lo*hi on the bf16 matrix cores (about
 * 16 significant bits; the forward entry points use the same choice).  An
 * unknown dtype is VSA_ERR_INVALID_ARG. */
int vsa_coarse_topk(const float* qc, const float* kc, const float* vc,
                    int B, int heads, int head_dim, int n_cubes, int topk, int dtype,
                    float* oc, float* lse_c, int32_t* sel_idx,
                    hipStream_t stream);

/* Coarse stage with the variable-length rule above instead of top-K: oc
 * and lse_c as vsa_coarse_topk (dtype sets the product precision the same
 * way); counts [B,heads,Nc] int32 list lengths; ids [B,heads,Nc,k_max]
 * int32, list r ascending in ids[r*k_max .. r*k_max + counts[r]) (the rest
 * of each row is left as it was). */
int vsa_coarse_select_mass(const float* qc, const float* kc, const float* vc,
                           int B, int heads, int head_dim, int n_cubes,
                           float mass, int k_min, int k_max, int dtype,
                           float* oc, float* lse_c, int32_t* counts, int32_t* ids,
                           hipStream_t stream);

/* Padded lists (counts [n_rows], ids_padded [n_rows, k_max] as written by
 * vsa_coarse_select_mass) -> CSR: kv_offsets [n_rows + 1] with
 * kv_offsets[r] = counts[0] + ... + counts[r-1], and kv_ids holding the
 * lists back to back in row order.  counts[r] must lie in [0, k_max]. */
int vsa_pack_lists(const int32_t* counts, const int32_t* ids_padded, int n_rows, int k_max,
                   int32_t* kv_offsets, int32_t* kv_ids, hipStream_t stream);

/* Fine stage + gated combine.  q: the raster input [B,N,heads,D] (read in
 * place); kp, vp: K and V tiles from vsa_cube_permute_pool; oc: coarse
 * output.
 * Key lists: when kv_offsets is NULL, list r is
 * kv_ids[r*topk .. r*topk + topk) (n_list_entries ignored); otherwise the
 * CSR lists as in block_sparse_attn_varlen, kv_ids holding n_list_entries
 * ids (topk ignored).  lse_f [B,heads,N] and
 * o_fine [B,heads,N,D] (fp32, cube-major) are written only if non-NULL
 * (both or neither).  order (optional, NULL = natural order): a permutation
 * of the B*heads*Nc query cubes (global ids (b*heads + h)*Nc + c) giving
 * the order in which the bf16 kernel runs them, as written by
 * vsa_fine_order; it changes no result.  An entry outside [0, B*heads*Nc)
 * runs nothing, so an order that is not a permutation leaves the rows of
 * the cubes it misses unwritten (and computes repeated cubes twice, with
 * the same result). */
int vsa_fine_forward(const void* q, const void* kp, const void* vp,
                     const float* oc, const void* gate_c, const void* gate_f,
                     int B, int heads, int head_dim, int T, int H, int W,
                     const int32_t* kv_offsets, const int32_t* kv_ids,
                     int64_t n_list_entries, int topk,
                     int dtype, void* out, float* lse_f, float* o_fine,
                     const int32_t* order, hipStream_t stream);

/* Processing order for the fine stage: each (b, h)'s query cubes sorted by
 * a key made from the entries at indices n/4 and 3n/4 of their key list of
 * n: each entry e becomes the 9-bit coordinate floor(e * 512 / Nc), and the
 * key interleaves the two (bit j of the first at bit 2j + 1, of the second
 * at bit 2j); cube index breaks ties.  Written as global ids into order
 * [B*heads*Nc] (int32).  Lists as in vsa_fine_forward; an empty list has
 * key 0, and an entry outside [0, Nc) counts as 0.  With ascending lists,
 * cubes whose lists cover similar key ranges then run side by side and
 * share more tile reads through the L2.  The forward entry points use it
 * for bf16 inputs.  Nc <= 4096. */
int vsa_fine_order(const int32_t* kv_offsets, const int32_t* kv_ids,
                   int64_t n_list_entries, int topk,
                   int B, int heads, int n_cubes, int32_t* order, hipStream_t stream);

/* --------------------------------------------------- list preconditions
 * vsa_validate_lists: checks caller-made key lists against what the fine
 * stage assumes ([VSA2-abs]: each query attends its own variable-length
 * set of key-value pairs, so the lists are caller input):
 *   CSR (kv_offsets non-NULL, n_rows + 1 entries): kv_offsets[0] == 0,
 *   non-decreasing, kv_offsets[n_rows] == n_list_entries;
 *   fixed length (kv_offsets NULL): n_rows lists of topk ids,
 *   n_list_entries == n_rows * topk;
 *   every id in [0, n_cubes) and no id twice within one list.
 * result (device, 2 int32, overwritten): result[0] = number of offset
 * faults, result[1] = number of lists with a bad or repeated id; both 0
 * means well formed.  Asynchronous like every call; read result after the
 * stream has drained.  n_cubes <= 4096 (VSA_ERR_UNSUPPORTED beyond).
 * VSA_VALIDATE=1 in the environment makes block_sparse_attn_varlen and
 * both backward calls run this check themselves, synchronize the stream
 * and return VSA_ERR_INVALID_ARG (queueing nothing more) for bad lists.
 */
int vsa_validate_lists(const int32_t* kv_offsets, const int32_t* kv_ids,
                       int64_t n_list_entries, int topk, int n_rows, int n_cubes,
                       int32_t* result, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* VSA_H */
