/*
 * vsa_probe.h - measurement helper of the MI355X VSA library (not part of
 * the operator).
 *
 * vsa_probe_tile_gather moves exactly the global bytes the fine stage of
 * [VSA-abs] ("VSA: Faster Video Diffusion with Trainable Sparse Attention",
 * Abstract: token attention only inside the selected tiles) reads for its
 * K and V operands, and does nothing else: one workgroup per (b, h, query
 * cube) streams the K and V tiles (64 x head_dim bf16 each, cube-major, as
 * written by vsa_cube_permute_pool) of the cube's `topk` selected key cubes
 * and folds them with XOR.  `depth` tiles are in flight per workgroup, and
 * workgroups are numbered as in the fine kernel (block i on XCD i % 8 takes
 * a contiguous range of query cubes).  Its time is the data-movement floor
 * of the fine stage for that selection.
 *
 * kp, vp: [BH, Nc, 64, head_dim] bf16 (device); ids: [BH, Nc, topk] int32
 * (device, each in [0, Nc), not checked on the GPU); sink: device buffer of
 * at least 4096 bytes, written only in the (never expected) case that the
 * folded value hits a fixed pattern.  head_dim in {64, 128}; depth in
 * {1, 2, 4, 8}.  Returns 0 on success, 1 on invalid arguments (nothing
 * queued), 4 if the launch failed.  Work is queued on `stream`.
 */
#ifndef VSA_PROBE_H
#define VSA_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int vsa_probe_tile_gather(const void* kp, const void* vp, int BH, int n_cubes, int head_dim,
                          const int32_t* ids, int topk, int depth, void* sink,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* VSA_PROBE_H */
