/*
 * splat.h - C ABI of libsplat, a tile rasterizer for point primitives on
 * AMD CDNA4 (gfx950).
 *
 * The method: project every primitive to the image, bin it to 16x16 pixel
 * tiles, sort each tile's list by depth, composite front to back per pixel,
 * and (optionally) send gradients back to the primitives and the camera.
 * Sources: Pulsar, "Efficient Sphere-based Neural Rendering" (arXiv
 * 2004.07484), sec. 3.2 and appendix B (enclosing rectangle, depth sort,
 * 16x16 blocks, draw with closest-five tracking, backward buffer, pixel-wise
 * backward, sphere-wise camera gradient); the NuRec profiling page
 * ("Optimizing NVIDIA Omniverse NuRec with Nsight...", sections on the
 * rendering kernel and renderBackward) for Gaussian splats, multi-sensor
 * (camera + lidar) rendering and the split camera/lidar backward.
 *
 * Conventions for every call:
 *  - All array pointers are caller-owned DEVICE memory unless marked HOST.
 *    The library allocates no device memory. Its global state, per device:
 *    (a) one side stream and two events, created by the first render call
 *    that composites Gaussians in both pinhole and spherical views (unless
 *    splat_params.serial_views = 1), and a mutex that such a call holds while
 *    it enqueues its work: those calls serialise their launches on one device
 *    (not their execution), and their pinhole views share the side stream;
 *    (b) the fixed device array of splat_bin_sort_noalloc. Every other call
 *    touches no library state, and calls on different streams may overlap.
 *  - Floating point arrays are fp32, row-major, C-contiguous.
 *  - Work is enqueued on `stream` (0 = the null stream); no call blocks on
 *    the device. Argument errors are detected on the host and returned before
 *    anything is enqueued. A failed launch returns SPLAT_ERR_HIP.
 *  - Pixel (i, j) is column i, row j, centred at (i + 0.5, j + 0.5).
 *  - Tiles are 16x16; view v has TW = ceil(W/16) x TH = ceil(H/16) tiles
 *    numbered ty*TW + tx; global tile ids stack the views in order.
 *  - Images are per view [Cv][H][W] (Cv = channels for pinhole views, 2 =
 *    (expected depth, opacity) for spherical views), views concatenated.
 *    Per-pixel buffers are per view [H][W], views concatenated.
 */
#ifndef SPLAT_H
#define SPLAT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPLAT_OK = 0,
  SPLAT_ERR_INVALID_ARG = -1,   /* bad pointer, size, kind or parameter (host check) */
  SPLAT_ERR_CAPACITY = -2,      /* workspace or buffer smaller than the size query */
  SPLAT_ERR_HIP = -3,           /* a HIP launch or query failed */
  SPLAT_ERR_UNSUPPORTED = -4    /* combination not implemented */
} splat_status;

typedef enum {
  SPLAT_PRIM_GAUSS2D = 0,       /* screen-space isotropic Gaussian splats */
  SPLAT_PRIM_GAUSS3D = 1,       /* anisotropic 3D Gaussian splats (EWA projection) */
  SPLAT_PRIM_SPHERE = 2         /* Pulsar-style spheres */
} splat_prim_kind;

typedef enum {
  SPLAT_CAM_PINHOLE = 0,
  SPLAT_CAM_SPHERICAL = 1,      /* lidar-like range view: columns = azimuth, rows = elevation */
  SPLAT_CAM_ORTHOGRAPHIC = 2    /* parallel projection along +z (spheres only, Pulsar B.1.1) */
} splat_cam_kind;

#define SPLAT_MAX_VIEWS 16
#define SPLAT_MAX_CHANNELS 64

/* HOST struct, one per view. Sensor point q = R x + t (R row-major).
 * Pinhole (x right, y down, z forward): u = fx qx/qz + cx, v = fy qy/qz + cy.
 * Orthographic (same axes; spheres only, other primitives return
 *   SPLAT_ERR_UNSUPPORTED): u = fx qx + cx, v = fy qy + cy with fx, fy in pixels per
 *   world unit; the ray of pixel centre (px, py) runs along +z through
 *   ((px - cx)/fx, (py - cy)/fy, 0), and a sphere keeps a radius of at least 0.75 px.
 * Spherical (x forward, y left, z up; width must be a multiple of 16):
 *   u = (pi - atan2(qy, qx)) W / (2 pi), v = (el_max - atan2(qz, |q_xy|)) H / (el_max - el_min).
 * znear culls (depth <= znear); for spheres znear/zfar also normalise depth: a
 * sphere view needs zfar > znear (else SPLAT_ERR_INVALID_ARG), and a sphere is
 * culled unless its front depth qz - r_eff, rounded to fp32, lies in (znear, zfar):
 * behind the far plane the early-stop bound would not hold (Pulsar sec. 3.2). */
typedef struct {
  int32_t kind, width, height;
  float R[9], t[3];
  float fx, fy, cx, cy;
  float el_min_deg, el_max_deg;
  float znear, zfar;
} splat_camera;

/* HOST struct of DEVICE pointers, one array per attribute (structure of arrays).
 *   GAUSS2D: pos [n][2] pixel centres, scale [n] sigma (px), depth [n] (> 0)
 *   GAUSS3D: pos [n][3] means, scale [n][3] axis scales, rot [n][4] quaternion (w,x,y,z),
 *            normalised inside the library
 *   SPHERE:  pos [n][3] centres, scale [n] radius
 *   all:     opacity [n] in (0, 1], feat [n][channels] (may be NULL if only spherical views) */
typedef struct {
  int32_t kind, n, channels;
  const float *pos, *scale, *rot, *opacity, *depth, *feat;
} splat_prims;

/* HOST struct. Gaussian alpha blending: alpha = min(alpha_max, o exp(-power)); entries
 * with alpha < alpha_min are skipped; a pixel stops after the entry that brings its
 * transmittance below T_min (Gaussians: T_min >= 1e-30, else SPLAT_ERR_INVALID_ARG,
 * so that the fp32 T_final the reverse pass divides back from cannot underflow).
 * Sphere blending: w = o D exp(o zhat / gamma) with
 * D = 1 - dist^2/r^2 (orthogonal ray distance), zhat = (zfar - qz)/(zfar - znear);
 * colour = (sum w f + bg_weight bg) / (sum w + bg_weight); a pixel stops at the first
 * sphere whose bound exp(zhat(front depth)/gamma) < tau * (sum w + bg_weight); the first
 * top_k contributing spheres per pixel are recorded and receive gradients. */
typedef struct {
  float alpha_min, alpha_max, T_min;
  float gamma, bg_weight, tau;
  int32_t top_k;                 /* 1..8 */
  const float *background;       /* HOST [channels] or NULL (= 0) */
  /* Spheres: 0 records each pixel's first top_k contributing spheres in list
   * order; 1 records the top_k contributing spheres whose surface the pixel's ray
   * enters first (smallest sensor depth of the entry point, list order breaking
   * ties; Pulsar B.1.3 and B.1.4 keep the closest five intersections). Either way
   * topk lists them in list order and only they receive gradients. Must be 0 for
   * Gaussians. */
  int32_t top_by_depth;
  /* Spheres: 1 blends relative to a per-pixel shift m = max(0, largest ln(o) +
   * o zhat / gamma of a contributing sphere), so that no weight overflows fp32
   * (required for gamma < 1/88, where exp(o zhat / gamma) can exceed the fp32
   * range). The image is unchanged; norm holds the normalisation times exp(-m),
   * and T_final (spheres: otherwise unused) receives m, which splat_render_bwd
   * then reads (T_final must be given to both calls). Must be 0 for Gaussians. */
  int32_t max_shift;
  /* Gaussians, render calls over both pinhole and spherical views: 0 (default) runs
   * the pinhole views on the library's side stream for the device, beside the
   * spherical views on `stream` (forked from and joined back into `stream`, see the
   * conventions above); 1 runs every kernel on `stream` alone, using no library state.
   * Must be 0 or 1. */
  int32_t serial_views;
} splat_params;

/* Gradient outputs (DEVICE); NULL = not requested (skipped, nothing written).
 * Shapes follow the inputs; cam_R [n_views][9], cam_t [n_views][3] (spheres only).
 * cam_K [n_views][4]: d loss / d (fx, fy, cx, cy) of each view, spheres only
 * (Pulsar section 3.2 and appendix A: gradients for the focal length and the
 * sensor placement); the pixel rays move with the intrinsics, while the
 * one-pixel radius floor, the tile rectangles and the gate are held fixed.
 * A non-NULL cam_K with Gaussian primitives returns SPLAT_ERR_UNSUPPORTED.
 * accumulate = 0: outputs are overwritten (zeroed on-stream first);
 * accumulate = 1: the call's gradients are added to what the buffers hold.
 * normalize = 1 (spheres only; Pulsar B.2): each sphere's position, radius,
 * opacity and feature gradients are divided by the number of pixels of the
 * call's views that recorded it among their top_k; each sphere's camera (R, t)
 * contribution is divided by its projected area in pixels, pi (fx r_eff / qz)
 * (fy r_eff / qz) (orthographic: pi (fx r_eff)(fy r_eff)), and by 1e-3. cam_K
 * stays the raw sum. normalize = 1 with Gaussians returns SPLAT_ERR_UNSUPPORTED.
 * sums_cleared = 1: the caller states that the
 * splat_render_fwd call before this one on the stream was given this call's workspace
 * (so it cleared the sums the reverse pass accumulates into) and that no
 * splat_render_bwd has used the workspace since; the call then skips that clearing.
 * Stating it falsely gives wrong gradients; 0 is always correct.
 * atomic_direct_max (spheres, up to four channels, without cam_K or normalize;
 * otherwise ignored): 0 (default) sums every recorded sphere's terms over the
 * wavefront before its global atomic adds; k > 0 lets the lanes of a wavefront
 * add their own terms with global atomics when at most k of them recorded the
 * sphere (the split between in-register reduction and atomic units of DISTWAR,
 * arXiv author page abstract). Same gradients up to summation order; on gfx950 it
 * measured slower for every k, so 0 is the default. Negative values are rejected. */
typedef struct {
  float *pos, *scale, *rot, *opacity, *feat;
  float *cam_R, *cam_t;
  float *cam_K;
  int32_t accumulate;
  int32_t normalize;
  int32_t sums_cleared;
  int32_t atomic_direct_max;
} splat_grads;

/* ---- size queries (host only, no device work) ---------------------------- */

/* Bytes of the opaque projected-record buffer for n_views x n primitives. */
size_t splat_projected_bytes(int n_views, int n);
/* Total 16x16 tiles over the views; -1 on invalid cameras. */
int64_t splat_total_tiles(const splat_camera *cams, int n_views);
/* Workspace bytes for splat_bin_sort with the given pair capacity. */
size_t splat_sort_workspace_bytes(const splat_camera *cams, int n_views, int n, int64_t capacity);
/* Workspace bytes for splat_render_bwd. */
size_t splat_bwd_workspace_bytes(int n_views, int n, int channels);

/* ---- the four calls ------------------------------------------------------ */

/* Project every (view, primitive): the per-primitive "Step 0" of Pulsar appendix B.1.1
 * (enclosing rectangle, depth, blending constants) and EWA splatting for Gaussians.
 * proj: [splat_projected_bytes] opaque records. pair_counts: [n_views*n] uint32, the
 * number of tiles each record overlaps (0 = culled: behind znear, degenerate, off image).
 * Spheres with up to four channels: the records also keep a copy of each primitive's
 * features (read from prims->feat here), which splat_render_fwd and splat_render_bwd
 * use; re-project after changing the features. */
int splat_project(const splat_camera *cams, int n_views, const splat_prims *prims,
                  const splat_params *prm, void *proj, uint32_t *pair_counts, hipStream_t stream);

/* Bin to tiles and depth-sort each tile's list (Pulsar B.1.1 depth sort, B.1.2 16x16 blocks):
 * one (key, value) per overlapped tile with key = (global tile << 32) | fp32 bits of the
 * depth and value = record index (view*n + i), ordered by (tile, depth bits, record index):
 * pairs are counted per tile, bucketed by tile, and each tile's segment is sorted by
 * (depth bits, record index); tile_ranges gives each tile's [start, end).
 * keys/vals: [capacity]; tile_ranges: [total_tiles][2] uint32 (empty tiles: 0, 0).
 * num_pairs (device int64) receives the needed pair count. If it exceeds capacity,
 * *overflow (device int32) is set to 1 and nothing else is written; the render calls
 * then return without writing. Otherwise *overflow is set to 0.
 * workspace: [splat_sort_workspace_bytes] device bytes. */
int splat_bin_sort(const splat_camera *cams, int n_views, int n, const void *proj,
                   const uint32_t *pair_counts, int64_t capacity, uint64_t *keys, uint32_t *vals,
                   uint32_t *tile_ranges, int64_t *num_pairs, int32_t *overflow, void *workspace,
                   size_t ws_bytes, hipStream_t stream);

/* splat_bin_sort without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, outputs and errors as splat_bin_sort; the workspace is
 * a fixed device array of SPLAT_NOALLOC_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends. Calls whose splat_sort_workspace_bytes exceeds it return
 * SPLAT_ERR_CAPACITY before any launch. The call allocates nothing (its first call on a
 * device only looks up that device's copy of the array). Every call on one GPU shares
 * that array: calls that overlap on one GPU (several streams or threads) race and must
 * be serialised by the caller. */
#define SPLAT_NOALLOC_SCRATCH_BYTES (64u << 20)
int splat_bin_sort_noalloc(const splat_camera *cams, int n_views, int n, const void *proj,
                           const uint32_t *pair_counts, int64_t capacity, uint64_t *keys, uint32_t *vals,
                           uint32_t *tile_ranges, int64_t *num_pairs, int32_t *overflow, hipStream_t stream);

/* Composite front to back per pixel, one workgroup per tile with the tile's list staged
 * through LDS in batches (Pulsar B.1.2-B.1.4; NuRec rendering kernel).
 *   img: image layout above.
 *   Gaussians: T_final [pixels] final transmittance, last [pixels] number of list entries
 *     up to and including the last composited one (the backward replays from there).
 *   Spheres: norm [pixels] the normalisation sum, topk [pixels][top_k] int32: for each of
 *     the first top_k contributing spheres, its index into the sorted keys/vals arrays of
 *     splat_bin_sort (-1 padded); vals[index] - view*n is the primitive id. Together they
 *     are the backward buffer of Pulsar B.1.4. Sphere outputs need capacity < 2^31.
 *     T_final/last may be NULL for spheres, norm/topk for Gaussians.
 * bwd_workspace (optional, may be NULL): the workspace of the splat_render_bwd call that
 *   follows on this stream, bwd_ws_bytes >= splat_bwd_workspace_bytes, 16-byte aligned.
 *   The forward then also clears the sums the reverse pass accumulates into (spheres: in
 *   workgroups appended to its grid that run while its longest tiles finish; Gaussians:
 *   in a launch after the pinhole views' kernel, which runs beside the spherical views'
 *   longest tiles when the call has both); that call can then pass
 *   splat_grads.sums_cleared = 1 and skip its own clearing. Errors: SPLAT_ERR_CAPACITY
 *   (too small), SPLAT_ERR_INVALID_ARG (misaligned). */
int splat_render_fwd(const splat_camera *cams, int n_views, const splat_prims *prims,
                     const splat_params *prm, const void *proj, const uint32_t *vals,
                     const uint32_t *tile_ranges, const int32_t *overflow, float *img,
                     float *T_final, uint32_t *last, float *norm, int32_t *topk,
                     void *bwd_workspace, size_t bwd_ws_bytes, hipStream_t stream);

/* Reverse pass for views [view_begin, view_begin + view_count): per-pixel gradients
 * reduced per primitive within each wavefront before global atomics, then the chain
 * rule per primitive and, for spheres, the sphere-wise camera gradient with a
 * device-wide reduction (Pulsar B.2). Pinhole and spherical views run in separate
 * kernels (the NuRec camera/lidar split). dL_dimg has the img layout (all views).
 * The forward outputs must come from splat_render_fwd on the same inputs.
 * workspace: [splat_bwd_workspace_bytes] device bytes. */
int splat_render_bwd(const splat_camera *cams, int n_views, int view_begin, int view_count,
                     const splat_prims *prims, const splat_params *prm, const void *proj,
                     const uint32_t *vals, const uint32_t *tile_ranges, const int32_t *overflow,
                     const float *img, const float *T_final, const uint32_t *last,
                     const float *norm, const int32_t *topk, const float *dL_dimg,
                     const splat_grads *grads, void *workspace, size_t ws_bytes,
                     hipStream_t stream);

/* ---- per-frame parameter assembly ---------------------------------------------
 * NuRec's profiling page ("Fusing small kernels and removing synchronizations"):
 * the per-frame interpolate step that assembles the primitives' parameters before
 * rendering, fused into one kernel. The page does not say what is interpolated;
 * here each primitive carries its centre and rotation quaternion at n_keys keyframe
 * times. For time t the bracketing keyframes k, k1 (key_times[k] <= t <=
 * key_times[k1]; t outside the range clamps to the end frame) and w = (t - t_k) /
 * (t_k1 - t_k) give
 *   pos = (1 - w) key_pos[k] + w key_pos[k1],
 *   rot = (1 - w) key_rot[k] + w s key_rot[k1],  s = -1 if their dot product < 0
 * (normalised linear interpolation on the shorter arc; splat_project normalises).
 * key_times: HOST [n_keys], finite, strictly increasing. key_pos [n_keys][n][3],
 * key_rot [n_keys][n][4], pos [n][3], rot [n][4]: DEVICE, caller-owned; rotation
 * buffers 16-byte aligned. A NULL key_pos/pos (or key_rot/rot) pair skips that
 * output. Argument errors return SPLAT_ERR_INVALID_ARG before any launch. */
int splat_interpolate(const float *key_times, int n_keys, float t, int n, const float *key_pos,
                      const float *key_rot, float *pos, float *rot, hipStream_t stream);

/* Reverse of splat_interpolate: ADDS the gradients w.r.t. the bracketing keyframes'
 * centres and rotations (frames k and k1 of d_key_pos [n_keys][n][3], d_key_rot
 * [n_keys][n][4]; the other frames are not touched, so the caller zeroes the buffers
 * once and can sum several frames) given d_pos [n][3], d_rot [n][4]. The sign s is a
 * discrete choice and carries no gradient. key_rot is needed for s when d_rot is
 * given. NULL d_pos/d_key_pos (or d_rot/d_key_rot) skips that part. */
int splat_interpolate_bwd(const float *key_times, int n_keys, float t, int n, const float *key_rot,
                          const float *d_pos, const float *d_rot, float *d_key_pos, float *d_key_rot,
                          hipStream_t stream);

const char *splat_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPLAT_H */
