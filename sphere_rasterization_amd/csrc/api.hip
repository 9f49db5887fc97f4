// extern "C" entry points of libsplat: argument checks on the host, view-table
// construction, then kernel launches on the caller's stream. No allocation of
// device memory and no host synchronisation. Global state per device: one side
// stream with its two events and lock (created on first use, see side_begin),
// and the array of splat_bin_sort_noalloc.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "render_common.h"
#include "splat_internal.h"

int launch_project(const ViewTable &vt, const splat_prims *pr, double gamma, double alpha_min, int max_shift,
                   void *proj, uint32_t *counts, hipStream_t stream);
size_t sort_workspace_bytes(const ViewTable &vt, int n, long long capacity);
int launch_bin_sort(const ViewTable &vt, int n, const void *proj, const uint32_t *counts, long long capacity,
                    uint64_t *keys, uint32_t *vals, uint32_t *ranges, int64_t *num_pairs, int32_t *overflow,
                    void *workspace, hipStream_t stream);
int launch_render_fwd(const ViewTable &vt, const FwdArgs &A, int kind, hipStream_t stream);
size_t bwd_workspace_bytes(long long nrec, int C);
int launch_render_bwd(const ViewTable &vt, int vbeg, int vend, BwdArgs A, const splat_prims *pr, BinArrays bin,
                      const splat_grads *gr, hipStream_t stream);
int launch_assemble(const float *key_pos, const float *key_rot, int k, int k1, float w, long long n, float *pos,
                    float *rot, hipStream_t stream);
int launch_assemble_bwd(const float *key_rot, int k, int k1, float w, long long n, const float *d_pos,
                        const float *d_rot, float *d_key_pos, float *d_key_rot, hipStream_t stream);

namespace {

struct SideStream {
  std::mutex mu;                 // held from side_begin to side_end
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];

}  // namespace

int side_begin(hipStream_t main, hipStream_t *side) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPLAT_ERR_HIP;
  SideStream &ss = g_side[dev];
  ss.mu.lock();
  if (!ss.s) {
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess) ss.s = nullptr;
    if (ss.s && hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess) ss.fork = nullptr;
    if (ss.s && hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) ss.join = nullptr;
    if (!ss.s || !ss.fork || !ss.join) {
      if (ss.fork) (void)hipEventDestroy(ss.fork);
      if (ss.s) (void)hipStreamDestroy(ss.s);
      ss.s = nullptr;
      ss.fork = ss.join = nullptr;
      ss.mu.unlock();
      return SPLAT_ERR_HIP;
    }
  }
  if (hipEventRecord(ss.fork, main) != hipSuccess || hipStreamWaitEvent(ss.s, ss.fork, 0) != hipSuccess) {
    ss.mu.unlock();
    return SPLAT_ERR_HIP;
  }
  *side = ss.s;
  return SPLAT_OK;
}

int side_end(hipStream_t main, hipStream_t side) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPLAT_ERR_HIP;
  SideStream &ss = g_side[dev];
  int rc = SPLAT_OK;
  if (side != ss.s || hipEventRecord(ss.join, ss.s) != hipSuccess || hipStreamWaitEvent(main, ss.join, 0) != hipSuccess)
    rc = SPLAT_ERR_HIP;
  ss.mu.unlock();
  return rc;
}

namespace {

bool debug_enabled() {
  static int v = -1;
  if (v < 0) {
    const char *e = getenv("SPLAT_DEBUG");
    v = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return v == 1;
}

int fail(int code, const char *what) {
  if (debug_enabled()) fprintf(stderr, "libsplat: %s (%d)\n", what, code);
  return code;
}

#define CHECK(cond, code, msg) \
  do {                         \
    if (!(cond)) return fail(code, msg); \
  } while (0)

// Validate cameras and build the device view table. Returns SPLAT_OK or an error.
int build_views(const splat_camera *cams, int n_views, int channels, ViewTable *vt) {
  CHECK(cams != nullptr, SPLAT_ERR_INVALID_ARG, "cams is NULL");
  CHECK(n_views >= 1 && n_views <= SPLAT_MAX_VIEWS, SPLAT_ERR_INVALID_ARG, "n_views out of range");
  memset(vt, 0, sizeof(*vt));
  vt->n = n_views;
  long long toff = 0, poff = 0, ioff = 0;
  for (int v = 0; v < n_views; v++) {
    const splat_camera &c = cams[v];
    ViewDev &d = vt->v[v];
    CHECK(c.kind == SPLAT_CAM_PINHOLE || c.kind == SPLAT_CAM_SPHERICAL || c.kind == SPLAT_CAM_ORTHOGRAPHIC,
          SPLAT_ERR_INVALID_ARG, "camera kind");
    CHECK(c.width > 0 && c.height > 0 && c.width <= (1 << 20) && c.height <= (1 << 20), SPLAT_ERR_INVALID_ARG,
          "camera size");
    for (int k = 0; k < 9; k++) CHECK(isfinite(c.R[k]), SPLAT_ERR_INVALID_ARG, "camera R not finite");
    for (int k = 0; k < 3; k++) CHECK(isfinite(c.t[k]), SPLAT_ERR_INVALID_ARG, "camera t not finite");
    CHECK(isfinite(c.znear) && isfinite(c.zfar) && c.znear >= 0.0f, SPLAT_ERR_INVALID_ARG, "camera depth range");
    if (c.kind != SPLAT_CAM_SPHERICAL) {
      CHECK(isfinite(c.fx) && isfinite(c.fy) && c.fx > 0.0f && c.fy > 0.0f, SPLAT_ERR_INVALID_ARG, "focal length");
      CHECK(isfinite(c.cx) && isfinite(c.cy), SPLAT_ERR_INVALID_ARG, "principal point");
    } else {
      CHECK(c.width % TILE == 0, SPLAT_ERR_INVALID_ARG, "spherical width must be a multiple of 16");
      CHECK(isfinite(c.el_min_deg) && isfinite(c.el_max_deg) && c.el_max_deg > c.el_min_deg, SPLAT_ERR_INVALID_ARG,
            "elevation range");
    }
    d.kind = c.kind;
    d.W = c.width;
    d.H = c.height;
    d.TW = (c.width + TILE - 1) / TILE;
    d.TH = (c.height + TILE - 1) / TILE;
    CHECK(d.TW <= 65535 && d.TH <= 65535, SPLAT_ERR_INVALID_ARG, "too many tiles");
    d.tile_off = (int)toff;
    d.chan = c.kind == SPLAT_CAM_SPHERICAL ? 2 : channels;
    d.pix_off = poff;
    d.img_off = ioff;
    memcpy(d.R, c.R, sizeof(d.R));
    memcpy(d.t, c.t, sizeof(d.t));
    d.fx = c.fx; d.fy = c.fy; d.cx = c.cx; d.cy = c.cy;
    d.el_min = c.el_min_deg; d.el_max = c.el_max_deg; d.znear = c.znear; d.zfar = c.zfar;
    d.ifx = c.kind == SPLAT_CAM_SPHERICAL ? 0.0 : 1.0 / (double)c.fx;
    d.ify = c.kind == SPLAT_CAM_SPHERICAL ? 0.0 : 1.0 / (double)c.fy;
    d.ispan = c.zfar > c.znear ? 1.0 / ((double)c.zfar - (double)c.znear) : 0.0;
    toff += (long long)d.TW * d.TH;
    poff += (long long)c.width * c.height;
    ioff += (long long)d.chan * c.width * c.height;
  }
  CHECK(toff < (1ll << 31), SPLAT_ERR_INVALID_ARG, "too many tiles");
  vt->total_tiles = (int)toff;
  vt->total_pix = poff;
  return SPLAT_OK;
}

int check_prims(const splat_prims *p, const ViewTable &vt) {
  CHECK(p != nullptr, SPLAT_ERR_INVALID_ARG, "prims is NULL");
  CHECK(p->kind == SPLAT_PRIM_GAUSS2D || p->kind == SPLAT_PRIM_GAUSS3D || p->kind == SPLAT_PRIM_SPHERE,
        SPLAT_ERR_INVALID_ARG, "primitive kind");
  CHECK(p->n >= 0, SPLAT_ERR_INVALID_ARG, "negative n");
  CHECK(p->channels >= 0 && p->channels <= SPLAT_MAX_CHANNELS, SPLAT_ERR_INVALID_ARG, "channels out of range");
  CHECK((long long)vt.n * p->n < (1ll << 32) - 1, SPLAT_ERR_INVALID_ARG, "too many records");
  bool any_pin = false, any_sph = false, any_orth = false;
  for (int v = 0; v < vt.n; v++) {
    if (vt.v[v].kind == SPLAT_CAM_SPHERICAL) any_sph = true;
    else if (vt.v[v].kind == SPLAT_CAM_ORTHOGRAPHIC) any_orth = true;
    else any_pin = true;
  }
  if (p->kind == SPLAT_PRIM_SPHERE) {
    CHECK(!any_sph, SPLAT_ERR_UNSUPPORTED, "spheres need pinhole or orthographic views");
    // the normalised device depth (zfar - qz) / (zfar - znear) needs a positive span
    for (int v = 0; v < vt.n; v++)
      CHECK(vt.v[v].zfar > vt.v[v].znear, SPLAT_ERR_INVALID_ARG, "sphere views need zfar > znear");
  }
  else CHECK(!any_orth, SPLAT_ERR_UNSUPPORTED, "orthographic views are for spheres only");
  if (p->kind == SPLAT_PRIM_GAUSS2D) CHECK(!any_sph, SPLAT_ERR_UNSUPPORTED, "screen-space Gaussians need pinhole views");
  if (p->n == 0) return SPLAT_OK;
  CHECK(p->pos && p->scale && p->opacity, SPLAT_ERR_INVALID_ARG, "missing primitive arrays");
  if (p->kind == SPLAT_PRIM_GAUSS3D) CHECK(p->rot != nullptr, SPLAT_ERR_INVALID_ARG, "missing rotations");
  if (p->kind == SPLAT_PRIM_GAUSS2D) CHECK(p->depth != nullptr, SPLAT_ERR_INVALID_ARG, "missing depths");
  if (any_pin || any_orth) CHECK(p->channels >= 1 && p->feat != nullptr, SPLAT_ERR_INVALID_ARG, "missing features");
  return SPLAT_OK;
}

int check_params(const splat_params *m, int kind) {
  CHECK(m != nullptr, SPLAT_ERR_INVALID_ARG, "params is NULL");
  CHECK(isfinite(m->alpha_min) && isfinite(m->alpha_max) && isfinite(m->T_min), SPLAT_ERR_INVALID_ARG,
        "alpha parameters");
  CHECK(m->alpha_max > 0.0f && m->alpha_max < 1.0f, SPLAT_ERR_INVALID_ARG, "alpha_max must lie in (0, 1)");
  CHECK(m->alpha_min >= 0.0f && m->T_min >= 0.0f, SPLAT_ERR_INVALID_ARG, "negative thresholds");
  CHECK(m->serial_views == 0 || m->serial_views == 1, SPLAT_ERR_INVALID_ARG, "serial_views must be 0 or 1");
  if (kind == SPLAT_PRIM_SPHERE) {
    CHECK(isfinite(m->gamma) && m->gamma > 0.0f, SPLAT_ERR_INVALID_ARG, "gamma must be > 0");
    CHECK(isfinite(m->tau) && m->tau >= 0.0f, SPLAT_ERR_INVALID_ARG, "tau must be >= 0");
    CHECK(isfinite(m->bg_weight) && m->bg_weight > 0.0f, SPLAT_ERR_INVALID_ARG, "bg_weight must be > 0");
    CHECK(m->top_k >= 1 && m->top_k <= SPLAT_TOPK_MAX, SPLAT_ERR_INVALID_ARG, "top_k must be in 1..8");
    CHECK(m->top_by_depth == 0 || m->top_by_depth == 1, SPLAT_ERR_INVALID_ARG, "top_by_depth must be 0 or 1");
    CHECK(m->max_shift == 0 || m->max_shift == 1, SPLAT_ERR_INVALID_ARG, "max_shift must be 0 or 1");
    CHECK(m->max_shift || m->gamma >= 1.0f / 88.0f, SPLAT_ERR_INVALID_ARG,
          "gamma below 1/88 overflows fp32 sphere weights: set max_shift");
  } else {
    // the reverse pass rebuilds each entry's transmittance from the fp32 T_final
    // by dividing out (1 - alpha): a T_min that lets T_final underflow fp32 would
    // zero or garble those gradients
    CHECK(m->T_min >= 1e-30f, SPLAT_ERR_INVALID_ARG, "T_min below 1e-30 underflows the stored transmittance");
    CHECK(m->top_by_depth == 0, SPLAT_ERR_UNSUPPORTED, "top_by_depth is for spheres only");
    CHECK(m->max_shift == 0, SPLAT_ERR_UNSUPPORTED, "max_shift is for spheres only");
  }
  return SPLAT_OK;
}

// Keyframe bracket of time t: frames k, k1 and the weight of k1 (host, fp64).
int key_bracket(const float *key_times, int n_keys, float t, int *k, int *k1, float *w) {
  CHECK(key_times != nullptr && n_keys >= 1, SPLAT_ERR_INVALID_ARG, "key times");
  CHECK(isfinite(t), SPLAT_ERR_INVALID_ARG, "time not finite");
  for (int i = 0; i < n_keys; i++) {
    CHECK(isfinite(key_times[i]), SPLAT_ERR_INVALID_ARG, "key time not finite");
    CHECK(i == 0 || key_times[i] > key_times[i - 1], SPLAT_ERR_INVALID_ARG, "key times must increase");
  }
  if (n_keys == 1 || t <= key_times[0]) {
    *k = *k1 = 0;
    *w = 0.0f;
  } else if (t >= key_times[n_keys - 1]) {
    *k = *k1 = n_keys - 1;
    *w = 0.0f;
  } else {
    int i = 0;
    while (!(key_times[i] <= t && t < key_times[i + 1])) i++;
    *k = i;
    *k1 = i + 1;
    *w = (float)(((double)t - (double)key_times[i]) / ((double)key_times[i + 1] - (double)key_times[i]));
  }
  return SPLAT_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

size_t splat_projected_bytes(int n_views, int n) {
  if (n_views < 1 || n < 0) return 0;
  return proj_bytes((long long)n_views * n);
}

int64_t splat_total_tiles(const splat_camera *cams, int n_views) {
  ViewTable vt;
  if (build_views(cams, n_views, 1, &vt) != SPLAT_OK) return -1;
  return vt.total_tiles;
}

size_t splat_sort_workspace_bytes(const splat_camera *cams, int n_views, int n, int64_t capacity) {
  ViewTable vt;
  if (build_views(cams, n_views, 1, &vt) != SPLAT_OK || n < 0 || capacity < 0) return 0;
  return sort_workspace_bytes(vt, n, capacity);
}

size_t splat_bwd_workspace_bytes(int n_views, int n, int channels) {
  if (n_views < 1 || n < 0 || channels < 0) return 0;
  return bwd_workspace_bytes((long long)n_views * n, channels);
}

int splat_project(const splat_camera *cams, int n_views, const splat_prims *prims, const splat_params *prm,
                  void *proj, uint32_t *pair_counts, hipStream_t stream) {
  ViewTable vt;
  int st = build_views(cams, n_views, prims ? prims->channels : 0, &vt);
  if (st) return st;
  if ((st = check_prims(prims, vt))) return st;
  if ((st = check_params(prm, prims->kind))) return st;
  if (prims->n == 0) return SPLAT_OK;
  CHECK(proj && pair_counts, SPLAT_ERR_INVALID_ARG, "proj / pair_counts NULL");
  return launch_project(vt, prims, (double)prm->gamma, (double)prm->alpha_min, prm->max_shift, proj, pair_counts,
                        stream);
}

int splat_bin_sort(const splat_camera *cams, int n_views, int n, const void *proj, const uint32_t *pair_counts,
                   int64_t capacity, uint64_t *keys, uint32_t *vals, uint32_t *tile_ranges, int64_t *num_pairs,
                   int32_t *overflow, void *workspace, size_t ws_bytes, hipStream_t stream) {
  ViewTable vt;
  int st = build_views(cams, n_views, 1, &vt);
  if (st) return st;
  CHECK(n >= 0 && (long long)n_views * n < (1ll << 32) - 1, SPLAT_ERR_INVALID_ARG, "n out of range");
  CHECK(capacity >= 0 && capacity < (1ll << 32) - 1, SPLAT_ERR_INVALID_ARG, "capacity out of range");
  CHECK(tile_ranges && num_pairs && overflow, SPLAT_ERR_INVALID_ARG, "NULL output");
  CHECK(n == 0 || (proj && pair_counts), SPLAT_ERR_INVALID_ARG, "NULL input");
  CHECK(capacity == 0 || (keys && vals), SPLAT_ERR_INVALID_ARG, "NULL keys / vals");
  CHECK(workspace != nullptr, SPLAT_ERR_INVALID_ARG, "NULL workspace");
  CHECK(ws_bytes >= sort_workspace_bytes(vt, n, capacity), SPLAT_ERR_CAPACITY,
        "sort workspace too small");
  return launch_bin_sort(vt, n, proj, pair_counts, capacity, keys, vals, tile_ranges, num_pairs, overflow, workspace,
                         stream);
}

// ---- splat_bin_sort_noalloc: the sort workspace in a fixed device array ----
// For callers that cannot allocate device memory. The array is file-scope device
// memory: its name in host code is only a host-side stand-in, so host code uses the
// address hipGetSymbolAddress gives on each device (looked up once per device on
// that device's first call), never the name itself.
namespace {

static __device__ __align__(256) unsigned char scratch[SPLAT_NOALLOC_SCRATCH_BYTES];

struct ScratchAddr {
  std::once_flag once;
  void *ptr = nullptr;
  int rc = SPLAT_OK;
};
ScratchAddr g_scratch[kMaxDevices];

// The calling thread's current device's copy of scratch (or an error).
int scratch_address(void **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(SPLAT_ERR_HIP, "current device");
  ScratchAddr &sa = g_scratch[dev];
  std::call_once(sa.once, [&sa]() {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      sa.rc = SPLAT_ERR_HIP;
      return;
    }
    sa.ptr = p;
  });
  if (sa.rc != SPLAT_OK) return fail(sa.rc, "scratch symbol address");
  *ptr = sa.ptr;
  return SPLAT_OK;
}

}  // namespace

int splat_bin_sort_noalloc(const splat_camera *cams, int n_views, int n, const void *proj,
                           const uint32_t *pair_counts, int64_t capacity, uint64_t *keys, uint32_t *vals,
                           uint32_t *tile_ranges, int64_t *num_pairs, int32_t *overflow, hipStream_t stream) {
  ViewTable vt;
  int st = build_views(cams, n_views, 1, &vt);
  if (st) return st;
  CHECK(n >= 0 && (long long)n_views * n < (1ll << 32) - 1, SPLAT_ERR_INVALID_ARG, "n out of range");
  CHECK(capacity >= 0 && capacity < (1ll << 32) - 1, SPLAT_ERR_INVALID_ARG, "capacity out of range");
  CHECK(tile_ranges && num_pairs && overflow, SPLAT_ERR_INVALID_ARG, "NULL output");
  CHECK(n == 0 || (proj && pair_counts), SPLAT_ERR_INVALID_ARG, "NULL input");
  CHECK(capacity == 0 || (keys && vals), SPLAT_ERR_INVALID_ARG, "NULL keys / vals");
  CHECK(sort_workspace_bytes(vt, n, capacity) <= (size_t)SPLAT_NOALLOC_SCRATCH_BYTES, SPLAT_ERR_CAPACITY,
        "sort workspace exceeds SPLAT_NOALLOC_SCRATCH_BYTES");
  void *ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return launch_bin_sort(vt, n, proj, pair_counts, capacity, keys, vals, tile_ranges, num_pairs, overflow, ws, stream);
}

int splat_render_fwd(const splat_camera *cams, int n_views, const splat_prims *prims, const splat_params *prm,
                     const void *proj, const uint32_t *vals, const uint32_t *tile_ranges, const int32_t *overflow,
                     float *img, float *T_final, uint32_t *last, float *norm, int32_t *topk, void *bwd_workspace,
                     size_t bwd_ws_bytes, hipStream_t stream) {
  ViewTable vt;
  int st = build_views(cams, n_views, prims ? prims->channels : 0, &vt);
  if (st) return st;
  if ((st = check_prims(prims, vt))) return st;
  if ((st = check_params(prm, prims->kind))) return st;
  CHECK(img && tile_ranges && overflow, SPLAT_ERR_INVALID_ARG, "NULL output");
  CHECK(prims->n == 0 || (proj && vals), SPLAT_ERR_INVALID_ARG, "NULL proj / vals");
  CHECK(prims->n > 0, SPLAT_ERR_INVALID_ARG, "render needs at least one primitive");
  FwdArgs A;
  memset(&A, 0, sizeof(A));
  A.n = prims->n; A.C = prims->channels; A.top_k = prm->top_k; A.top_by_depth = prm->top_by_depth;
  A.max_shift = prm->max_shift;
  A.serial_views = prm->serial_views;
  A.alpha_min = prm->alpha_min; A.alpha_max = prm->alpha_max; A.T_min = prm->T_min;
  A.tau = prm->tau; A.bg_weight = prm->bg_weight;
  for (int c = 0; c < A.C; c++) A.bg[c] = prm->background ? prm->background[c] : 0.0f;
  ProjLayout L = proj_layout(const_cast<void *>(proj), (long long)n_views * prims->n);
  A.draw = L.draw; A.aux = L.aux; A.vals = vals; A.ranges = tile_ranges; A.overflow = overflow;
  A.feat = prims->feat; A.img = img; A.T_final = T_final; A.last = last; A.norm = norm; A.topk = topk;
  if (bwd_workspace) {
    const long long nrec = (long long)n_views * prims->n;
    CHECK(((uintptr_t)bwd_workspace & 15u) == 0, SPLAT_ERR_INVALID_ARG, "backward workspace not 16-byte aligned");
    CHECK(bwd_ws_bytes >= bwd_workspace_bytes(nrec, prims->channels), SPLAT_ERR_CAPACITY,
          "backward workspace smaller than splat_bwd_workspace_bytes");
  }
  if (bwd_workspace && prims->kind != SPLAT_PRIM_SPHERE) {
    // Gaussians: the fp64 geometric and feature sums of every record (each region
    // starts on an aligned boundary and is padded past its end)
    const long long nrec = (long long)n_views * prims->n;
    const AccLayout acc = acc_layout(bwd_workspace, nrec, prims->channels);
    A.clr[0] = reinterpret_cast<uint4 *>(acc.g);
    A.nclr[0] = (nrec * ACC_G * (long long)sizeof(double) + 15) / 16;
    A.clr[1] = reinterpret_cast<uint4 *>(acc.f);
    A.nclr[1] = (nrec * prims->channels * (long long)sizeof(double) + 15) / 16;
    A.clear = 1;
  } else if (bwd_workspace) {
    const long long nrec = (long long)n_views * prims->n;
    const AccLayout acc = acc_layout(bwd_workspace, nrec, prims->channels);
    A.clr[0] = reinterpret_cast<uint4 *>(acc.g);        // fp32 rows of 5 + C values (16-byte multiples)
    A.nclr[0] = nrec * sph_row_stride(prims->channels) * (long long)sizeof(float) / 16;
    A.clr[1] = reinterpret_cast<uint4 *>(acc.kslot);    // intrinsic-gradient slots of every view
    A.nclr[1] = ((long long)n_views * SPLAT_K_SLOTS * 4 * (long long)sizeof(double) + 15) / 16;
    A.clr[2] = reinterpret_cast<uint4 *>(acc.cnt);      // recording-pixel counts
    A.nclr[2] = (nrec * (long long)sizeof(uint32_t) + 15) / 16;
    A.clear = 1;
  }
  return launch_render_fwd(vt, A, prims->kind, stream);
}

int splat_render_bwd(const splat_camera *cams, int n_views, int view_begin, int view_count, const splat_prims *prims,
                     const splat_params *prm, const void *proj, const uint32_t *vals, const uint32_t *tile_ranges,
                     const int32_t *overflow, const float *img, const float *T_final, const uint32_t *last,
                     const float *norm, const int32_t *topk, const float *dL_dimg, const splat_grads *grads,
                     void *workspace, size_t ws_bytes, hipStream_t stream) {
  ViewTable vt;
  int st = build_views(cams, n_views, prims ? prims->channels : 0, &vt);
  if (st) return st;
  if ((st = check_prims(prims, vt))) return st;
  if ((st = check_params(prm, prims->kind))) return st;
  CHECK(view_begin >= 0 && view_count >= 1 && view_begin + view_count <= n_views, SPLAT_ERR_INVALID_ARG,
        "view range");
  CHECK(grads != nullptr, SPLAT_ERR_INVALID_ARG, "grads is NULL");
  CHECK(prims->n > 0, SPLAT_ERR_INVALID_ARG, "backward needs at least one primitive");
  CHECK(proj && vals && tile_ranges && overflow && dL_dimg, SPLAT_ERR_INVALID_ARG, "NULL input");
  if (prims->kind == SPLAT_PRIM_SPHERE) {
    CHECK(img && norm && topk, SPLAT_ERR_INVALID_ARG, "sphere backward needs img, norm and topk");
    CHECK(!prm->max_shift || T_final, SPLAT_ERR_INVALID_ARG, "max-shifted backward needs T_final (the shifts)");
  } else {
    CHECK(T_final && last, SPLAT_ERR_INVALID_ARG, "Gaussian backward needs T_final and last");
    CHECK(grads->cam_K == nullptr, SPLAT_ERR_UNSUPPORTED, "intrinsic gradients are for spheres only");
    CHECK(!grads->normalize, SPLAT_ERR_UNSUPPORTED, "gradient normalisation is for spheres only");
  }
  CHECK(grads->atomic_direct_max >= 0, SPLAT_ERR_INVALID_ARG, "atomic_direct_max must be >= 0");
  CHECK(workspace != nullptr, SPLAT_ERR_INVALID_ARG, "NULL workspace");
  CHECK(ws_bytes >= bwd_workspace_bytes((long long)n_views * prims->n, prims->channels), SPLAT_ERR_CAPACITY,
        "backward workspace too small");
  BwdArgs A;
  memset(&A, 0, sizeof(A));
  A.n = prims->n; A.C = prims->channels; A.top_k = prm->top_k;
  A.alpha_min = prm->alpha_min; A.alpha_max = prm->alpha_max; A.gamma = prm->gamma;
  A.igamma = (float)(1.0 / (double)prm->gamma);
  A.max_shift = prims->kind == SPLAT_PRIM_SPHERE ? prm->max_shift : 0;
  A.serial_views = prm->serial_views;
  ProjLayout L = proj_layout(const_cast<void *>(proj), (long long)n_views * prims->n);
  A.draw = L.draw; A.aux = L.aux; A.vals = vals; A.ranges = tile_ranges; A.overflow = overflow;
  A.feat = prims->feat; A.img = img; A.T_final = T_final; A.last = last; A.norm = norm; A.topk = topk;
  A.dimg = dL_dimg;
  AccLayout acc = acc_layout(workspace, (long long)n_views * prims->n, prims->channels);
  A.accg = acc.g;
  A.accf = acc.f;
  A.accs = reinterpret_cast<float *>(acc.g);
  A.rs = sph_row_stride(prims->channels);
  A.cam_part = acc.cam;
  A.kslot = grads->cam_K ? acc.kslot : nullptr;
  A.cnt = grads->normalize ? acc.cnt : nullptr;
  A.direct_max = prims->kind == SPLAT_PRIM_SPHERE ? grads->atomic_direct_max : 0;
  return launch_render_bwd(vt, view_begin, view_begin + view_count, A, prims, L.bin, grads, stream);
}

int splat_interpolate(const float *key_times, int n_keys, float t, int n, const float *key_pos,
                      const float *key_rot, float *pos, float *rot, hipStream_t stream) {
  int k = 0, k1 = 0;
  float w = 0.0f;
  int st = key_bracket(key_times, n_keys, t, &k, &k1, &w);
  if (st) return st;
  CHECK(n >= 0, SPLAT_ERR_INVALID_ARG, "negative n");
  const bool do_pos = key_pos && pos, do_rot = key_rot && rot;
  CHECK(do_pos || do_rot || n == 0, SPLAT_ERR_INVALID_ARG, "nothing to assemble");
  CHECK(!do_rot || (aligned16(key_rot) && aligned16(rot)), SPLAT_ERR_INVALID_ARG, "rotation buffers not 16-byte aligned");
  return launch_assemble(do_pos ? key_pos : nullptr, do_rot ? key_rot : nullptr, k, k1, w, n, pos, rot, stream);
}

int splat_interpolate_bwd(const float *key_times, int n_keys, float t, int n, const float *key_rot,
                          const float *d_pos, const float *d_rot, float *d_key_pos, float *d_key_rot,
                          hipStream_t stream) {
  int k = 0, k1 = 0;
  float w = 0.0f;
  int st = key_bracket(key_times, n_keys, t, &k, &k1, &w);
  if (st) return st;
  CHECK(n >= 0, SPLAT_ERR_INVALID_ARG, "negative n");
  const bool do_pos = d_pos && d_key_pos, do_rot = d_rot && d_key_rot;
  if (do_rot) {
    CHECK(k == k1 || key_rot != nullptr, SPLAT_ERR_INVALID_ARG, "key_rot needed for the rotation gradient");
    CHECK(aligned16(d_rot) && aligned16(d_key_rot) && (!key_rot || aligned16(key_rot)), SPLAT_ERR_INVALID_ARG,
          "rotation buffers not 16-byte aligned");
  }
  return launch_assemble_bwd(key_rot, k, k1, w, n, do_pos ? d_pos : nullptr, do_rot ? d_rot : nullptr,
                             do_pos ? d_key_pos : nullptr, do_rot ? d_key_rot : nullptr, stream);
}

const char *splat_status_string(int status) {
  switch (status) {
    case SPLAT_OK: return "ok";
    case SPLAT_ERR_INVALID_ARG: return "invalid argument";
    case SPLAT_ERR_CAPACITY: return "buffer or workspace too small";
    case SPLAT_ERR_HIP: return "HIP launch error";
    case SPLAT_ERR_UNSUPPORTED: return "unsupported combination";
  }
  return "unknown status";
}

}  // extern "C"
