// Internal definitions shared by the libsplat HIP sources (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splat.h"

#define TILE 16
#define TILE_PIX 256
#define WAVE 64

// ---------------------------------------------------------------------------
// View table, passed by value to every kernel (fits the kernel-argument block).
// ---------------------------------------------------------------------------
struct ViewDev {
  int kind, W, H, TW, TH;
  int tile_off;         // first global tile of the view
  int chan;             // image channels of the view (C, or 2 for spherical)
  int pad0;
  long long pix_off;    // first pixel of the view in per-pixel buffers
  long long img_off;    // first float of the view in the image buffer
  float R[9], t[3];
  float fx, fy, cx, cy;
  float el_min, el_max, znear, zfar;
  double ifx, ify;      // 1 / fx, 1 / fy (host, correctly rounded)
  double ispan;         // 1 / (zfar - znear) (host)
};

struct ViewTable {
  int n;
  int total_tiles;
  long long total_pix;
  ViewDev v[SPLAT_MAX_VIEWS];
};

__device__ __forceinline__ int view_of_tile(const ViewTable &vt, int gtile) {
  int v = 0;
#pragma unroll 1
  while (v + 1 < vt.n && vt.v[v + 1].tile_off <= gtile) v++;
  return v;
}

// ---------------------------------------------------------------------------
// Projected records (structure of arrays inside the opaque proj buffer).
// ---------------------------------------------------------------------------
// Binning part, read by the counting and bucketing kernels: two arrays, so that
// the counting reads the 8-byte tile rectangles alone.
struct BinRec {          // a record's binning fields, in registers
  uint32_t key;          // fp32 bits of the depth key
  uint16_t tx0, ntx;     // tile columns tx0 .. tx0+ntx-1 (mod TW for spherical views)
  uint16_t ty0, ty1;     // tile rows (inclusive)
};

struct BinArrays {
  uint32_t *key;         // [records] depth keys
  uint2 *rect;           // [records] (tx0 | ntx << 16, ty0 | ty1 << 16)
};

__host__ __device__ inline uint2 pack_rect(const BinRec &b) {
  return make_uint2((uint32_t)b.tx0 | ((uint32_t)b.ntx << 16), (uint32_t)b.ty0 | ((uint32_t)b.ty1 << 16));
}

// Record k's rectangle (key 0) or its rectangle and key.
__device__ inline BinRec bin_rect(const BinArrays &b, long long k) {
  const uint2 r = b.rect[k];
  BinRec o;
  o.key = 0u;
  o.tx0 = (uint16_t)(r.x & 0xffffu);
  o.ntx = (uint16_t)(r.x >> 16);
  o.ty0 = (uint16_t)(r.y & 0xffffu);
  o.ty1 = (uint16_t)(r.y >> 16);
  return o;
}

__device__ inline BinRec bin_full(const BinArrays &b, long long k) {
  BinRec o = bin_rect(b, k);
  o.key = b.key[k];
  return o;
}

// Compositing part, staged into LDS by the render kernels (48 bytes).
//  Gaussians: projected mean (u, v), conic (a, b, c) with power = (a dx^2 + 2 b dx dy + c dy^2)/2,
//             w = opacity, e unused.
//  Spheres:   (u, v) = normalised centre (qx/qz, qy/qz), a = A = qz^2 / r_eff^2,
//             (b, c) = the features as four fp32 (up to SPLAT_REC_FEAT channels, zero
//             padded; more channels: projected centre in pixels), w = o exp(o zhat / gamma),
//             e = stop bound.
// Positions and the quadratic form stay fp64: an elongated footprint makes the three
// conic terms cancel by the covariance's condition number, and per-pixel offsets from
// a far tile need the full mantissa.
// (i0..i1) x (j0..j1) is the inclusive pixel rectangle outside which the primitive
// cannot contribute (Gaussians: opacity-aware alpha support; spheres: tangent box);
// the compositors use it to give each wave of a tile only the entries that reach
// its quadrant.
constexpr int SPLAT_REC_FEAT = 4;   // sphere features carried in the draw record up to this many channels

struct __align__(16) DrawRec {
  double u, v;
  double a, b, c;
  float w, e;
  int i0, i1, j0, j1;
};

// Backward-only part.
//  Gaussians: depth (range for spherical views) in z; rest unused.
//  Spheres:   sensor-frame depth qz in z, r_eff in w, opacity, flags (bit0 floored,
//             bit1 gated); the normalised device depth (zfar - qz) / (zfar - znear) is
//             formed again where it is needed.
struct __align__(16) AuxRec {
  float z, w, opac, flags;
};

// Sphere feature ch kept in a draw record (channels <= SPLAT_REC_FEAT).
__device__ __forceinline__ float rec_feat(const DrawRec &d, int ch) {
  const float2 f = __builtin_bit_cast(float2, ch < 2 ? d.b : d.c);
  return (ch & 1) ? f.y : f.x;
}

struct ProjLayout {
  BinArrays bin;
  DrawRec *draw;
  AuxRec *aux;
};

static inline size_t proj_align(size_t x) { return (x + 255) & ~(size_t)255; }

static inline ProjLayout proj_layout(void *base, long long nrec) {
  char *p = (char *)base;
  ProjLayout L;
  L.bin.key = (uint32_t *)p;
  p += proj_align(sizeof(uint32_t) * (size_t)nrec);
  L.bin.rect = (uint2 *)p;
  p += proj_align(sizeof(uint2) * (size_t)nrec);
  L.draw = (DrawRec *)p;
  p += proj_align(sizeof(DrawRec) * (size_t)nrec);
  L.aux = (AuxRec *)p;
  return L;
}

static inline size_t proj_bytes(long long nrec) {
  return proj_align(sizeof(uint32_t) * (size_t)nrec) + proj_align(sizeof(uint2) * (size_t)nrec) +
         proj_align(sizeof(DrawRec) * (size_t)nrec) +
         proj_align(sizeof(AuxRec) * (size_t)nrec);
}

// Per-record gradient accumulators in the backward workspace, fp64:
//  Gaussians, two arrays: [records][ACC_G] = [du, dv, d_ca, d_cb, d_cc, d_opac,
//    d_depth, -] and [records][channels] features;
//  spheres, one array: [records][5 + channels] = [dq0, dq1, dq2, d_reff, d_opac,
//    d_feat...] (one row of 64 bytes at three channels).
// The geometric sums feed an ill-conditioned chain (conic -> covariance ->
// rotation), so they are formed and summed in double precision. Every value
// takes one global atomic add per (tile, record): a primitive that covers the
// whole frame receives thousands of per-tile partial sums, too many for a
// single-precision running sum. The workspace is sized for the Gaussian layout,
// which is the larger.
#define ACC_G 8

// After the accumulators: per-block camera partial sums of the sphere gradient
// pass ([SPLAT_CAM_BLOCKS][12] fp64).
#define SPLAT_CAM_BLOCKS 1024
// Then the intrinsic-gradient slots of the sphere reverse pass: per view,
// SPLAT_K_SLOTS rows of (fx, fy, cx, cy) fp64 sums; compositor block b adds
// into row b mod SPLAT_K_SLOTS, so that few blocks share an address.
#define SPLAT_K_SLOTS 256

// Last, per record, the number of pixels that recorded it (gradient
// normalisation of spheres).
struct AccLayout {
  double *g;
  double *f;
  double *cam;
  double *kslot;
  uint32_t *cnt;
};

// Sphere reverse-pass rows: fp32 [records][sph_row_stride(C)], the 5 + C values
// (dq0, dq1, dq2, d_reff, d_opac, d_feat...) padded to a multiple of four floats
// so that every row starts on a 16-byte boundary (they use the region of the
// Gaussians' geometric and feature sums).
__host__ __device__ static inline int sph_row_stride(int C) { return (5 + C + 3) & ~3; }

static inline size_t acc_bytes(long long nrec, int C) {
  return proj_align(sizeof(double) * ACC_G * (size_t)nrec) + proj_align(sizeof(double) * (size_t)nrec * C) +
         proj_align(sizeof(double) * 12 * SPLAT_CAM_BLOCKS) +
         proj_align(sizeof(double) * 4 * SPLAT_K_SLOTS * SPLAT_MAX_VIEWS) +
         proj_align(sizeof(uint32_t) * (size_t)nrec);
}

static inline AccLayout acc_layout(void *base, long long nrec, int C) {
  AccLayout a;
  char *p = (char *)base;
  a.g = (double *)p;    p += proj_align(sizeof(double) * ACC_G * (size_t)nrec);
  a.f = (double *)p;    p += proj_align(sizeof(double) * (size_t)nrec * C);
  a.cam = (double *)p;  p += proj_align(sizeof(double) * 12 * SPLAT_CAM_BLOCKS);
  a.kslot = (double *)p; p += proj_align(sizeof(double) * 4 * SPLAT_K_SLOTS * SPLAT_MAX_VIEWS);
  a.cnt = (uint32_t *)p;
  return a;
}

// ---------------------------------------------------------------------------
// Wave64 helpers.
// ---------------------------------------------------------------------------
// Inclusive prefix sum across the wave with DPP row shifts and row broadcasts;
// lane 63 ends up holding the wave total.
__device__ __forceinline__ float wave_sum_to_last(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));  // row_shr:1
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));  // row_shr:2
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));  // row_shr:4
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));  // row_shr:8
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false)); // row_bcast:15
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false)); // row_bcast:31
  return x;
}

// Wave total, uniform across lanes.
__device__ __forceinline__ float wave_sum(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_to_last(x)), 63));
}

// DPP move of a double (two 32-bit halves).
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __builtin_bit_cast(long long, x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), CTRL, ROWS, 0xf, BOUND);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xf, BOUND);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (long long)(unsigned)lo);
}

// fp64 sum within each 16-lane row; lanes 15, 31, 47, 63 hold the row sums.
__device__ __forceinline__ double row_sum_to_last_f64(double x) {
  x += dpp_f64<0x111, 0xf, true>(x);
  x += dpp_f64<0x112, 0xf, true>(x);
  x += dpp_f64<0x114, 0xf, true>(x);
  x += dpp_f64<0x118, 0xf, true>(x);
  return x;
}

// fp64 wave total, uniform across lanes.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x = row_sum_to_last_f64(x);
  x += dpp_f64<0x142, 0xa, false>(x);   // row_bcast:15
  x += dpp_f64<0x143, 0xc, false>(x);   // row_bcast:31
  const long long b = __builtin_bit_cast(long long, x);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), 63);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
  return __builtin_bit_cast(double, ((long long)hi << 32) | (long long)(unsigned)lo);
}

__device__ __forceinline__ unsigned lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ __forceinline__ uint64_t ballot64(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// HIP error check used by the host-side launchers.
// A second stream per device on which the pinhole-view compositors run beside
// the spherical ones: a lidar tile list can be far longer than any camera
// tile's, and on one stream the camera views would wait for it.
// side_begin makes the side stream wait for `main` and holds the device's lock
// until side_end, which makes `main` wait for the side stream; every side_begin
// that returns SPLAT_OK is followed by side_end. The stream and its two events
// are created on first use and kept until the process ends.
int side_begin(hipStream_t main, hipStream_t *side);
int side_end(hipStream_t main, hipStream_t side);

#define SPLAT_LAUNCH_CHECK()                                   \
  do {                                                         \
    if (hipPeekAtLastError() != hipSuccess) {                  \
      (void)hipGetLastError();                                 \
      return SPLAT_ERR_HIP;                                    \
    }                                                          \
  } while (0)
