// Per-pixel arithmetic shared by the forward and backward compositors. Both
// passes evaluate the same inline functions on the same staged values, so the
// backward takes exactly the decisions the forward took (skip, stop, top-K).
#pragma once
#include "splat_internal.h"

#define SPLAT_TOPK_MAX 8

struct FwdArgs {
  int n, C, top_k;
  float alpha_min, alpha_max, T_min, tau, bg_weight;
  const DrawRec *draw;
  const AuxRec *aux;
  const uint32_t *vals;
  const uint32_t *ranges;
  const int32_t *overflow;
  const float *feat;
  float *img;
  float *T_final;
  uint32_t *last;
  float *norm;
  int32_t *topk;
  float bg[SPLAT_MAX_CHANNELS];
};

struct BwdArgs {
  int n, C, top_k;
  float alpha_min, alpha_max, gamma;
  const DrawRec *draw;
  const AuxRec *aux;
  const uint32_t *vals;
  const uint32_t *ranges;
  const int32_t *overflow;
  const float *feat;
  const float *img;
  const float *T_final;
  const uint32_t *last;
  const float *norm;
  const int32_t *topk;
  const float *dimg;
  double *accg;           // [records][ACC_G]
  float *accf;            // [records][C]
};

struct TilePix {
  int i, j;
  bool inside;
  float x0, y0;      // tile origin (pixels)
  float pxr, pyr;    // pixel centre relative to the tile origin
};

// Thread tid of a tile's workgroup owns pixel (tid % 16, tid / 16); a wave64
// covers four rows of the tile.
__device__ __forceinline__ TilePix tile_pixel(const ViewDev &c, int gtile, unsigned tid) {
  const int lt = gtile - c.tile_off;
  const int ty = lt / c.TW, tx = lt - ty * c.TW;
  const int li = (int)(tid & 15u), lj = (int)(tid >> 4);
  TilePix t;
  t.i = tx * TILE + li;
  t.j = ty * TILE + lj;
  t.inside = t.i < c.W && t.j < c.H;
  t.x0 = (float)(tx * TILE);
  t.y0 = (float)(ty * TILE);
  t.pxr = (float)li + 0.5f;
  t.pyr = (float)lj + 0.5f;
  return t;
}

__device__ __forceinline__ int channel_bucket_dev(int C) { return C; }

static inline int channel_bucket(int C) {
  if (C <= 1) return 1;
  if (C <= 2) return 2;
  if (C <= 3) return 3;
  if (C <= 4) return 4;
  if (C <= 8) return 8;
  if (C <= 16) return 16;
  if (C <= 32) return 32;
  return 64;
}

// ---------------------------------------------------------------------------
// Spheres: orthogonal distance from the sphere centre q to the pixel ray d.
// With a = q / qz and delta = d - a = (sx, sy, 0) (both in normalised image
// coordinates), |q x d|^2 = qz^2 (sx^2 + sy^2 + (ax sy - ay sx)^2), so
//   D = 1 - dist^2 / r^2 = 1 - (qz^2 / r^2) * g * s,  g = 1 / |d|^2,
// with no cancellation between large terms (delta comes straight from the
// tile-relative pixel offset).
//
// This runs in fp64: near a sphere's rim D is a small difference of numbers
// close to 1, and a dominant sphere's weight is proportional to D there. On
// CDNA4 an fp64 FMA issues at the same per-lane rate as a non-packed fp32 FMA,
// so exact geometry costs register space, not issue slots.
// ---------------------------------------------------------------------------
struct SphereRay {
  double ifx, ify;
  double dx, dy;     // normalised ray direction (dx, dy, 1)
  double g;          // 1 / (1 + dx^2 + dy^2)
  double pxr, pyr;   // tile-relative pixel centre
};

__device__ __forceinline__ SphereRay sphere_ray(const ViewDev &c, const TilePix &tp) {
  SphereRay r;
  r.ifx = 1.0 / (double)c.fx;
  r.ify = 1.0 / (double)c.fy;
  r.dx = ((double)tp.i + 0.5 - (double)c.cx) * r.ifx;
  r.dy = ((double)tp.j + 0.5 - (double)c.cy) * r.ify;
  r.g = 1.0 / (1.0 + r.dx * r.dx + r.dy * r.dy);
  r.pxr = (double)tp.pxr;
  r.pyr = (double)tp.pyr;
  return r;
}

// Staged sphere geometry: tile-relative centre, normalised centre, A.
struct SphereGeo {
  double u, v, ax, ay, A;
};

__device__ __forceinline__ SphereGeo sphere_geo(const ViewDev &c, const TilePix &tp, const DrawRec &d) {
  SphereGeo s;
  s.u = d.u - (double)tp.x0;
  s.v = d.v - (double)tp.y0;
  s.ax = (d.u - (double)c.cx) / (double)c.fx;
  s.ay = (d.v - (double)c.cy) / (double)c.fy;
  s.A = d.a;
  return s;
}

// Returns D = 1 - dist^2 / r_eff^2; sx, sy receive the normalised offsets.
__device__ __forceinline__ double sphere_D_ex(const SphereRay &ray, double u, double v, double ax, double ay,
                                              double A, double &sx, double &sy) {
  sx = (ray.pxr - u) * ray.ifx;
  sy = (ray.pyr - v) * ray.ify;
  const double cr = __builtin_fma(ax, sy, -(ay * sx));
  const double s = __builtin_fma(sx, sx, __builtin_fma(sy, sy, cr * cr));
  return __builtin_fma(-(A * ray.g), s, 1.0);
}

// ---------------------------------------------------------------------------
// Gaussians.
// ---------------------------------------------------------------------------
// Tile-relative centre in fp64; for spherical views the horizontal part is
// wrapped to the full turn nearest the tile.
__device__ __forceinline__ double2 stage_uv(const ViewDev &c, const TilePix &tp, const DrawRec &d, bool lidar) {
  double t = d.u - (double)tp.x0;
  if (lidar) {
    const double half = 0.5 * (double)c.W;
    if (t - 8.0 >= half) t -= (double)c.W;
    else if (t - 8.0 < -half) t += (double)c.W;
  }
  return make_double2(t, d.v - (double)tp.y0);
}

// Staged conic: (a/2, b) and (c/2, opacity) with power = (a dx^2 + 2 b dx dy + c dy^2) / 2.
struct Conic {
  double2 ab;
  double2 co;
};

__device__ __forceinline__ Conic stage_conic(const DrawRec &d) {
  Conic k;
  k.ab = make_double2(0.5 * d.a, d.b);
  k.co = make_double2(0.5 * d.c, (double)d.w);
  return k;
}

// alpha = min(amax, o exp(-power)). The offsets and the quadratic form are fp64 (an
// elongated footprint makes the three terms cancel); exp runs in fp32.
template <bool LIDAR>
__device__ __forceinline__ float splat_alpha(const ViewDev &c, double pxr, double pyr, const double2 uv,
                                             const double2 ab, const double2 co, float amax, float &G, float &og,
                                             double &dx, double &dy) {
  dx = pxr - uv.x;
  dy = pyr - uv.y;
  if (LIDAR) {
    const double half = 0.5 * (double)c.W;
    if (dx >= half) dx -= (double)c.W;
    else if (dx < -half) dx += (double)c.W;
  }
  const double power = __builtin_fma(dx, __builtin_fma(ab.x, dx, ab.y * dy), (co.x * dy) * dy);
  G = __expf(-(float)power);
  og = (float)co.y * G;
  return fminf(amax, og);
}
