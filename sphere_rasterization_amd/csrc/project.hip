// Projection: one thread per (view, primitive); the grid's second dimension is
// the view, so a workgroup's camera is uniform (scalar loads).
//
// Pulsar appendix B.1.1 ("Step 0: enclosing rectangle"): a sphere-parallel pass
// that computes each primitive's screen rectangle and the data the draw step
// needs, kept in separate binning and drawing records. Gaussians use EWA
// splatting (covariance pushed through the Jacobian of the image mapping).
//
// Everything here runs in fp64: the work is per primitive, and double
// precision keeps the projected centre and the conic (or the sphere's
// normalised centre and A) exact enough for the per-pixel compositing.
// The expressions that decide integer outputs (pixel and tile ranges, depth
// key) are evaluated in a fixed operand order with contraction disabled
// (-ffp-contract=off), so any IEEE double implementation of the same
// expressions reaches the same integers.
#include "splat_internal.h"

namespace {

constexpr double kPi = 3.141592653589793;
// Gaussian footprint: alpha >= 1/255 with opacity <= 1 needs power <= ln 255, i.e.
// the ellipse Delta^T Sigma^-1 Delta <= 2 ln 255, whose bounding half-width is
// sqrt(2 ln 255 * Sigma_xx).
constexpr double kSupport = 11.082527090316852;  // 2 ln 255, correctly rounded

struct Rect {
  int valid;
  int tx0, ntx, ty0, ty1;
  int i0, i1, j0, j1;      // inclusive pixel range (columns unwrapped for spherical views)
};

__device__ Rect make_rect(const ViewDev &c, double xl, double xh, double yl, double yh) {
  Rect r = {0, 0, 0, 0, 0, 0, -1, 0, -1};
  double fx0 = ceil(xl - 0.5), fx1 = floor(xh - 0.5);
  double fy0 = ceil(yl - 0.5), fy1 = floor(yh - 0.5);
  if (fy0 < 0.0) fy0 = 0.0;
  if (fy1 > (double)(c.H - 1)) fy1 = (double)(c.H - 1);
  if (c.kind != SPLAT_CAM_SPHERICAL) {
    if (fx0 < 0.0) fx0 = 0.0;
    if (fx1 > (double)(c.W - 1)) fx1 = (double)(c.W - 1);
  } else if (fx1 - fx0 + 1.0 >= (double)c.W) {
    fx0 = 0.0;            // a full turn or more: every column once
    fx1 = (double)(c.W - 1);
  }
  if (!(fx0 <= fx1) || !(fy0 <= fy1)) return r;
  long long x0 = (long long)fx0, x1 = (long long)fx1;
  int y0 = (int)fy0, y1 = (int)fy1;
  r.i0 = (int)x0; r.i1 = (int)x1; r.j0 = y0; r.j1 = y1;
  r.ty0 = y0 / TILE;
  r.ty1 = y1 / TILE;
  if (c.kind != SPLAT_CAM_SPHERICAL) {
    r.tx0 = (int)(x0 / TILE);
    r.ntx = (int)(x1 / TILE) - r.tx0 + 1;
  } else {
    long long a0 = x0 >= 0 ? x0 / TILE : -((-x0 + TILE - 1) / TILE);
    long long a1 = x1 >= 0 ? x1 / TILE : -((-x1 + TILE - 1) / TILE);
    long long nt = a1 - a0 + 1;
    if (nt > c.TW) nt = c.TW;
    long long m = a0 % c.TW;
    if (m < 0) m += c.TW;
    r.tx0 = (int)m;
    r.ntx = (int)nt;
  }
  r.valid = 1;
  return r;
}

__device__ __forceinline__ void sensor_point(const ViewDev &c, double x0, double x1, double x2, double m[3]) {
#pragma unroll
  for (int i = 0; i < 3; i++)
    m[i] = (double)c.R[3 * i + 0] * x0 + (double)c.R[3 * i + 1] * x1 + (double)c.R[3 * i + 2] * x2 + (double)c.t[i];
}

__device__ void write_culled(const ProjLayout &L, long long k, uint32_t *counts) {
  L.bin.key[k] = 0u;
  L.bin.rect[k] = make_uint2(0u, 0u);
  counts[k] = 0;
}

__device__ void write_rect(const ProjLayout &L, long long k, uint32_t *counts, const Rect &r, float key_depth) {
  BinRec b;
  b.key = __float_as_uint(key_depth);
  b.tx0 = (uint16_t)r.tx0; b.ntx = (uint16_t)r.ntx;
  b.ty0 = (uint16_t)r.ty0; b.ty1 = (uint16_t)r.ty1;
  L.bin.key[k] = b.key;
  L.bin.rect[k] = pack_rect(b);
  counts[k] = (uint32_t)(r.ntx * (r.ty1 - r.ty0 + 1));
}

struct PrimArgs {
  int kind, n, C;
  const float *pos, *scale, *rot, *opacity, *depth, *feat;
  double gamma, alpha_min;
  int max_shift;      // spheres: draw records carry log-weights (see below)
};

// One (view, primitive): the binning record and pair count go straight to
// memory; the drawing and backward records into the workgroup's LDS slots dd
// and aa. Returns false for a culled primitive (slots untouched: nothing reads
// a culled record's drawing or backward data).
template <int KIND>
__device__ __forceinline__ bool project_one(const ViewDev &c, const PrimArgs &P, const ProjLayout &L, uint32_t *counts,
                                            long long k, int i, DrawRec &dd, AuxRec &aa) {
  double o;
  if (KIND != SPLAT_PRIM_SPHERE) o = (double)P.opacity[i];

  if (KIND == SPLAT_PRIM_SPHERE) {
    // all five inputs in flight together (the opacity would otherwise be
    // loaded after the culling tests, one memory latency later)
    float px = P.pos[3 * i], py = P.pos[3 * i + 1], pz = P.pos[3 * i + 2], pr = P.scale[i], po = P.opacity[i];
    asm volatile("" : "+v"(px), "+v"(py), "+v"(pz), "+v"(pr), "+v"(po));
    o = (double)po;
    double q[3];
    sensor_point(c, (double)px, (double)py, (double)pz, q);
    double r = (double)pr;
    double fx = (double)c.fx, fy = (double)c.fy;
    double fmin = fx < fy ? fx : fy;
    const bool orth = c.kind == SPLAT_CAM_ORTHOGRAPHIC;
    // every sphere keeps at least one pixel: a projected radius of 0.75 px
    double rfl = orth ? 0.75 / fmin : 0.75 * q[2] / fmin;
    double re = r >= rfl ? r : rfl;
    double zf = q[2] - re;
    if (!(zf > (double)c.znear) || !(zf > 0.0) || !isfinite(r) || !(r > 0.0)) { write_culled(L, k, counts); return false; }
    // beyond the far plane zhat < 0, where a lower opacity weighs more and the
    // stop bound exp(zhat(front) / gamma) no longer bounds the spheres behind
    // (Pulsar sec. 3.2, Figure 3): culled, tested on the fp32 key depth the
    // bound is formed from
    if (!((double)(float)zf < (double)c.zfar)) { write_culled(L, k, counts); return false; }
    double xl, xh, yl, yh;
    if (orth) {
      // parallel projection: the outline is the circle of radius r_eff
      xl = fx * (q[0] - re) + (double)c.cx;
      xh = fx * (q[0] + re) + (double)c.cx;
      yl = fy * (q[1] - re) + (double)c.cy;
      yh = fy * (q[1] + re) + (double)c.cy;
    } else {
      // tangent planes through the sensor origin
      double den = q[2] * q[2] - re * re;
      double sx = sqrt(q[0] * q[0] + q[2] * q[2] - re * re);
      double sy = sqrt(q[1] * q[1] + q[2] * q[2] - re * re);
      xl = fx * ((q[0] * q[2] - re * sx) / den) + (double)c.cx;
      xh = fx * ((q[0] * q[2] + re * sx) / den) + (double)c.cx;
      yl = fy * ((q[1] * q[2] - re * sy) / den) + (double)c.cy;
      yh = fy * ((q[1] * q[2] + re * sy) / den) + (double)c.cy;
    }
    if (!isfinite(xl) || !isfinite(xh) || !isfinite(yl) || !isfinite(yh)) { write_culled(L, k, counts); return false; }
    Rect rc = make_rect(c, xl, xh, yl, yh);
    if (!rc.valid) { write_culled(L, k, counts); return false; }
    float key = (float)zf;
    write_rect(L, k, counts, rc, key);
    double u = (orth ? fx * q[0] : fx * q[0] / q[2]) + (double)c.cx;
    double v = (orth ? fy * q[1] : fy * q[1] / q[2]) + (double)c.cy;
    double span = (double)c.zfar - (double)c.znear;
    double zhat = ((double)c.zfar - q[2]) / span;
    double e = exp(o * zhat / P.gamma);
    double bnd = exp((((double)c.zfar - (double)key) / span) / P.gamma);
    double area = orth ? kPi * (fx * r) * (fy * r) : kPi * (fx * r / q[2]) * (fy * r / q[2]);
    int floored = r < rfl, gated = !(area > 3.0);
    DrawRec d;
    // pinhole: normalised centre a = q / qz and A = qz^2 / r_eff^2;
    // orthographic: (qx, qy) and A = 1 / r_eff^2
    d.u = orth ? q[0] : q[0] / q[2];
    d.v = orth ? q[1] : q[1] / q[2];
    d.a = orth ? 1.0 / (re * re) : q[2] * q[2] / (re * re);
    if (P.C <= SPLAT_REC_FEAT) {
      // the features ride in the record: the compositors' staging then fetches one
      // record per list entry instead of the record and a separate feature row
      float f[SPLAT_REC_FEAT] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (P.feat)
#pragma unroll
        for (int ch = 0; ch < SPLAT_REC_FEAT; ch++)
          if (ch < P.C) f[ch] = P.feat[(size_t)i * P.C + ch];
      d.b = __builtin_bit_cast(double, make_float2(f[0], f[1]));
      d.c = __builtin_bit_cast(double, make_float2(f[2], f[3]));
    } else {
      d.b = u;                         // projected centre (pixels), informational
      d.c = v;
    }
    if (P.max_shift) {
      // logs: ln(o exp(o zhat / gamma)) and ln(bound); the compositors blend
      // relative to a per-pixel shift, so nothing overflows for small gamma
      d.w = (float)(log(o) + o * zhat / P.gamma);
      d.e = (float)((((double)c.zfar - (double)key) / span) / P.gamma);
    } else {
      d.w = (float)(o * e);
      d.e = (float)bnd;
    }
    d.i0 = rc.i0; d.i1 = rc.i1; d.j0 = rc.j0; d.j1 = rc.j1;
    dd = d;
    AuxRec a;
    a.z = (float)q[2]; a.w = (float)re;
    a.opac = (float)o;
    a.flags = (float)(floored | (gated << 1));
    aa = a;
    return true;
  }

  double u, v, sxx, sxy, syy, depth;
  if (KIND == SPLAT_PRIM_GAUSS2D) {
    u = (double)P.pos[2 * i];
    v = (double)P.pos[2 * i + 1];
    double s = (double)P.scale[i];
    sxx = s * s; syy = s * s; sxy = 0.0;
    depth = (double)P.depth[i];
  } else {
    double s0 = P.scale[3 * i], s1 = P.scale[3 * i + 1], s2 = P.scale[3 * i + 2];
    double qw = P.rot[4 * i], qx = P.rot[4 * i + 1], qy = P.rot[4 * i + 2], qz = P.rot[4 * i + 3];
    double nq = sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
    double w = qw / nq, x = qx / nq, y = qy / nq, z = qz / nq;
    double Rq[9];
    Rq[0] = 1.0 - 2.0 * (y * y + z * z);
    Rq[1] = 2.0 * (x * y - w * z);
    Rq[2] = 2.0 * (x * z + w * y);
    Rq[3] = 2.0 * (x * y + w * z);
    Rq[4] = 1.0 - 2.0 * (x * x + z * z);
    Rq[5] = 2.0 * (y * z - w * x);
    Rq[6] = 2.0 * (x * z - w * y);
    Rq[7] = 2.0 * (y * z + w * x);
    Rq[8] = 1.0 - 2.0 * (x * x + y * y);
    double M[9];
#pragma unroll
    for (int a = 0; a < 3; a++) {
      M[3 * a + 0] = Rq[3 * a + 0] * s0;
      M[3 * a + 1] = Rq[3 * a + 1] * s1;
      M[3 * a + 2] = Rq[3 * a + 2] * s2;
    }
    double S3[9];
#pragma unroll
    for (int a = 0; a < 3; a++)
#pragma unroll
      for (int b = 0; b < 3; b++)
        S3[3 * a + b] = M[3 * a] * M[3 * b] + M[3 * a + 1] * M[3 * b + 1] + M[3 * a + 2] * M[3 * b + 2];
    double m[3];
    sensor_point(c, (double)P.pos[3 * i], (double)P.pos[3 * i + 1], (double)P.pos[3 * i + 2], m);
    double J[6];
    if (c.kind == SPLAT_CAM_PINHOLE) {
      if (!(m[2] > (double)c.znear)) { write_culled(L, k, counts); return false; }
      depth = m[2];
      double fx = c.fx, fy = c.fy;
      J[0] = fx / m[2];
      J[1] = 0.0;
      J[2] = -(fx * m[0]) / (m[2] * m[2]);
      J[3] = 0.0;
      J[4] = fy / m[2];
      J[5] = -(fy * m[1]) / (m[2] * m[2]);
      u = fx * m[0] / m[2] + (double)c.cx;
      v = fy * m[1] / m[2] + (double)c.cy;
    } else {
      double rho2 = m[0] * m[0] + m[1] * m[1];
      double rr = sqrt(rho2 + m[2] * m[2]);
      if (!(rr > (double)c.znear) || !(rho2 > 0.0)) { write_culled(L, k, counts); return false; }
      depth = rr;
      double rho = sqrt(rho2);
      double r2 = rho2 + m[2] * m[2];
      double th_max = (double)c.el_max * (kPi / 180.0), th_min = (double)c.el_min * (kPi / 180.0);
      double ka = (double)c.W / (2.0 * kPi);
      double kb = (double)c.H / (th_max - th_min);
      J[0] = ka * m[1] / rho2;
      J[1] = -(ka * m[0]) / rho2;
      J[2] = 0.0;
      J[3] = kb * m[0] * m[2] / (r2 * rho);
      J[4] = kb * m[1] * m[2] / (r2 * rho);
      J[5] = -(kb * rho) / r2;
      u = (kPi - atan2(m[1], m[0])) * ka;
      v = (th_max - atan2(m[2], rho)) * kb;
    }
    double T[6], U[6];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 3; b++)
        T[3 * a + b] = J[3 * a] * (double)c.R[b] + J[3 * a + 1] * (double)c.R[3 + b] + J[3 * a + 2] * (double)c.R[6 + b];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
      for (int b = 0; b < 3; b++)
        U[3 * a + b] = T[3 * a] * S3[b] + T[3 * a + 1] * S3[3 + b] + T[3 * a + 2] * S3[6 + b];
    sxx = U[0] * T[0] + U[1] * T[1] + U[2] * T[2];
    sxy = U[0] * T[3] + U[1] * T[4] + U[2] * T[5];
    syy = U[3] * T[3] + U[4] * T[4] + U[5] * T[5];
  }
  double det = sxx * syy - sxy * sxy;
  if (!(det > 0.0) || !(depth > 0.0) || !isfinite(u) || !isfinite(v)) { write_culled(L, k, counts); return false; }
  double hx = sqrt(kSupport * sxx), hy = sqrt(kSupport * syy);
  if (!isfinite(hx) || !isfinite(hy)) { write_culled(L, k, counts); return false; }
  Rect rc = make_rect(c, u - hx, u + hx, v - hy, v + hy);
  if (!rc.valid) { write_culled(L, k, counts); return false; }
  write_rect(L, k, counts, rc, (float)depth);
  DrawRec d;
  d.u = u;
  d.v = v;
  d.a = syy / det;
  d.b = -sxy / det;
  d.c = sxx / det;
  d.w = (float)o;
  d.e = 0.0f;
  // Pixels that can reach alpha >= alpha_min: power <= ln(o / alpha_min); the
  // threshold is inflated by 1e-4 to cover fp32 rounding of alpha.
  d.i0 = 0; d.i1 = -1; d.j0 = 0; d.j1 = -1;
  const double lim = log(o / P.alpha_min) + 1e-4;
  if (lim > 0.0) {
    if (c.kind == SPLAT_CAM_SPHERICAL) {
      d.i0 = -(1 << 30); d.i1 = 1 << 30;     // columns wrap: every quadrant
      d.j0 = rc.j0; d.j1 = rc.j1;
    } else {
      const double ax = sqrt(2.0 * lim * sxx), ay = sqrt(2.0 * lim * syy);
      const Rect dr = make_rect(c, u - ax, u + ax, v - ay, v + ay);
      if (dr.valid) { d.i0 = dr.i0; d.i1 = dr.i1; d.j0 = dr.j0; d.j1 = dr.j1; }
    }
  }
  dd = d;
  AuxRec a;
  a.z = (float)depth; a.w = 0.f;
  a.opac = (float)o; a.flags = 0.f;
  aa = a;
  return true;
}

// Thread per (view, primitive); grid (ceil(n / 256), views). The drawing records
// (64 B) are staged in LDS and leave as whole contiguous blocks: stored from
// registers, each lane's 16-byte pieces would land 64 bytes apart and the
// partial-line writes run at half the write bandwidth. The backward records
// (16 B) are contiguous across the lanes already and are stored directly.
template <int KIND>
__global__ __launch_bounds__(256) void k_project(ViewTable vt, PrimArgs P, ProjLayout L, uint32_t *counts) {
  __shared__ DrawRec s_d[256];
  __shared__ unsigned char s_vis[256];
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int view = blockIdx.y;
  const ViewDev &c = vt.v[view];
  bool vis = false;
  const long long k = (long long)view * P.n + i;
  if (i < P.n) {
    AuxRec a;
    vis = project_one<KIND>(c, P, L, counts, k, i, s_d[threadIdx.x], a);
    if (vis) L.aux[k] = a;
  }
  s_vis[threadIdx.x] = vis ? 1 : 0;
  __syncthreads();
  // only visible records' pieces are stored (a view may cull most of the scene)
  const int nblk = min((int)blockDim.x, P.n - (int)(blockIdx.x * blockDim.x));
  const long long k0 = (long long)view * P.n + (long long)blockIdx.x * blockDim.x;
  constexpr int DW = sizeof(DrawRec) / 16;
  uint4 *gd = reinterpret_cast<uint4 *>(L.draw + k0);
  const uint4 *sd = reinterpret_cast<const uint4 *>(s_d);
  for (int j = threadIdx.x; j < nblk * DW; j += blockDim.x)
    if (s_vis[j / DW]) gd[j] = sd[j];
}

}  // namespace

int launch_project(const ViewTable &vt, const splat_prims *pr, double gamma, double alpha_min, int max_shift,
                   void *proj, uint32_t *counts, hipStream_t stream) {
  long long nrec = (long long)vt.n * pr->n;
  if (nrec == 0) return SPLAT_OK;
  PrimArgs P;
  P.kind = pr->kind; P.n = pr->n;
  P.pos = pr->pos; P.scale = pr->scale; P.rot = pr->rot; P.opacity = pr->opacity; P.depth = pr->depth;
  P.gamma = gamma;
  P.alpha_min = alpha_min;
  P.max_shift = max_shift;
  P.C = pr->channels;
  P.feat = pr->feat;
  ProjLayout L = proj_layout(proj, nrec);
  const dim3 grid((unsigned)((pr->n + 255) / 256), (unsigned)vt.n);
  if (pr->kind == SPLAT_PRIM_SPHERE)
    hipLaunchKernelGGL(k_project<SPLAT_PRIM_SPHERE>, grid, dim3(256), 0, stream, vt, P, L, counts);
  else if (pr->kind == SPLAT_PRIM_GAUSS2D)
    hipLaunchKernelGGL(k_project<SPLAT_PRIM_GAUSS2D>, grid, dim3(256), 0, stream, vt, P, L, counts);
  else
    hipLaunchKernelGGL(k_project<SPLAT_PRIM_GAUSS3D>, grid, dim3(256), 0, stream, vt, P, L, counts);
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}
