/*
 * CPU oracle for the tile rasterizer of point primitives.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code with the HIP kernels.
 *
 * Plain, slow, double precision. It follows the method step by step:
 *   project every primitive            (Pulsar, sec. B.1.1 "Step 0: enclosing
 *                                        rectangle"; EWA splatting for Gaussians)
 *   bin to 16x16 tiles and sort each    (Pulsar, sec. B.1.1 depth sort and
 *   tile's list by depth                 sec. B.1.2 16x16 blocks)
 *   composite per pixel front to back   (Pulsar sec. 3.2 and B.1.3 for spheres;
 *                                        alpha blending for Gaussian splats)
 *   reverse-mode gradients per pixel,   (Pulsar sec. B.2; NuRec page,
 *   then chain rule per primitive        "renderBackward")
 * The exact formulas are readings of the pages (they print none); each one is
 * listed with its reading in the design notes of the repository.
 *
 * Integer outputs (pixel rectangles, tile lists, sort keys) come from the same
 * double-precision expressions the GPU evaluates, written in the same operand
 * order with no contraction (build with -ffp-contract=off), so that both sides
 * take the binning decisions identically.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { PRIM_GAUSS2D = 0, PRIM_GAUSS3D = 1, PRIM_SPHERE = 2 };
enum { CAM_PINHOLE = 0, CAM_SPHERICAL = 1, CAM_ORTHO = 2 };

/* Near ties: decisions that an fp32 evaluation of the same step may take the
 * other way. The windows are the rounding error of such an evaluation (single
 * precision alpha from an fp32 exponential, transmittance carried in double,
 * the sphere normalisation summed in single precision in list order), with a
 * margin of about two:
 *   EPS_ALPHA   relative error of alpha = o exp(-power) with power rounded to
 *               fp32 (|power| <= ln 255 where alpha can reach the threshold: 3.3e-7),
 *               the exponential through exp2 of an fp32 product (3.3e-7 plus a
 *               couple of ulps) and the product with o (6e-8): 8.5e-7 in all;
 *   T           after entry k relative error EPS_ALPHA * sum over the unclamped
 *               composited entries j <= k of alpha_j / (1 - alpha_j);
 *   sphere N    relative error u * (sum over hits of N after the hit + 3 w) / N,
 *               u = 2^-24 (sequential fp32 sum of fp32 products), plus one
 *               rounding of the bound and one of its division by tau.
 * A pixel's flags say which kinds of tie it met. */
enum {
  FLAG_ALPHA_MIN = 1,   /* an alpha within EPS_ALPHA (relative) of the skip threshold */
  FLAG_T_STOP = 2,      /* transmittance within its error bound of the stop threshold */
  FLAG_CLAMP = 4,       /* opacity*G within EPS_ALPHA (relative) of the clamp */
  FLAG_SPH_EDGE = 8,    /* a sphere's distance factor within 1e-8 of 0 (top-K may flip) */
  FLAG_SPH_STOP = 16,   /* a stop bound within the error bound of tau*N */
  FLAG_SPH_ZTIE = 32,   /* closest-K by depth: K-th and next intersection depth within 2e-6 (relative) */
  FLAG_UNRESOLVED = 64  /* more near ties along one outcome than the alternatives enumerate */
};
#define EPS_ALPHA 1.5e-6
#define U32 (1.0 / 16777216.0)
/* near-tie decisions whose both outcomes the alternatives enumerate */
#define MAX_TIES 3

#define CAM_STRIDE 24
#define TILE 16
/* support constant of the Gaussian footprint: 2 ln 255 (alpha >= 1/255 needs power <= ln 255) */
static double k_support(void) { return 2.0 * log(255.0); }

typedef struct {
  int kind, width, height, tiles_x, tiles_y;
  long long tile_off, pix_off;
  double R[9], t[3], fx, fy, cx, cy, el_min, el_max, znear, zfar;
} ocam;

typedef struct {
  int valid;
  long long x0, x1, y0, y1;     /* inclusive pixel range (x unclipped for spherical) */
  int tx0, ntx, ty0, ty1;       /* tile columns tx0..tx0+ntx-1 (mod tiles_x), rows ty0..ty1 */
  long long ntiles;
  float key_depth;
  double depth;                 /* m_z, range, given depth, or sphere front depth */
  double m[3];                  /* sensor-frame centre */
  double u, v;
  double sxx, sxy, syy;         /* 2D covariance */
  double ca, cb, cc;            /* conic */
  double opac;
  /* sphere */
  double r, r_eff, e, b, zhat;
  int floored, gated;
} orec;

typedef struct {
  int kind, n, C, V, K;
  int top_by_depth;             /* spheres: record the K closest intersections, not the first K */
  int max_shift;                /* spheres: report the normalisation relative to a per-pixel shift */
  double *pos, *scale, *rot, *opac, *depth, *feat;   /* inputs, promoted to double */
  double alpha_min, alpha_max, T_min, gamma, bg_weight, tau;
  double *bg;
  ocam *cams;
  long long total_tiles, total_pix;
  orec *rec;                    /* [V*n] */
  /* tile lists */
  long long npairs;
  long long *tile_start;        /* [total_tiles+1] */
  uint32_t *pair_id;            /* [npairs] record index v*n+i, sorted per tile */
  uint32_t *pair_bits;          /* [npairs] fp32 depth bits */
  int32_t *branch;              /* [total_pix] or NULL: per pixel, which near-tie decisions the
                                   backward flips (bit e: the e-th tie met along the way) */
} octx;

static int pdim(int kind) { return kind == PRIM_GAUSS2D ? 2 : 3; }
static int sdim(int kind) { return kind == PRIM_GAUSS3D ? 3 : 1; }

static double *dup_d(const double *a, long long count) {
  if (!a) return NULL;
  double *p = (double *)malloc(sizeof(double) * (size_t)(count > 0 ? count : 1));
  memcpy(p, a, sizeof(double) * (size_t)count);
  return p;
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ------------------------------------------------------------------------- */
/* Projection (Pulsar sec. B.1.1; EWA splatting for the Gaussian covariance)  */
/* ------------------------------------------------------------------------- */

/* world -> sensor: m = R x + t, each row summed left to right */
static void cam_xform(const ocam *c, const double x[3], double m[3]) {
  for (int i = 0; i < 3; i++)
    m[i] = c->R[3 * i + 0] * x[0] + c->R[3 * i + 1] * x[1] + c->R[3 * i + 2] * x[2] + c->t[i];
}

/* Unit-quaternion (w,x,y,z) rotation matrix, row-major. */
static void quat_rot(const double qn[4], double Rq[9]) {
  double w = qn[0], x = qn[1], y = qn[2], z = qn[3];
  Rq[0] = 1.0 - 2.0 * (y * y + z * z);
  Rq[1] = 2.0 * (x * y - w * z);
  Rq[2] = 2.0 * (x * z + w * y);
  Rq[3] = 2.0 * (x * y + w * z);
  Rq[4] = 1.0 - 2.0 * (x * x + z * z);
  Rq[5] = 2.0 * (y * z - w * x);
  Rq[6] = 2.0 * (x * z - w * y);
  Rq[7] = 2.0 * (y * z + w * x);
  Rq[8] = 1.0 - 2.0 * (x * x + y * y);
}

/* Jacobian of the image mapping at sensor point m, and mean 2D position.
 * Pinhole: u = fx mx/mz + cx. Spherical: u = (pi - atan2(my,mx)) W/(2pi),
 * v = (el_max - atan2(mz, rho)) H/(el_max - el_min). */
static void image_map(const ocam *c, const double m[3], double J[6], double *u, double *v) {
  if (c->kind == CAM_PINHOLE) {
    J[0] = c->fx / m[2];
    J[1] = 0.0;
    J[2] = -(c->fx * m[0]) / (m[2] * m[2]);
    J[3] = 0.0;
    J[4] = c->fy / m[2];
    J[5] = -(c->fy * m[1]) / (m[2] * m[2]);
    *u = c->fx * m[0] / m[2] + c->cx;
    *v = c->fy * m[1] / m[2] + c->cy;
  } else {
    double rho2 = m[0] * m[0] + m[1] * m[1];
    double rho = sqrt(rho2);
    double r2 = rho2 + m[2] * m[2];
    double th_max = c->el_max * (M_PI / 180.0), th_min = c->el_min * (M_PI / 180.0);
    double a = (double)c->width / (2.0 * M_PI);
    double b = (double)c->height / (th_max - th_min);
    J[0] = a * m[1] / rho2;
    J[1] = -(a * m[0]) / rho2;
    J[2] = 0.0;
    J[3] = b * m[0] * m[2] / (r2 * rho);
    J[4] = b * m[1] * m[2] / (r2 * rho);
    J[5] = -(b * rho) / r2;
    *u = (M_PI - atan2(m[1], m[0])) * a;
    *v = (th_max - atan2(m[2], rho)) * b;
  }
}

static void set_rect_empty(orec *o) { o->valid = 0; o->ntiles = 0; }

/* Pixel rectangle [xl, xh] x [yl, yh] (pixel-centre coordinates, double) to
 * clipped pixel and tile ranges; columns wrap for the spherical sensor. */
static void set_rect(const ocam *c, orec *o, double xl, double xh, double yl, double yh) {
  double fx0 = ceil(xl - 0.5), fx1 = floor(xh - 0.5);
  double fy0 = ceil(yl - 0.5), fy1 = floor(yh - 0.5);
  if (fy0 < 0.0) fy0 = 0.0;
  if (fy1 > (double)(c->height - 1)) fy1 = (double)(c->height - 1);
  if (c->kind != CAM_SPHERICAL) {
    if (fx0 < 0.0) fx0 = 0.0;
    if (fx1 > (double)(c->width - 1)) fx1 = (double)(c->width - 1);
  } else if (fx1 - fx0 + 1.0 >= (double)c->width) {
    /* a span of a full turn or more covers every column once */
    fx0 = 0.0;
    fx1 = (double)(c->width - 1);
  }
  if (!(fx0 <= fx1) || !(fy0 <= fy1)) { set_rect_empty(o); return; }
  o->x0 = (long long)fx0; o->x1 = (long long)fx1;
  o->y0 = (long long)fy0; o->y1 = (long long)fy1;
  o->ty0 = (int)(o->y0 / TILE); o->ty1 = (int)(o->y1 / TILE);
  if (c->kind != CAM_SPHERICAL) {
    o->tx0 = (int)(o->x0 / TILE);
    o->ntx = (int)(o->x1 / TILE) - o->tx0 + 1;
  } else {
    long long a0 = o->x0 >= 0 ? o->x0 / TILE : -((-o->x0 + TILE - 1) / TILE);
    long long a1 = o->x1 >= 0 ? o->x1 / TILE : -((-o->x1 + TILE - 1) / TILE);
    long long nt = a1 - a0 + 1;
    if (nt > c->tiles_x) nt = c->tiles_x;
    long long m = a0 % c->tiles_x;
    if (m < 0) m += c->tiles_x;
    o->tx0 = (int)m;
    o->ntx = (int)nt;
  }
  o->ntiles = (long long)o->ntx * (long long)(o->ty1 - o->ty0 + 1);
  o->valid = 1;
}

static void project_one(const octx *X, int view, int i, orec *o) {
  const ocam *c = &X->cams[view];
  memset(o, 0, sizeof(*o));
  o->opac = (double)X->opac[i];
  const double K = k_support();
  if (X->kind == PRIM_SPHERE) {
    double p[3] = {X->pos[3 * i], X->pos[3 * i + 1], X->pos[3 * i + 2]};
    double r = (double)X->scale[i];
    double q[3];
    cam_xform(c, p, q);
    double fmin = c->fx < c->fy ? c->fx : c->fy;
    int ortho = c->kind == CAM_ORTHO;
    /* at least one pixel (Pulsar B.1.1): a projected radius of 0.75 px */
    double rfl = ortho ? 0.75 / fmin : 0.75 * q[2] / fmin;
    double re = r >= rfl ? r : rfl;
    o->m[0] = q[0]; o->m[1] = q[1]; o->m[2] = q[2];
    o->r = r; o->r_eff = re; o->floored = r < rfl;
    double zf = q[2] - re;
    if (!(zf > c->znear) || !(zf > 0.0) || !isfinite(r) || !(r > 0.0)) { set_rect_empty(o); return; }
    /* Beyond the far plane the normalised depth is negative, and a smaller
       opacity then gives a larger weight exp(o zhat / gamma): the stop bound
       exp(zhat(front) / gamma) would no longer bound the weights behind it
       (Pulsar sec. 3.2, Figure 3). Such spheres lie outside the depth range the
       normalised device depth spans and are culled; the test is on the fp32 key
       depth, from which the bound is formed, so every drawn sphere has a
       positive bound exponent. */
    if (!((double)(float)zf < c->zfar)) { set_rect_empty(o); return; }
    if (ortho) {
      /* parallel projection: the sphere's outline is the circle of radius r_eff */
      double xl = c->fx * (q[0] - re) + c->cx, xh = c->fx * (q[0] + re) + c->cx;
      double yl = c->fy * (q[1] - re) + c->cy, yh = c->fy * (q[1] + re) + c->cy;
      if (!isfinite(xl) || !isfinite(xh) || !isfinite(yl) || !isfinite(yh)) { set_rect_empty(o); return; }
      o->u = c->fx * q[0] + c->cx;
      o->v = c->fy * q[1] + c->cy;
      o->depth = zf;
      o->key_depth = (float)zf;
      double span = c->zfar - c->znear;
      o->zhat = (c->zfar - q[2]) / span;
      o->e = exp(o->opac * o->zhat / X->gamma);
      o->b = exp(((c->zfar - (double)o->key_depth) / span) / X->gamma);
      double area = M_PI * (c->fx * r) * (c->fy * r);
      o->gated = !(area > 3.0);
      set_rect(c, o, xl, xh, yl, yh);
      return;
    }
    /* tangent planes through the sensor origin, trig-free (Pulsar B.1.1) */
    double den = q[2] * q[2] - re * re;
    double sx = sqrt(q[0] * q[0] + q[2] * q[2] - re * re);
    double sy = sqrt(q[1] * q[1] + q[2] * q[2] - re * re);
    double xl = c->fx * ((q[0] * q[2] - re * sx) / den) + c->cx;
    double xh = c->fx * ((q[0] * q[2] + re * sx) / den) + c->cx;
    double yl = c->fy * ((q[1] * q[2] - re * sy) / den) + c->cy;
    double yh = c->fy * ((q[1] * q[2] + re * sy) / den) + c->cy;
    if (!isfinite(xl) || !isfinite(xh) || !isfinite(yl) || !isfinite(yh)) { set_rect_empty(o); return; }
    o->u = c->fx * q[0] / q[2] + c->cx;
    o->v = c->fy * q[1] / q[2] + c->cy;
    o->depth = zf;
    o->key_depth = (float)zf;
    double span = c->zfar - c->znear;
    o->zhat = (c->zfar - q[2]) / span;
    o->e = exp(o->opac * o->zhat / X->gamma);
    o->b = exp(((c->zfar - (double)o->key_depth) / span) / X->gamma);
    double area = M_PI * (c->fx * r / q[2]) * (c->fy * r / q[2]);
    o->gated = !(area > 3.0);                   /* Pulsar sec. 6 / A: > 3 projected pixels */
    set_rect(c, o, xl, xh, yl, yh);
    return;
  }
  double m[3], u, v, sxx, sxy, syy;
  if (c->kind == CAM_ORTHO) { set_rect_empty(o); return; }   /* orthographic views: spheres only */
  if (X->kind == PRIM_GAUSS2D) {
    u = (double)X->pos[2 * i];
    v = (double)X->pos[2 * i + 1];
    double s = (double)X->scale[i];
    sxx = s * s; syy = s * s; sxy = 0.0;
    o->depth = X->depth[i];
    o->key_depth = (float)X->depth[i];
    m[0] = m[1] = 0.0; m[2] = o->depth;
  } else {
    double mu[3] = {X->pos[3 * i], X->pos[3 * i + 1], X->pos[3 * i + 2]};
    double s[3] = {X->scale[3 * i], X->scale[3 * i + 1], X->scale[3 * i + 2]};
    double qq[4] = {X->rot[4 * i], X->rot[4 * i + 1], X->rot[4 * i + 2], X->rot[4 * i + 3]};
    double nq = sqrt(qq[0] * qq[0] + qq[1] * qq[1] + qq[2] * qq[2] + qq[3] * qq[3]);
    double qn[4] = {qq[0] / nq, qq[1] / nq, qq[2] / nq, qq[3] / nq};
    double Rq[9], M[9], S3[9];
    quat_rot(qn, Rq);
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++) M[3 * a + b] = Rq[3 * a + b] * s[b];
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++)
        S3[3 * a + b] = M[3 * a] * M[3 * b] + M[3 * a + 1] * M[3 * b + 1] + M[3 * a + 2] * M[3 * b + 2];
    cam_xform(c, mu, m);
    if (c->kind == CAM_PINHOLE) {
      if (!(m[2] > c->znear)) { set_rect_empty(o); return; }
      o->depth = m[2];
    } else {
      double rho2 = m[0] * m[0] + m[1] * m[1];
      double rr = sqrt(rho2 + m[2] * m[2]);
      if (!(rr > c->znear) || !(rho2 > 0.0)) { set_rect_empty(o); return; }
      o->depth = rr;
    }
    o->key_depth = (float)o->depth;
    double J[6], T[6], U[6];
    image_map(c, m, J, &u, &v);
    for (int a = 0; a < 2; a++)
      for (int b = 0; b < 3; b++)
        T[3 * a + b] = J[3 * a] * c->R[b] + J[3 * a + 1] * c->R[3 + b] + J[3 * a + 2] * c->R[6 + b];
    for (int a = 0; a < 2; a++)
      for (int b = 0; b < 3; b++)
        U[3 * a + b] = T[3 * a] * S3[b] + T[3 * a + 1] * S3[3 + b] + T[3 * a + 2] * S3[6 + b];
    sxx = U[0] * T[0] + U[1] * T[1] + U[2] * T[2];
    sxy = U[0] * T[3] + U[1] * T[4] + U[2] * T[5];
    syy = U[3] * T[3] + U[4] * T[4] + U[5] * T[5];
  }
  o->m[0] = m[0]; o->m[1] = m[1]; o->m[2] = m[2];
  o->u = u; o->v = v; o->sxx = sxx; o->sxy = sxy; o->syy = syy;
  double det = sxx * syy - sxy * sxy;
  if (!(det > 0.0) || !(o->depth > 0.0) || !isfinite(u) || !isfinite(v)) { set_rect_empty(o); return; }
  o->ca = syy / det; o->cb = -sxy / det; o->cc = sxx / det;
  double hx = sqrt(K * sxx), hy = sqrt(K * syy);
  if (!isfinite(hx) || !isfinite(hy)) { set_rect_empty(o); return; }
  set_rect(c, o, u - hx, u + hx, v - hy, v + hy);
}

/* ------------------------------------------------------------------------- */
/* Context                                                                    */
/* ------------------------------------------------------------------------- */

void or_destroy(octx *X) {
  if (!X) return;
  free(X->pos); free(X->scale); free(X->rot); free(X->opac); free(X->depth); free(X->feat);
  free(X->bg); free(X->cams); free(X->rec); free(X->tile_start); free(X->pair_id); free(X->pair_bits);
  free(X->branch);
  free(X);
}

/* params: alpha_min, alpha_max, T_min, gamma, bg_weight, tau, top_k, then bg[C] */
octx *or_create(int kind, int n, int C, const double *pos, const double *scale, const double *rot,
                const double *opac, const double *depth, const double *feat, int V, const double *cams,
                const double *params) {
  octx *X = (octx *)calloc(1, sizeof(octx));
  X->kind = kind; X->n = n; X->C = C; X->V = V;
  X->pos = dup_d(pos, (long long)n * pdim(kind));
  X->scale = dup_d(scale, (long long)n * sdim(kind));
  X->rot = dup_d(rot, kind == PRIM_GAUSS3D ? (long long)n * 4 : 0);
  X->opac = dup_d(opac, n);
  X->depth = dup_d(depth, kind == PRIM_GAUSS2D ? n : 0);
  X->feat = feat ? dup_d(feat, (long long)n * C) : NULL;
  X->alpha_min = params[0]; X->alpha_max = params[1]; X->T_min = params[2];
  X->gamma = params[3]; X->bg_weight = params[4]; X->tau = params[5]; X->K = (int)params[6];
  X->top_by_depth = (int)params[7];
  X->max_shift = (int)params[8];
  X->bg = (double *)calloc((size_t)(C > 0 ? C : 1), sizeof(double));
  for (int c = 0; c < C; c++) X->bg[c] = params[9 + c];
  X->cams = (ocam *)calloc((size_t)V, sizeof(ocam));
  long long toff = 0, poff = 0;
  for (int v = 0; v < V; v++) {
    const double *a = cams + (size_t)CAM_STRIDE * v;
    ocam *c = &X->cams[v];
    c->kind = (int)a[0]; c->width = (int)a[1]; c->height = (int)a[2];
    for (int k = 0; k < 9; k++) c->R[k] = a[3 + k];
    for (int k = 0; k < 3; k++) c->t[k] = a[12 + k];
    c->fx = a[15]; c->fy = a[16]; c->cx = a[17]; c->cy = a[18];
    c->el_min = a[19]; c->el_max = a[20]; c->znear = a[21]; c->zfar = a[22];
    c->tiles_x = (c->width + TILE - 1) / TILE;
    c->tiles_y = (c->height + TILE - 1) / TILE;
    c->tile_off = toff; c->pix_off = poff;
    toff += (long long)c->tiles_x * c->tiles_y;
    poff += (long long)c->width * c->height;
  }
  X->total_tiles = toff; X->total_pix = poff;
  X->rec = (orec *)calloc((size_t)V * (size_t)n + 1, sizeof(orec));
  #pragma omp parallel for schedule(static)
  for (long long k = 0; k < (long long)V * n; k++) project_one(X, (int)(k / n), (int)(k % n), &X->rec[k]);
  return X;
}

/* OpenMP threads the oracle's parallel loops use (n > 0 sets them). */
int or_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

long long or_total_tiles(const octx *X) { return X->total_tiles; }
long long or_total_pix(const octx *X) { return X->total_pix; }

/* Per record: [u, v, sxx, sxy, syy, ca, cb, cc, depth, m0, m1, m2, r_eff, e, b, zhat, opac]
 * and ints [valid, x0, x1, y0, y1, tx0, ntx, ty0, ty1, ntiles, key_bits, floored, gated] */
#define NPD 17
#define NPI 13
void or_get_proj(const octx *X, double *d, long long *ii) {
  for (long long k = 0; k < (long long)X->V * X->n; k++) {
    const orec *o = &X->rec[k];
    double *p = d + NPD * k;
    p[0] = o->u; p[1] = o->v; p[2] = o->sxx; p[3] = o->sxy; p[4] = o->syy;
    p[5] = o->ca; p[6] = o->cb; p[7] = o->cc; p[8] = o->depth;
    p[9] = o->m[0]; p[10] = o->m[1]; p[11] = o->m[2];
    p[12] = o->r_eff; p[13] = o->e; p[14] = o->b; p[15] = o->zhat; p[16] = o->opac;
    long long *q = ii + NPI * k;
    q[0] = o->valid; q[1] = o->x0; q[2] = o->x1; q[3] = o->y0; q[4] = o->y1;
    q[5] = o->tx0; q[6] = o->ntx; q[7] = o->ty0; q[8] = o->ty1; q[9] = o->valid ? o->ntiles : 0;
    q[10] = o->valid ? f32_bits(o->key_depth) : 0; q[11] = o->floored; q[12] = o->gated;
  }
}

/* ------------------------------------------------------------------------- */
/* Binning and per-tile depth sort                                            */
/* ------------------------------------------------------------------------- */

typedef struct { uint32_t bits, id; } opair;

static int cmp_pair(const void *a, const void *b) {
  const opair *x = (const opair *)a, *y = (const opair *)b;
  if (x->bits != y->bits) return x->bits < y->bits ? -1 : 1;
  if (x->id != y->id) return x->id < y->id ? -1 : 1;
  return 0;
}

/* Every (tile, record) overlap, then each tile's list sorted by (fp32 depth bits, id). */
long long or_bin(octx *X) {
  long long T = X->total_tiles, NV = (long long)X->V * X->n;
  long long *cnt = (long long *)calloc((size_t)T + 1, sizeof(long long));
  for (long long k = 0; k < NV; k++) {
    const orec *o = &X->rec[k];
    if (!o->valid) continue;
    const ocam *c = &X->cams[k / X->n];
    for (int ty = o->ty0; ty <= o->ty1; ty++)
      for (int a = 0; a < o->ntx; a++) {
        int tx = (o->tx0 + a) % c->tiles_x;
        cnt[c->tile_off + (long long)ty * c->tiles_x + tx]++;
      }
  }
  free(X->tile_start); free(X->pair_id); free(X->pair_bits);
  X->tile_start = (long long *)calloc((size_t)T + 1, sizeof(long long));
  for (long long t = 0; t < T; t++) X->tile_start[t + 1] = X->tile_start[t] + cnt[t];
  X->npairs = X->tile_start[T];
  opair *pairs = (opair *)malloc(sizeof(opair) * (size_t)(X->npairs + 1));
  for (long long t = 0; t < T; t++) cnt[t] = X->tile_start[t];
  for (long long k = 0; k < NV; k++) {
    const orec *o = &X->rec[k];
    if (!o->valid) continue;
    const ocam *c = &X->cams[k / X->n];
    for (int ty = o->ty0; ty <= o->ty1; ty++)
      for (int a = 0; a < o->ntx; a++) {
        int tx = (o->tx0 + a) % c->tiles_x;
        long long t = c->tile_off + (long long)ty * c->tiles_x + tx;
        opair pr = {f32_bits(o->key_depth), (uint32_t)k};
        pairs[cnt[t]++] = pr;
      }
  }
  #pragma omp parallel for schedule(dynamic, 16)
  for (long long t = 0; t < T; t++) {
    long long s = X->tile_start[t], e = X->tile_start[t + 1];
    if (e - s > 1) qsort(pairs + s, (size_t)(e - s), sizeof(opair), cmp_pair);
  }
  X->pair_id = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(X->npairs + 1));
  X->pair_bits = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(X->npairs + 1));
  for (long long p = 0; p < X->npairs; p++) { X->pair_id[p] = pairs[p].id; X->pair_bits[p] = pairs[p].bits; }
  free(pairs); free(cnt);
  return X->npairs;
}

/* keys = (global tile << 32) | depth bits, vals = record index; ranges [T][2] */
void or_get_pairs(const octx *X, uint64_t *keys, uint32_t *vals, uint32_t *ranges) {
  for (long long t = 0; t < X->total_tiles; t++) {
    long long s = X->tile_start[t], e = X->tile_start[t + 1];
    if (ranges) { ranges[2 * t] = (uint32_t)(e > s ? s : 0); ranges[2 * t + 1] = (uint32_t)(e > s ? e : 0); }
    for (long long p = s; p < e; p++) {
      if (keys) keys[p] = ((uint64_t)t << 32) | X->pair_bits[p];
      if (vals) vals[p] = X->pair_id[p];
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Per-pixel compositing                                                      */
/* ------------------------------------------------------------------------- */

/* The ray through pixel centre (px, py) in sensor coordinates, o + s d. Pulsar
 * B.1.1 treats two sphere cameras. Pinhole: o = 0, d = ((px - cx)/fx,
 * (py - cy)/fy, 1). Orthographic: every ray runs along +z, o = ((px - cx)/fx,
 * (py - cy)/fy, 0) and d = (0, 0, 1) (fx, fy in pixels per world unit). */
static void pixel_ray(const ocam *c, double px, double py, double o[3], double d[3]) {
  double x = (px - c->cx) / c->fx, y = (py - c->cy) / c->fy;
  if (c->kind == CAM_ORTHO) {
    o[0] = x; o[1] = y; o[2] = 0.0;
    d[0] = 0.0; d[1] = 0.0; d[2] = 1.0;
  } else {
    o[0] = 0.0; o[1] = 0.0; o[2] = 0.0;
    d[0] = x; d[1] = y; d[2] = 1.0;
  }
}

/* Squared orthogonal distance of point q from the ray o + s d (Pulsar A):
 * |e x d|^2 / |d|^2 with e = q - o. (The equal form |e|^2 - (e.d)^2/|d|^2
 * cancels |q|^2 ~ 400 against r^2 ~ 1e-5 and keeps only ~1e-9 of D.) */
static double ray_dist2(const double q[3], const double o[3], const double d[3], double dd) {
  double e[3] = {q[0] - o[0], q[1] - o[1], q[2] - o[2]};
  double c0 = e[1] * d[2] - e[2] * d[1];
  double c1 = e[2] * d[0] - e[0] * d[2];
  double c2 = e[0] * d[1] - e[1] * d[0];
  return (c0 * c0 + c1 * c1 + c2 * c2) / dd;
}

/* Depth (sensor z) of the point where the ray o + s d enters the sphere of
 * centre q and radius r: the smaller root s of |o + s d - q|^2 = r^2, i.e.
 * s = ((e.d) - sqrt(|d|^2 (r^2 - dist^2))) / |d|^2. */
static double ray_entry_depth(const double q[3], const double o[3], const double d[3], double dd, double r) {
  double e[3] = {q[0] - o[0], q[1] - o[1], q[2] - o[2]};
  double ed = e[0] * d[0] + e[1] * d[1] + e[2] * d[2];
  double disc = dd * (r * r - ray_dist2(q, o, d, dd));
  double sroot = (ed - sqrt(disc > 0.0 ? disc : 0.0)) / dd;
  return o[2] + sroot * d[2];
}

typedef struct {          /* per-entry trace kept for the backward pass */
  int idx;                /* position in the tile list */
  uint32_t rec;
  double alpha, T_before, G, dx, dy;   /* alpha path */
  int clamped;
  double w, D, dist2;                  /* sphere path */
  double o[3], d[3], dd;
} otrace;

typedef struct {
  double col[64 + 2];
  double T, N, dep;
  double shift;         /* spheres, max-shift: max(0, largest log-weight of a contributing sphere) */
  long long last, ncontrib, processed;
  int32_t top[16];
  int ntop, flags;
  int nties;            /* near-tie decisions met */
  double errb;          /* Gaussians: relative error bound of T; spheres: of N */
} opix;

/* A near-tie decision: the e-th one met takes the other outcome when bit e of
 * flip is set. */
static int tie_choice(opix *P, unsigned flip, int decision) {
  int e = P->nties++;
  if (e < 31 && ((flip >> e) & 1u)) decision = !decision;
  return decision;
}

static int find_view(const octx *X, long long gpix) {
  int v = 0;
  while (v + 1 < X->V && X->cams[v + 1].pix_off <= gpix) v++;
  return v;
}

static double wrap_dx(double dx, int W) {
  double h = 0.5 * (double)W;
  if (dx >= h) dx -= (double)W;
  else if (dx < -h) dx += (double)W;
  return dx;
}

/* Composite one pixel over its tile's sorted list. tr (optional) receives the
 * composited entries in front-to-back order; returns their number. flip picks
 * the other outcome at near-tie decisions (see tie_choice). */
static int composite(const octx *X, long long gpix, opix *P, otrace *tr, int tr_cap, unsigned flip) {
  int v = find_view(X, gpix);
  const ocam *c = &X->cams[v];
  long long lp = gpix - c->pix_off;
  int i = (int)(lp % c->width), j = (int)(lp / c->width);
  long long t = c->tile_off + (long long)(j / TILE) * c->tiles_x + (i / TILE);
  long long s = X->tile_start[t], e = X->tile_start[t + 1];
  int C = X->C, ntr = 0;
  memset(P, 0, sizeof(*P));
  for (int k = 0; k < 16; k++) P->top[k] = -1;
  double px = (double)i + 0.5, py = (double)j + 0.5;
  if (X->kind == PRIM_SPHERE) {
    double ro[3], d[3];
    pixel_ray(c, px, py, ro, d);
    double dd = d[0] * d[0] + d[1] * d[1] + d[2] * d[2];
    double N = X->bg_weight;
    double S[64];
    for (int ch = 0; ch < C; ch++) S[ch] = X->bg_weight * X->bg[ch];
    /* closest-K mode (Pulsar B.1.3 and B.1.4 keep each pixel's closest five
       intersections): the K + 1 contributing spheres of smallest entry depth so
       far, ordered by (depth, list position) */
    int topd = X->top_by_depth, nc = 0;
    double cz[17];
    otrace ctr[17];
    double nsum = 0.0;          /* sum over hits of N after the hit + 3 w: rounding of an fp32 N */
    for (long long p = s; p < e; p++) {
      const orec *o = &X->rec[X->pair_id[p]];
      P->processed++;
      double lim = X->tau * N;
      int stop = o->b < lim;                                   /* early stop (Pulsar 3.2, B.1.3) */
      double win = 2.0 * U32 * (4.0 + nsum / N);
      if (X->max_shift && lim > 0.0) {
        /* max-shift: an fp32 comparison of beta - ln tau with m + ln(N exp(-m)),
           beta = ln b and m the shift so far; each term rounds relative to its
           size, so the window is u times their magnitudes (doubled) */
        double beta = log(o->b), ltau = log(X->tau), lnN = log(N), m = P->shift;
        win += 2.0 * U32 * (fabs(beta) + fabs(beta - ltau) + 2.0 * fabs(ltau) + fabs(m) + 2.0 * fabs(lnN - m) +
                            fabs(lnN) + 8.0);
      }
      if (lim > 0.0 && fabs(o->b - lim) <= win * lim) {
        P->flags |= FLAG_SPH_STOP;
        stop = tie_choice(P, flip, stop);
      }
      if (stop) break;
      double dist2 = ray_dist2(o->m, ro, d, dd);               /* orthogonal ray distance^2 */
      double r2 = o->r_eff * o->r_eff;
      double D = 1.0 - dist2 / r2;
      int hit = dist2 < r2;
      if (fabs(D) < 1e-8 && (topd || P->ntop < X->K)) {
        P->flags |= FLAG_SPH_EDGE;
        hit = tie_choice(P, flip, hit);
      }
      if (!hit) continue;
      double w = o->opac * D * o->e;
      N += w;
      nsum += N + 3.0 * fabs(w);
      uint32_t id = X->pair_id[p] % (uint32_t)X->n;
      for (int ch = 0; ch < C; ch++) S[ch] += w * X->feat[(size_t)id * C + ch];
      P->ncontrib++;
      {
        double lw = log(o->opac) + o->opac * o->zhat / X->gamma;   /* log of o exp(o zhat / gamma) */
        if (lw > P->shift) P->shift = lw;
      }
      P->last = p - s + 1;
      if (topd) {
        double z = ray_entry_depth(o->m, ro, d, dd, o->r_eff);
        int at = nc;                                   /* insertion point: later positions lose ties */
        while (at > 0 && z < cz[at - 1]) at--;
        if (at <= X->K) {
          int last = nc < X->K + 1 ? nc : X->K;
          for (int k = last; k > at; k--) { cz[k] = cz[k - 1]; ctr[k] = ctr[k - 1]; }
          cz[at] = z;
          otrace *r = &ctr[at];
          r->idx = (int)(p - s); r->rec = X->pair_id[p]; r->w = w; r->D = D; r->dist2 = dist2;
          for (int a = 0; a < 3; a++) { r->o[a] = ro[a]; r->d[a] = d[a]; }
          r->dd = dd;
          if (nc < X->K + 1) nc++;
        }
        continue;
      }
      if (P->ntop < X->K) {
        P->top[P->ntop++] = (int32_t)id;
        if (tr && ntr < tr_cap) {
          otrace *r = &tr[ntr++];
          r->idx = (int)(p - s); r->rec = X->pair_id[p]; r->w = w; r->D = D; r->dist2 = dist2;
          for (int a = 0; a < 3; a++) { r->o[a] = ro[a]; r->d[a] = d[a]; }
          r->dd = dd;
        }
      }
    }
    if (topd) {
      int k = nc < X->K ? nc : X->K;
      /* the kernels form entry depths in fp32 to about 5 ulps */
      if (nc > X->K && fabs(cz[X->K] - cz[X->K - 1]) <= 2e-6 * fabs(cz[X->K - 1])) P->flags |= FLAG_SPH_ZTIE;
      /* the selected ones in list order (the order the reverse pass walks) */
      for (int a = 1; a < k; a++)
        for (int b = a; b > 0 && ctr[b].idx < ctr[b - 1].idx; b--) {
          otrace tmp = ctr[b]; ctr[b] = ctr[b - 1]; ctr[b - 1] = tmp;
        }
      for (int a = 0; a < k; a++) {
        P->top[a] = (int32_t)(ctr[a].rec % (uint32_t)X->n);
        if (tr && ntr < tr_cap) tr[ntr++] = ctr[a];
      }
      P->ntop = k;
    }
    P->N = N;
    P->errb = U32 * nsum / N;
    for (int ch = 0; ch < C; ch++) P->col[ch] = S[ch] / N;
    return ntr;
  }
  /* alpha compositing of Gaussian splats, front to back */
  int lidar = c->kind == CAM_SPHERICAL;
  double T = 1.0, dep = 0.0;
  double tsens = 0.0;         /* sum of alpha / (1 - alpha) over unclamped composited entries */
  double Ccol[64];
  for (int ch = 0; ch < C; ch++) Ccol[ch] = 0.0;
  for (long long p = s; p < e; p++) {
    const orec *o = &X->rec[X->pair_id[p]];
    P->processed++;
    double dx = px - o->u, dy = py - o->v;
    if (lidar) dx = wrap_dx(dx, c->width);
    double power = 0.5 * (o->ca * dx * dx + 2.0 * o->cb * dx * dy + o->cc * dy * dy);
    double G = exp(-power);
    double og = o->opac * G;
    double a = og > X->alpha_max ? X->alpha_max : og;
    if (fabs(og - X->alpha_max) <= EPS_ALPHA * X->alpha_max) P->flags |= FLAG_CLAMP;
    int skip = a < X->alpha_min;
    if (fabs(a - X->alpha_min) <= EPS_ALPHA * X->alpha_min) {
      P->flags |= FLAG_ALPHA_MIN;
      skip = tie_choice(P, flip, skip);
    }
    if (skip) continue;
    double w = T * a;
    uint32_t id = X->pair_id[p] % (uint32_t)X->n;
    if (!lidar)
      for (int ch = 0; ch < C; ch++) Ccol[ch] += w * X->feat[(size_t)id * C + ch];
    else
      dep += w * o->depth;
    if (tr && ntr < tr_cap) {
      otrace *r = &tr[ntr++];
      r->idx = (int)(p - s); r->rec = X->pair_id[p]; r->alpha = a; r->T_before = T; r->G = G;
      r->dx = dx; r->dy = dy; r->clamped = og > X->alpha_max;
    }
    T = T * (1.0 - a);
    if (!(og > X->alpha_max)) tsens += a / (1.0 - a);          /* a clamped alpha is exact */
    P->ncontrib++;
    P->last = p - s + 1;
    int stop = T < X->T_min;                                   /* include, then stop */
    if (fabs(T - X->T_min) <= (EPS_ALPHA * tsens + 1e-12) * X->T_min) {
      P->flags |= FLAG_T_STOP;
      stop = tie_choice(P, flip, stop);
    }
    if (stop) break;
  }
  P->T = T;
  P->errb = EPS_ALPHA * tsens;
  if (!lidar) for (int ch = 0; ch < C; ch++) P->col[ch] = Ccol[ch];
  else { P->col[0] = dep; P->col[1] = 1.0 - T; }
  P->dep = dep;
  return ntr;
}

/* One pixel's outputs into slot q of the output arrays. */
static void put_pixel(const octx *X, const opix *P, long long q, double *img, double *T, long long *last,
                      double *N, int32_t *top) {
  int Cm = X->C > 2 ? X->C : 2;
  for (int ch = 0; ch < Cm; ch++) img[q * Cm + ch] = P->col[ch];
  /* max-shift (spheres): T carries the shift m, N the normalisation times exp(-m) */
  if (T) T[q] = X->max_shift && X->kind == PRIM_SPHERE ? P->shift : P->T;
  if (last) last[q] = P->last;
  if (N) N[q] = X->max_shift && X->kind == PRIM_SPHERE ? P->N * exp(-P->shift) : P->N;
  if (top) for (int k = 0; k < X->K; k++) top[q * X->K + k] = P->top[k];
}

/* Forward over npix global pixel ids (or all pixels when pix == NULL).
 * img: [npix][Cmax] with Cmax = max(C, 2); top: [npix][K]. errb (optional):
 * the relative error bound of an fp32 evaluation's T (Gaussians) or N (spheres). */
void or_render(const octx *X, long long npix, const long long *pix, double *img, double *T,
               long long *last, double *N, int32_t *top, int32_t *flags, long long *processed,
               long long *ncontrib, double *errb) {
  long long cnt = pix ? npix : X->total_pix;
  #pragma omp parallel for schedule(dynamic, 256)
  for (long long q = 0; q < cnt; q++) {
    long long g = pix ? pix[q] : q;
    opix P;
    composite(X, g, &P, NULL, 0, 0u);
    put_pixel(X, &P, q, img, T, last, N, top);
    if (flags) flags[q] = P.flags | (P.nties > MAX_TIES ? FLAG_UNRESOLVED : 0);
    if (processed) processed[q] = P.processed;
    if (ncontrib) ncontrib[q] = P.ncontrib;
    if (errb) errb[q] = P.errb;
  }
}

/* Every outcome of each given pixel over its near-tie decisions: flip mask m
 * (bit e: the e-th tie met takes the other outcome) for all m < 2^MAX_TIES
 * whose set bits all fall on ties the path meets. Per pixel q, nalt[q]
 * outcomes in slots q * 2^MAX_TIES + a: mask, img, T, last, N, top (layouts of
 * or_render). unresolved[q] = 1 when some outcome meets more than MAX_TIES
 * ties (the later ones are then left at their default outcome). */
void or_render_alts(const octx *X, long long npix, const long long *pix, int32_t *nalt, int32_t *mask,
                    double *img, double *T, long long *last, double *N, int32_t *top, int32_t *unresolved) {
  const int NA = 1 << MAX_TIES;
  #pragma omp parallel for schedule(dynamic, 16)
  for (long long q = 0; q < npix; q++) {
    int na = 0, unres = 0;
    for (int m = 0; m < NA; m++) {
      opix P;
      composite(X, pix[q], &P, NULL, 0, (unsigned)m);
      int met = P.nties < MAX_TIES ? P.nties : MAX_TIES;
      if (P.nties > MAX_TIES) unres = 1;
      if ((unsigned)m >> met) continue;                  /* flips a tie this path never meets */
      long long slot = q * NA + na;
      mask[slot] = m;
      put_pixel(X, &P, slot, img, T, last, N, top);
      na++;
    }
    nalt[q] = na;
    unresolved[q] = unres;
  }
}

/* Per global pixel, the flip mask its reverse pass takes (NULL: none). */
void or_set_branches(octx *X, const int32_t *branch) {
  free(X->branch);
  X->branch = NULL;
  if (!branch) return;
  X->branch = (int32_t *)malloc(sizeof(int32_t) * (size_t)(X->total_pix + 1));
  memcpy(X->branch, branch, sizeof(int32_t) * (size_t)X->total_pix);
}

/* Brute force: every valid record, globally sorted by (depth bits, id), with
 * no tiles. Spheres: pixels outside a sphere's box are rejected by the
 * distance test itself; Gaussians: by the 1/255 alpha test. */
static int cmp_rec_order(const void *a, const void *b) { return cmp_pair(a, b); }

void or_render_bruteforce(const octx *X, int v, double *img, double *T, double *N, int32_t *top) {
  const ocam *c = &X->cams[v];
  int C = X->C, Cm = X->C > 2 ? X->C : 2;
  opair *ord = (opair *)malloc(sizeof(opair) * (size_t)(X->n + 1));
  int m = 0;
  for (int i = 0; i < X->n; i++) {
    const orec *o = &X->rec[(long long)v * X->n + i];
    if (!o->valid) continue;
    opair pr = {f32_bits(o->key_depth), (uint32_t)((long long)v * X->n + i)};
    ord[m++] = pr;
  }
  qsort(ord, (size_t)m, sizeof(opair), cmp_rec_order);
  int lidar = c->kind == CAM_SPHERICAL;
  #pragma omp parallel for schedule(dynamic, 16)
  for (int j = 0; j < c->height; j++) {
    for (int i = 0; i < c->width; i++) {
      long long q = (long long)j * c->width + i;
      double px = i + 0.5, py = j + 0.5;
      int ntop = 0;
      if (top) for (int k = 0; k < X->K; k++) top[q * X->K + k] = -1;
      if (X->kind == PRIM_SPHERE) {
        double ro[3], d[3];
        pixel_ray(c, px, py, ro, d);
        double dd = d[0] * d[0] + d[1] * d[1] + d[2] * d[2];
        double Nn = X->bg_weight, S[64];
        for (int ch = 0; ch < C; ch++) S[ch] = X->bg_weight * X->bg[ch];
        for (int k = 0; k < m; k++) {
          const orec *o = &X->rec[ord[k].id];
          if (o->b < X->tau * Nn) break;
          double dist2 = ray_dist2(o->m, ro, d, dd);
          double r2 = o->r_eff * o->r_eff;
          if (!(dist2 < r2)) continue;
          double w = o->opac * (1.0 - dist2 / r2) * o->e;
          Nn += w;
          uint32_t id = ord[k].id % (uint32_t)X->n;
          for (int ch = 0; ch < C; ch++) S[ch] += w * X->feat[(size_t)id * C + ch];
          if (top && ntop < X->K) top[q * X->K + ntop] = (int32_t)id;
          ntop++;
        }
        for (int ch = 0; ch < C; ch++) img[q * Cm + ch] = S[ch] / Nn;
        if (N) N[q] = Nn;
        if (T) T[q] = 0.0;
      } else {
        double Tt = 1.0, dep = 0.0, Cc[64];
        for (int ch = 0; ch < C; ch++) Cc[ch] = 0.0;
        for (int k = 0; k < m; k++) {
          const orec *o = &X->rec[ord[k].id];
          double dx = px - o->u, dy = py - o->v;
          if (lidar) dx = wrap_dx(dx, c->width);
          double power = 0.5 * (o->ca * dx * dx + 2.0 * o->cb * dx * dy + o->cc * dy * dy);
          double og = o->opac * exp(-power);
          double a = og > X->alpha_max ? X->alpha_max : og;
          if (a < X->alpha_min) continue;
          uint32_t id = ord[k].id % (uint32_t)X->n;
          if (!lidar) for (int ch = 0; ch < C; ch++) Cc[ch] += Tt * a * X->feat[(size_t)id * C + ch];
          else dep += Tt * a * o->depth;
          Tt = Tt * (1.0 - a);
          if (Tt < X->T_min) break;
        }
        if (!lidar) for (int ch = 0; ch < C; ch++) img[q * Cm + ch] = Cc[ch];
        else { img[q * Cm] = dep; img[q * Cm + 1] = 1.0 - Tt; }
        if (T) T[q] = Tt;
        if (N) N[q] = 0.0;
      }
    }
  }
  free(ord);
}

/* ------------------------------------------------------------------------- */
/* Backward                                                                   */
/* ------------------------------------------------------------------------- */

/* Per-record 2D accumulator layout, NG = 8 + C doubles:
 * Gaussians: [du, dv, d_ca, d_cb, d_cc, d_opac, d_depth, 0, d_feat...]
 * spheres:   [dq0, dq1, dq2, d_reff, d_opac, count, 0, 0, d_feat...]
 * (count: pixels whose recorded spheres include the record)               */
#define G_OFF 8

/* Reverse pass of one pixel; loc[list position][NG] accumulates.
 *
 * mloc (optional, same layout) accumulates a running magnitude of every term:
 * each factor replaced by its absolute value and each difference a - b by
 * |a| + |b|. It bounds what rounding can do to the sums (an fp32 evaluation of
 * a term carries an error relative to the term's magnitude, so a sum of many
 * terms that cancel is only accurate relative to the sum of magnitudes). It
 * plays no part in the gradient itself. */
static void pixel_backward(const octx *X, long long gpix, const double *g, double *loc, double *mloc, int NG,
                           otrace *tr, int tr_cap, double *kacc, double *kmag) {
  int C = X->C;
  opix P;
  int v = find_view(X, gpix);
  const ocam *c = &X->cams[v];
  int ntr = composite(X, gpix, &P, tr, tr_cap, X->branch ? (unsigned)X->branch[gpix] : 0u);
  if (X->kind == PRIM_SPHERE) {
    double N = P.N;
    for (int k = 0; k < ntr; k++) {
      const otrace *r = &tr[k];
      const orec *o = &X->rec[r->rec];
      uint32_t id = r->rec % (uint32_t)X->n;
      double *A = loc + (size_t)r->idx * NG;
      double *M = mloc ? mloc + (size_t)r->idx * NG : NULL;
      double dw = 0.0, mdw = 0.0;
      A[5] += 1.0;
      for (int ch = 0; ch < C; ch++) {
        double f = X->feat[(size_t)id * C + ch];
        A[G_OFF + ch] += g[ch] * r->w / N;
        dw += g[ch] * (f - P.col[ch]) / N;
        if (M) {
          M[G_OFF + ch] += fabs(g[ch]) * r->w / N;
          mdw += fabs(g[ch]) * (fabs(f) + fabs(P.col[ch])) / N;
        }
      }
      /* w = o * D * exp(o * zhat / gamma) */
      double e = o->e, oo = o->opac;
      A[4] += dw * (r->D * e + r->w * o->zhat / X->gamma);
      if (M) M[4] += mdw * (r->D * e + r->w * fabs(o->zhat) / X->gamma);
      if (o->gated) continue;                       /* tiny spheres: features and opacity only */
      double dD = dw * oo * e;
      double dzhat = dw * r->w * oo / X->gamma;
      double r2 = o->r_eff * o->r_eff;
      double ddist2 = -dD / r2;
      /* dist2 = |e|^2 - (e.d)^2/|d|^2 with e = q - o: d dist2 / d q = 2 (e - (e.d) d/|d|^2) */
      double q[3] = {o->m[0] - r->o[0], o->m[1] - r->o[1], o->m[2] - r->o[2]};
      double qd = q[0] * r->d[0] + q[1] * r->d[1] + q[2] * r->d[2];
      for (int a = 0; a < 3; a++) A[a] += ddist2 * (2.0 * q[a] - 2.0 * qd * r->d[a] / r->dd);
      A[2] += dzhat * (-1.0 / (c->zfar - c->znear));
      if (!o->floored) A[3] += dD * 2.0 * r->dist2 / (r2 * o->r_eff);
      /* Intrinsics (Pulsar 3.2 and appendix A: gradients for focal length and
         sensor placement). x = (px - cx)/fx and y = (py - cy)/fy move with them,
         d x / d fx = -x / fx, d x / d cx = -1 / fx. Pinhole: (x, y) are d's first
         components, d dist2 / d d_a = -2 (e.d)/|d|^2 (e_a - (e.d) d_a/|d|^2).
         Orthographic: (x, y) are o's, d dist2 / d o_a = -d dist2 / d q_a. The
         one-pixel floor of r_eff is held fixed, as for the position. */
      for (int a = 0; a < 2; a++) {
        double f = a == 0 ? c->fx : c->fy;
        double gd, xa;
        if (c->kind == CAM_ORTHO) {
          gd = -ddist2 * (2.0 * q[a] - 2.0 * qd * r->d[a] / r->dd);
          xa = r->o[a];
        } else {
          gd = ddist2 * (-2.0 * qd / r->dd) * (q[a] - qd * r->d[a] / r->dd);
          xa = r->d[a];
        }
        kacc[a] += gd * (-xa / f);
        kacc[2 + a] += gd * (-1.0 / f);
      }
      if (M) {
        double mD = mdw * oo * e, mz = mdw * r->w * oo / X->gamma, m2 = mD / r2;
        for (int a = 0; a < 3; a++) M[a] += m2 * (2.0 * fabs(q[a]) + 2.0 * fabs(qd * r->d[a]) / r->dd);
        M[2] += mz / (c->zfar - c->znear);
        if (!o->floored) M[3] += mD * 2.0 * r->dist2 / (r2 * o->r_eff);
        for (int a = 0; a < 2; a++) {
          double f = a == 0 ? c->fx : c->fy;
          double mg, xa;
          if (c->kind == CAM_ORTHO) {
            mg = m2 * (2.0 * fabs(q[a]) + 2.0 * fabs(qd * r->d[a]) / r->dd);
            xa = r->o[a];
          } else {
            mg = m2 * 2.0 * fabs(qd) / r->dd * (fabs(q[a]) + fabs(qd * r->d[a]) / r->dd);
            xa = r->d[a];
          }
          kmag[a] += mg * fabs(xa) / f;
          kmag[2 + a] += mg / f;
        }
      }
    }
    return;
  }
  int lidar = c->kind == CAM_SPHERICAL;
  int nC = lidar ? 0 : C;
  double Sb[64], Sd = 0.0;
  for (int ch = 0; ch < nC; ch++) Sb[ch] = 0.0;
  double gD = lidar ? g[0] : 0.0, gA = lidar ? g[1] : 0.0;
  double Tfin = P.T;
  for (int k = ntr - 1; k >= 0; k--) {
    const otrace *r = &tr[k];
    const orec *o = &X->rec[r->rec];
    uint32_t id = r->rec % (uint32_t)X->n;
    double *A = loc + (size_t)r->idx * NG;
    double *M = mloc ? mloc + (size_t)r->idx * NG : NULL;
    double a = r->alpha, Tk = r->T_before;
    double da = 0.0, mda = 0.0;
    for (int ch = 0; ch < nC; ch++) {
      double f = X->feat[(size_t)id * C + ch];
      A[G_OFF + ch] += Tk * a * g[ch];
      da += Tk * (f - Sb[ch]) * g[ch];
      if (M) {
        M[G_OFF + ch] += Tk * a * fabs(g[ch]);
        mda += Tk * (fabs(f) + fabs(Sb[ch])) * fabs(g[ch]);
      }
      Sb[ch] = a * f + (1.0 - a) * Sb[ch];
    }
    if (lidar) {
      A[6] += Tk * a * gD;
      da += Tk * (o->depth - Sd) * gD + Tfin / (1.0 - a) * gA;
      if (M) {
        M[6] += Tk * a * fabs(gD);
        mda += Tk * (fabs(o->depth) + fabs(Sd)) * fabs(gD) + Tfin / (1.0 - a) * fabs(gA);
      }
      Sd = a * o->depth + (1.0 - a) * Sd;
    }
    if (r->clamped) continue;                      /* alpha = 0.99 constant there */
    A[5] += r->G * da;
    double dpower = -a * da;
    double dx = r->dx, dy = r->dy;
    A[0] -= dpower * (o->ca * dx + o->cb * dy);
    A[1] -= dpower * (o->cb * dx + o->cc * dy);
    A[2] += dpower * 0.5 * dx * dx;
    A[3] += dpower * dx * dy;
    A[4] += dpower * 0.5 * dy * dy;
    if (M) {
      double mp = a * mda;
      M[5] += r->G * mda;
      M[0] += mp * (fabs(o->ca * dx) + fabs(o->cb * dy));
      M[1] += mp * (fabs(o->cb * dx) + fabs(o->cc * dy));
      M[2] += mp * 0.5 * dx * dx;
      M[3] += mp * fabs(dx * dy);
      M[4] += mp * 0.5 * dy * dy;
    }
  }
}

/* Derivative of the image-map Jacobian entries J[k] with respect to m[a]: dJ[k][a]. */
static void image_map_dJ(const ocam *c, const double m[3], double dJ[6][3]) {
  memset(dJ, 0, sizeof(double) * 18);
  if (c->kind == CAM_PINHOLE) {
    double z2 = m[2] * m[2], z3 = z2 * m[2];
    dJ[0][2] = -c->fx / z2;
    dJ[2][0] = -c->fx / z2;
    dJ[2][2] = 2.0 * c->fx * m[0] / z3;
    dJ[4][2] = -c->fy / z2;
    dJ[5][1] = -c->fy / z2;
    dJ[5][2] = 2.0 * c->fy * m[1] / z3;
  } else {
    double th_max = c->el_max * (M_PI / 180.0), th_min = c->el_min * (M_PI / 180.0);
    double a = (double)c->width / (2.0 * M_PI), b = (double)c->height / (th_max - th_min);
    double x = m[0], y = m[1], z = m[2];
    double rho2 = x * x + y * y, rho = sqrt(rho2), r2 = rho2 + z * z;
    double rho4 = rho2 * rho2, r4 = r2 * r2;
    dJ[0][0] = -2.0 * a * x * y / rho4;
    dJ[0][1] = a * (x * x - y * y) / rho4;
    dJ[1][0] = a * (x * x - y * y) / rho4;
    dJ[1][1] = 2.0 * a * x * y / rho4;
    double h = 1.0 / (r2 * rho);
    double hx = -x * (2.0 * rho2 + r2) / (r4 * rho2 * rho);
    double hy = -y * (2.0 * rho2 + r2) / (r4 * rho2 * rho);
    double hz = -2.0 * z / (r4 * rho);
    dJ[3][0] = b * z * (h + x * hx);
    dJ[3][1] = b * x * z * hy;
    dJ[3][2] = b * x * (h + z * hz);
    dJ[4][0] = b * y * z * hx;
    dJ[4][1] = b * z * (h + y * hy);
    dJ[4][2] = b * y * (h + z * hz);
    dJ[5][0] = -b * x * (r2 - 2.0 * rho2) / (rho * r4);
    dJ[5][1] = -b * y * (r2 - 2.0 * rho2) / (rho * r4);
    dJ[5][2] = 2.0 * b * rho * z / r4;
  }
}

/* Chain rule from the 2D accumulator of one record to the primitive parameters.
 * out_* are per-primitive (summed over views by the caller, serially). */
static void project_backward(const octx *X, long long k, const double *A, double *dpos, double *dscale,
                             double *drot, double *dop) {
  const orec *o = &X->rec[k];
  int i = (int)(k % X->n), v = (int)(k / X->n);
  const ocam *c = &X->cams[v];
  *dop += A[X->kind == PRIM_SPHERE ? 4 : 5];
  if (X->kind == PRIM_SPHERE) {
    const double *dq = A;
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++) dpos[a] += c->R[3 * b + a] * dq[b];   /* R^T dq */
    dscale[0] += A[3];
    return;
  }
  if (X->kind == PRIM_GAUSS2D) {
    double s = (double)X->scale[i];
    dpos[0] += A[0];
    dpos[1] += A[1];
    /* ca = cc = 1/s^2 */
    dscale[0] += (A[2] + A[4]) * (-2.0 / (s * s * s));
    return;
  }
  /* GAUSS3D: conic -> cov2D -> (T, Sigma3D) -> (m, Rq, s) -> (mu, quaternion) */
  double Q[4] = {o->ca, o->cb, o->cb, o->cc};
  double Gq[4] = {A[2], 0.5 * A[3], 0.5 * A[3], A[4]};
  double QG[4], dS2[4];
  QG[0] = Q[0] * Gq[0] + Q[1] * Gq[2]; QG[1] = Q[0] * Gq[1] + Q[1] * Gq[3];
  QG[2] = Q[2] * Gq[0] + Q[3] * Gq[2]; QG[3] = Q[2] * Gq[1] + Q[3] * Gq[3];
  dS2[0] = -(QG[0] * Q[0] + QG[1] * Q[2]); dS2[1] = -(QG[0] * Q[1] + QG[1] * Q[3]);
  dS2[2] = -(QG[2] * Q[0] + QG[3] * Q[2]); dS2[3] = -(QG[2] * Q[1] + QG[3] * Q[3]);
  /* recompute the forward quantities */
  double s[3] = {X->scale[3 * i], X->scale[3 * i + 1], X->scale[3 * i + 2]};
  double qq[4] = {X->rot[4 * i], X->rot[4 * i + 1], X->rot[4 * i + 2], X->rot[4 * i + 3]};
  double nq = sqrt(qq[0] * qq[0] + qq[1] * qq[1] + qq[2] * qq[2] + qq[3] * qq[3]);
  double qn[4] = {qq[0] / nq, qq[1] / nq, qq[2] / nq, qq[3] / nq};
  double Rq[9], M[9], S3[9], J[6], T[6], u, vv;
  quat_rot(qn, Rq);
  for (int a = 0; a < 3; a++) for (int b = 0; b < 3; b++) M[3 * a + b] = Rq[3 * a + b] * s[b];
  for (int a = 0; a < 3; a++) for (int b = 0; b < 3; b++)
    S3[3 * a + b] = M[3 * a] * M[3 * b] + M[3 * a + 1] * M[3 * b + 1] + M[3 * a + 2] * M[3 * b + 2];
  const double *m = o->m;
  image_map(c, m, J, &u, &vv);
  for (int a = 0; a < 2; a++) for (int b = 0; b < 3; b++)
    T[3 * a + b] = J[3 * a] * c->R[b] + J[3 * a + 1] * c->R[3 + b] + J[3 * a + 2] * c->R[6 + b];
  /* Sigma2 = T S3 T^T: dS3 = T^T dS2 T ; dT = 2 dS2 T S3 */
  double dS3[9], dT[6], TS3[6];
  for (int a = 0; a < 3; a++) for (int b = 0; b < 3; b++) {
    double acc = 0.0;
    for (int p = 0; p < 2; p++) for (int q = 0; q < 2; q++) acc += T[3 * p + a] * dS2[2 * p + q] * T[3 * q + b];
    dS3[3 * a + b] = acc;
  }
  for (int a = 0; a < 2; a++) for (int b = 0; b < 3; b++) {
    double acc = 0.0;
    for (int q = 0; q < 3; q++) acc += T[3 * a + q] * S3[3 * q + b];
    TS3[3 * a + b] = acc;
  }
  for (int a = 0; a < 2; a++) for (int b = 0; b < 3; b++)
    dT[3 * a + b] = 2.0 * (dS2[2 * a] * TS3[b] + dS2[2 * a + 1] * TS3[3 + b]);
  /* T = J W: dJ = dT W^T */
  double dJ[6];
  for (int a = 0; a < 2; a++) for (int b = 0; b < 3; b++)
    dJ[3 * a + b] = dT[3 * a] * c->R[3 * b] + dT[3 * a + 1] * c->R[3 * b + 1] + dT[3 * a + 2] * c->R[3 * b + 2];
  double Jm[6][3];
  image_map_dJ(c, m, Jm);
  double dm[3] = {0, 0, 0};
  for (int a = 0; a < 3; a++) {
    for (int k2 = 0; k2 < 6; k2++) dm[a] += dJ[k2] * Jm[k2][a];
    dm[a] += A[0] * J[a] + A[1] * J[3 + a];           /* mean 2D */
  }
  if (c->kind == CAM_SPHERICAL) {
    double rr = o->depth;
    for (int a = 0; a < 3; a++) dm[a] += A[6] * m[a] / rr;   /* range */
  }
  for (int a = 0; a < 3; a++)
    dpos[a] += c->R[a] * dm[0] + c->R[3 + a] * dm[1] + c->R[6 + a] * dm[2];
  /* Sigma3 = M M^T: dM = 2 dS3 M (dS3 symmetric) */
  double dM[9];
  for (int a = 0; a < 3; a++) for (int b = 0; b < 3; b++)
    dM[3 * a + b] = 2.0 * (dS3[3 * a] * M[b] + dS3[3 * a + 1] * M[3 + b] + dS3[3 * a + 2] * M[6 + b]);
  double dRq[9];
  for (int a = 0; a < 3; a++) for (int b = 0; b < 3; b++) {
    dscale[b] += dM[3 * a + b] * Rq[3 * a + b];
    dRq[3 * a + b] = dM[3 * a + b] * s[b];
  }
  double w = qn[0], x = qn[1], y = qn[2], z = qn[3];
  double dqn[4];
  dqn[0] = 2.0 * (-z * dRq[1] + y * dRq[2] + z * dRq[3] - x * dRq[5] - y * dRq[6] + x * dRq[7]);
  dqn[1] = 2.0 * (y * dRq[1] + z * dRq[2] + y * dRq[3] - 2.0 * x * dRq[4] - w * dRq[5] + z * dRq[6]
                  + w * dRq[7] - 2.0 * x * dRq[8]);
  dqn[2] = 2.0 * (-2.0 * y * dRq[0] + x * dRq[1] + w * dRq[2] + x * dRq[3] + z * dRq[5] - w * dRq[6]
                  + z * dRq[7] - 2.0 * y * dRq[8]);
  dqn[3] = 2.0 * (-2.0 * z * dRq[0] - w * dRq[1] + x * dRq[2] + w * dRq[3] - 2.0 * z * dRq[4]
                  + y * dRq[5] + x * dRq[6] + y * dRq[7]);
  double dot = qn[0] * dqn[0] + qn[1] * dqn[1] + qn[2] * dqn[2] + qn[3] * dqn[3];
  for (int a = 0; a < 4; a++) drot[a] += (dqn[a] - qn[a] * dot) / nq;
}

/* Magnitude through the chain rule: the map from a record's accumulator to the
 * primitive's parameter gradients is linear, so each accumulator slot j moves
 * the outputs by column j of that map; the magnitudes add |column j| * M[j]. */
static void project_backward_mag(const octx *X, long long k, const double *M, double *mpos, double *mscale,
                                 double *mrot, double *mop) {
  double e[G_OFF];
  for (int j = 0; j < G_OFF; j++) {
    if (M[j] == 0.0) continue;
    for (int q = 0; q < G_OFF; q++) e[q] = q == j ? 1.0 : 0.0;
    double tp[3] = {0, 0, 0}, ts[3] = {0, 0, 0}, tr[4] = {0, 0, 0, 0}, to = 0.0;
    project_backward(X, k, e, tp, ts, tr, &to);
    for (int a = 0; a < 3; a++) mpos[a] += fabs(tp[a]) * M[j];
    for (int a = 0; a < 3; a++) mscale[a] += fabs(ts[a]) * M[j];
    for (int a = 0; a < 4; a++) mrot[a] += fabs(tr[a]) * M[j];
    *mop += fabs(to) * M[j];
  }
}

typedef struct {
  double *pos, *scale, *rot, *op, *feat, *R, *t;
} omag;

/* Backward. dimg: concatenated per-view [Cv][H][W] float32 upstream gradients
 * (Cv = C for pinhole views, 2 = (depth, opacity) for spherical views).
 * Outputs are written (not accumulated). acc_out (optional) receives the
 * per-record 2D accumulators [V*n][8+C]. dK [V][4] receives the gradient
 * w.r.t. each view's fx, fy, cx, cy (spheres; zero for Gaussians), summed per
 * tile and then over tiles in order; mK (optional) its magnitudes. mag
 * (optional) receives the running magnitudes of every output, in the outputs'
 * layouts. normalize (spheres): Pulsar B.2's normalisation, sphere gradients
 * averaged over their contributing pixels, camera contributions divided by the
 * projected area and by 1e-3; the intrinsic gradients stay raw per-pixel sums. */
static void backward_core(const octx *X, const float *dimg, double *dpos, double *dscale, double *drot,
                          double *dop, double *dfeat, double *dR, double *dt, double *acc_out, double *dK,
                          double *mK, const omag *mag, int normalize) {
  int C = X->C, NG = G_OFF + C;
  long long NV = (long long)X->V * X->n;
  double *acc = (double *)calloc((size_t)NV * NG + 1, sizeof(double));
  double *macc = mag ? (double *)calloc((size_t)NV * NG + 1, sizeof(double)) : NULL;
  long long ntile = X->total_tiles;
  memset(dK, 0, sizeof(double) * 4 * (size_t)X->V);
  if (mK) memset(mK, 0, sizeof(double) * 4 * (size_t)X->V);
  /* Tiles run in parallel; each accumulates by tile-list position into a private
     buffer, merged into the per-record sums in tile order (deterministic). */
  #pragma omp parallel
  {
    double *loc = NULL, *mloc = NULL;
    otrace *tr = NULL;
    long long cap = 0;
    #pragma omp for schedule(dynamic, 4) ordered
    for (long long t = 0; t < ntile; t++) {
      int v = 0;
      while (v + 1 < X->V && X->cams[v + 1].tile_off <= t) v++;
      const ocam *c = &X->cams[v];
      long long s = X->tile_start[t], e = X->tile_start[t + 1], len = e - s;
      if (len > cap) {
        free(loc); free(mloc); free(tr);
        cap = len;
        loc = (double *)malloc(sizeof(double) * (size_t)(cap * NG));
        mloc = macc ? (double *)malloc(sizeof(double) * (size_t)(cap * NG)) : NULL;
        tr = (otrace *)malloc(sizeof(otrace) * (size_t)cap);
      }
      int lt = (int)(t - c->tile_off);
      int tx = lt % c->tiles_x, ty = lt / c->tiles_x;
      int Cv = c->kind == CAM_SPHERICAL ? 2 : C;
      const float *gv = dimg;
      for (int u = 0; u < v; u++)
        gv += (size_t)(X->cams[u].kind == CAM_SPHERICAL ? 2 : C) * X->cams[u].width * X->cams[u].height;
      int any = 0;
      double kt[4] = {0, 0, 0, 0}, kmt[4] = {0, 0, 0, 0};
      for (long long p = 0; p < len * NG; p++) loc[p] = 0.0;
      if (mloc) for (long long p = 0; p < len * NG; p++) mloc[p] = 0.0;
      for (int jj = 0; jj < TILE && len > 0; jj++)
        for (int ii = 0; ii < TILE; ii++) {
          int i = tx * TILE + ii, j = ty * TILE + jj;
          if (i >= c->width || j >= c->height) continue;
          double g[66];
          int nz = 0;
          for (int ch = 0; ch < Cv; ch++) {
            g[ch] = (double)gv[(size_t)ch * c->width * c->height + (size_t)j * c->width + i];
            nz |= g[ch] != 0.0;
          }
          /* spheres: a pixel whose upstream gradient is zero still counts among the
             pixels a recorded sphere contributes to (gradient normalisation) */
          if (!nz && X->kind != PRIM_SPHERE) continue;
          any = 1;
          pixel_backward(X, c->pix_off + (long long)j * c->width + i, g, loc, mloc, NG, tr, (int)len, kt, kmt);
        }
      #pragma omp ordered
      {
        for (int a = 0; a < 4; a++) {
          dK[4 * v + a] += kt[a];
          if (mK) mK[4 * v + a] += kmt[a];
        }
        if (any)
          for (long long p = s; p < e; p++) {
            double *B = acc + (size_t)X->pair_id[p] * NG;
            const double *L = loc + (p - s) * NG;
            for (int q = 0; q < NG; q++) B[q] += L[q];
            if (macc) {
              double *MB = macc + (size_t)X->pair_id[p] * NG;
              const double *ML = mloc + (p - s) * NG;
              for (int q = 0; q < NG; q++) MB[q] += ML[q];
            }
          }
      }
    }
    free(loc); free(mloc); free(tr);
  }
  /* per-primitive chain rule, views summed in order */
  int n = X->n;
  int pd = X->kind == PRIM_GAUSS2D ? 2 : 3, sd = X->kind == PRIM_GAUSS3D ? 3 : 1;
  memset(dpos, 0, sizeof(double) * (size_t)n * pd);
  memset(dscale, 0, sizeof(double) * (size_t)n * sd);
  if (drot) memset(drot, 0, sizeof(double) * (size_t)n * 4);
  memset(dop, 0, sizeof(double) * (size_t)n);
  if (dfeat) memset(dfeat, 0, sizeof(double) * (size_t)n * C);
  memset(dR, 0, sizeof(double) * 9 * (size_t)X->V);
  memset(dt, 0, sizeof(double) * 3 * (size_t)X->V);
  #pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) {
    double lpos[3] = {0, 0, 0}, ls[3] = {0, 0, 0}, lr[4] = {0, 0, 0, 0}, lo = 0.0;
    for (int v = 0; v < X->V; v++) {
      long long k = (long long)v * n + i;
      if (!X->rec[k].valid) continue;
      const double *A = acc + (size_t)k * NG;
      project_backward(X, k, A, lpos, ls, lr, &lo);
      if (dfeat) for (int ch = 0; ch < C; ch++) dfeat[(size_t)i * C + ch] += A[G_OFF + ch];
    }
    /* Pulsar B.2 normalisation: a sphere's gradients averaged over the pixels that
       sent it gradients (its recorded contributions, all views of the call) */
    double sc = 1.0;
    if (normalize && X->kind == PRIM_SPHERE) {
      double cnt = 0.0;
      for (int v = 0; v < X->V; v++) {
        long long k = (long long)v * n + i;
        if (X->rec[k].valid) cnt += acc[(size_t)k * NG + 5];
      }
      sc = cnt > 0.0 ? 1.0 / cnt : 0.0;
      for (int a = 0; a < 3; a++) lpos[a] *= sc;
      ls[0] *= sc;
      lo *= sc;
      if (dfeat) for (int ch = 0; ch < C; ch++) dfeat[(size_t)i * C + ch] *= sc;
    }
    for (int a = 0; a < pd; a++) dpos[(size_t)i * pd + a] = lpos[a];
    for (int a = 0; a < sd; a++) dscale[(size_t)i * sd + a] = ls[a];
    if (drot) for (int a = 0; a < 4; a++) drot[(size_t)i * 4 + a] = lr[a];
    dop[i] = lo;
    if (mag) {
      double mp[3] = {0, 0, 0}, ms[3] = {0, 0, 0}, mr[4] = {0, 0, 0, 0}, mo = 0.0;
      for (int v = 0; v < X->V; v++) {
        long long k = (long long)v * n + i;
        if (!X->rec[k].valid) continue;
        const double *M = macc + (size_t)k * NG;
        project_backward_mag(X, k, M, mp, ms, mr, &mo);
        if (mag->feat) for (int ch = 0; ch < C; ch++) mag->feat[(size_t)i * C + ch] += M[G_OFF + ch] * sc;
      }
      for (int a = 0; a < 3; a++) mp[a] *= sc;
      ms[0] *= sc;
      mo *= sc;
      for (int a = 0; a < pd; a++) mag->pos[(size_t)i * pd + a] = mp[a];
      for (int a = 0; a < sd; a++) mag->scale[(size_t)i * sd + a] = ms[a];
      if (mag->rot) for (int a = 0; a < 4; a++) mag->rot[(size_t)i * 4 + a] = mr[a];
      mag->op[i] = mo;
    }
  }
  if (X->kind == PRIM_SPHERE) {
    /* camera: sphere-wise contributions summed over all spheres (Pulsar B.2).
       Normalised: each sphere's contribution divided by its projected area in
       pixels, pi (fx r_eff / qz)(fy r_eff / qz) (orthographic: pi (fx r_eff)(fy r_eff)),
       and by 1e-3. */
    for (int v = 0; v < X->V; v++)
      for (int i = 0; i < n; i++) {
        long long k = (long long)v * n + i;
        if (!X->rec[k].valid) continue;
        const double *A = acc + (size_t)k * NG;
        const orec *o = &X->rec[k];
        const ocam *c = &X->cams[v];
        double sc = 1.0;
        if (normalize) {
          double iz = c->kind == CAM_ORTHO ? 1.0 : 1.0 / o->m[2];
          double area = M_PI * (c->fx * o->r_eff * iz) * (c->fy * o->r_eff * iz);
          sc = 1.0 / (area * 1e-3);
        }
        double p[3] = {X->pos[3 * i], X->pos[3 * i + 1], X->pos[3 * i + 2]};
        for (int a = 0; a < 3; a++) {
          for (int b = 0; b < 3; b++) dR[9 * v + 3 * a + b] += A[a] * sc * p[b];
          dt[3 * v + a] += A[a] * sc;
          if (mag) {
            const double *M = macc + (size_t)k * NG;
            for (int b = 0; b < 3; b++) mag->R[9 * v + 3 * a + b] += M[a] * sc * fabs(p[b]);
            mag->t[3 * v + a] += M[a] * sc;
          }
        }
      }
  }
  if (acc_out) memcpy(acc_out, acc, sizeof(double) * (size_t)NV * NG);
  free(acc);
  free(macc);
}

void or_backward(const octx *X, const float *dimg, double *dpos, double *dscale, double *drot,
                 double *dop, double *dfeat, double *dR, double *dt, double *acc_out, double *dK,
                 int normalize) {
  backward_core(X, dimg, dpos, dscale, drot, dop, dfeat, dR, dt, acc_out, dK, NULL, NULL, normalize);
}

/* Same as or_backward, plus the magnitudes (zero-initialised by the caller,
 * same layouts as the gradients; mfeat and mrot may be NULL when absent). */
void or_backward_mag(const octx *X, const float *dimg, double *dpos, double *dscale, double *drot,
                     double *dop, double *dfeat, double *dR, double *dt, double *acc_out, double *mpos,
                     double *mscale, double *mrot, double *mop, double *mfeat, double *mR, double *mt,
                     double *dK, double *mK, int normalize) {
  omag m = {mpos, mscale, mrot, mop, mfeat, mR, mt};
  backward_core(X, dimg, dpos, dscale, drot, dop, dfeat, dR, dt, acc_out, dK, mK, &m, normalize);
}
