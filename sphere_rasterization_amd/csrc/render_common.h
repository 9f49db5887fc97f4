// Per-pixel arithmetic shared by the forward and backward compositors. Both
// passes evaluate the same inline functions on the same staged values, so the
// backward takes exactly the decisions the forward took (skip, stop, top-K).
#pragma once
#include "splat_internal.h"

#define SPLAT_TOPK_MAX 8

// Workgroups appended to the sphere forward's grid to clear the reverse pass's
// sums (when the caller hands over the reverse pass's workspace).
constexpr int FWD_CLEAR_BLOCKS = 256;
constexpr int FWD_CLEAR_GRID = 8192;     // workgroups of the Gaussians' clearing launch

struct FwdArgs {
  int n, C, top_k;
  int top_by_depth;       // spheres: record the top_k closest entry points, not the first top_k
  int max_shift;          // spheres: draw records hold log-weights; blend relative to a per-pixel shift
  int serial_views;       // Gaussians: camera and spherical views on the caller's stream only
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
  // optional: the reverse pass's sums to clear (16-byte units; spheres: the
  // FWD_CLEAR_BLOCKS workgroups after the tiles' do it, Gaussians: k_fwd_clear)
  int clear;
  uint4 *clr[3];
  long long nclr[3];
};

struct BwdArgs {
  int n, C, top_k;
  float alpha_min, alpha_max, gamma;
  float igamma;           // 1 / gamma (host)
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
  double *accg;           // Gaussians: [records][ACC_G]; unused for spheres
  double *accf;           // Gaussians: [records][C]; unused for spheres
  float *accs;            // spheres: [records][rs] fp32 rows of 5 + C values
  int rs;                 // spheres: row stride (floats)
  double *cam_part;       // [SPLAT_CAM_BLOCKS][12] per-block camera sums (spheres)
  double *kslot;          // [views][SPLAT_K_SLOTS][4] intrinsic-gradient sums, or NULL (not requested)
  uint32_t *cnt;          // [records] pixels that recorded the sphere, or NULL (no normalisation)
  int max_shift;          // spheres: weights relative to the per-pixel shift held in T_final
  int direct_max;         // spheres: entries recorded by at most this many lanes add lane by lane
  int serial_views;       // Gaussians: camera and spherical views on the caller's stream only
};

struct TilePix {
  int i, j;
  bool inside;
  float x0, y0;      // tile origin (pixels)
  float pxr, pyr;    // pixel centre relative to the tile origin
};

// Thread tid of a tile's workgroup: wave w = tid / 64 owns the 8x8 quadrant
// (w & 1, w >> 1) of the 16x16 tile, its 16-lane group g = (tid / 16) & 3 the
// 4x4 block (g & 1, g >> 1) of that quadrant, and lane l the pixel
// (l & 3, (l >> 2) & 3) of the block.
__device__ __forceinline__ TilePix tile_pixel(const ViewDev &c, int gtile, unsigned tid) {
  const int lt = gtile - c.tile_off;
  const int ty = lt / c.TW, tx = lt - ty * c.TW;
  const unsigned w = tid >> 6, g = (tid >> 4) & 3u, l = tid & 15u;
  const int li = (int)((w & 1u) * 8u + (g & 1u) * 4u + (l & 3u));
  const int lj = (int)((w >> 1) * 8u + (g >> 1) * 4u + (l >> 2));
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

// Which quadrants of the tile at (x0, y0) the pixel rectangle of d reaches (4 bits).
__device__ __forceinline__ unsigned quadrant_mask(const TilePix &tp, const DrawRec &d) {
  const int x0 = (int)tp.x0, y0 = (int)tp.y0;
  const bool c0 = d.i0 <= x0 + 7 && d.i1 >= x0;
  const bool c1 = d.i0 <= x0 + 15 && d.i1 >= x0 + 8;
  const bool r0 = d.j0 <= y0 + 7 && d.j1 >= y0;
  const bool r1 = d.j0 <= y0 + 15 && d.j1 >= y0 + 8;
  return (unsigned)(c0 && r0) | ((unsigned)(c1 && r0) << 1) | ((unsigned)(c0 && r1) << 2) |
         ((unsigned)(c1 && r1) << 3);
}

// Per-quadrant lists of the staged batch, in batch order: every wave then walks
// only the entries that reach its quadrant.
struct QuadLists {
  unsigned char idx[4][256];
  int cnt[4];
  int wcnt[4][4];
};

// All 256 threads call this with their staged entry's mask (0 if none); it
// synchronises twice and leaves L ready to read.
__device__ __forceinline__ void build_quad_lists(QuadLists &L, unsigned mask) {
  const unsigned tid = threadIdx.x, lane = tid & 63u, sw = tid >> 6;
  const uint64_t below = lane ? (~0ull >> (64u - lane)) : 0ull;
  unsigned rank[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint64_t b = __builtin_amdgcn_ballot_w64(((mask >> q) & 1u) != 0u);
    rank[q] = (unsigned)__popcll(b & below);
    if (lane == 0) L.wcnt[sw][q] = __popcll(b);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; q++) {
    if ((mask >> q) & 1u) {
      int off = 0;
      for (unsigned s2 = 0; s2 < sw; s2++) off += L.wcnt[s2][q];
      L.idx[q][off + rank[q]] = (unsigned char)tid;
    }
  }
  if (tid < 4) L.cnt[tid] = L.wcnt[0][tid] + L.wcnt[1][tid] + L.wcnt[2][tid] + L.wcnt[3][tid];
  __syncthreads();
}

// Which 4x4 blocks of the tile at (x0, y0) the pixel rectangle of d reaches:
// bit 4 w + g for block g of wave w's quadrant (as in tile_pixel).
__device__ __forceinline__ unsigned block_mask(const TilePix &tp, const DrawRec &d) {
  const int x0 = (int)tp.x0, y0 = (int)tp.y0;
  unsigned cm = 0, rm = 0;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    cm |= (unsigned)((d.i0 <= x0 + 4 * c + 3) & (d.i1 >= x0 + 4 * c)) << c;
    rm |= (unsigned)((d.j0 <= y0 + 4 * c + 3) & (d.j1 >= y0 + 4 * c)) << c;
  }
  unsigned m = 0;
#pragma unroll
  for (int ry = 0; ry < 4; ry++)
#pragma unroll
    for (int cx = 0; cx < 4; cx++) {
      const int bit = 4 * ((cx >> 1) + 2 * (ry >> 1)) + (cx & 1) + 2 * (ry & 1);
      m |= ((cm >> cx) & (rm >> ry) & 1u) << bit;
    }
  return m;
}

// Per-block lists of the staged batch (in batch order): each 16-lane group then
// walks only the entries that reach its 4x4 block.
template <int B>
struct BlockLists {
  unsigned char idx[16][B];   // B: entries staged per batch
  int cnt[16];
  int woff[4][16];        // per wave: first slot of its entries in each list
};

// All 256 threads call this with their staged entry's mask (0 if none); it
// synchronises three times and leaves L ready to read.
template <int B>
__device__ __forceinline__ void build_block_lists(BlockLists<B> &L, unsigned mask) {
  const unsigned tid = threadIdx.x, lane = tid & 63u, sw = tid >> 6;
  const uint64_t below = lane ? (~0ull >> (64u - lane)) : 0ull;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const uint64_t b = __builtin_amdgcn_ballot_w64(((mask >> q) & 1u) != 0u);
    if (lane == 0) L.woff[sw][q] = __popcll(b);
  }
  __syncthreads();
  if (tid < 16) {
    int run = 0;
#pragma unroll
    for (int s2 = 0; s2 < 4; s2++) {
      const int c = L.woff[s2][tid];
      L.woff[s2][tid] = run;
      run += c;
    }
    L.cnt[tid] = run;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const uint64_t b = __builtin_amdgcn_ballot_w64(((mask >> q) & 1u) != 0u);
    if ((mask >> q) & 1u) L.idx[q][L.woff[sw][q] + __popcll(b & below)] = (unsigned char)tid;
  }
  __syncthreads();
}

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
// Spheres: D = 1 - dist^2 / r_eff^2 with dist the orthogonal distance from the
// sphere centre q to the pixel ray d = (x, y, 1). With a = q / qz and
// A = qz^2 / r_eff^2,
//   dist^2 / r_eff^2 = A |a x d|^2 / |d|^2,  so  D = g (|d|^2 - A |a x d|^2),
// g = 1 / |d|^2. Both |d|^2 and |a x d|^2 are quadratic in the pixel offset
// (X, Y) from the tile centre, so per (tile, sphere) the staging thread forms
//   D / g = Q0 + Q1 X + Q2 Y + Q3 X^2 + Q4 X Y + Q5 Y^2
// and each pixel evaluates it with five fp64 FMAs. fp64 matters: across a tile
// the terms reach (8 px / r_px)^2 while near the rim their sum is ~D, and a
// dominant sphere's weight is proportional to D there. On CDNA4 an fp64 FMA
// issues at the non-packed fp32 rate.
// Orthographic views: the pixel's ray runs along +z through (x, y, 0), the
// record holds a = (qx, qy) and A = 1 / r_eff^2, and D = 1 - A |(x, y) - a|^2,
// the same quadratic with g = 1.
// ---------------------------------------------------------------------------
struct SphereRay {
  double x, y;       // (x, y) = ((px - cx) / fx, (py - cy) / fy): the ray direction
                     // (x, y, 1) (pinhole) or the ray origin (x, y, 0) (orthographic)
  double g;          // 1 / (1 + x^2 + y^2) (pinhole), 1 (orthographic)
  double X, Y;       // pixel centre minus tile centre (pixels)
};

__device__ __forceinline__ SphereRay sphere_ray(const ViewDev &c, const TilePix &tp) {
  SphereRay r;
  const double ifx = c.ifx, ify = c.ify;
  r.x = ((double)tp.i + 0.5 - (double)c.cx) * ifx;
  r.y = ((double)tp.j + 0.5 - (double)c.cy) * ify;
  r.g = c.kind == SPLAT_CAM_ORTHOGRAPHIC ? 1.0 : 1.0 / (1.0 + r.x * r.x + r.y * r.y);
  r.X = (double)tp.pxr - 8.0;
  r.Y = (double)tp.pyr - 8.0;
  return r;
}

struct SphereQuad {
  double2 q01, q23, q45;
};

// Coefficients of D / g over the tile of tp (d: the sphere's draw record).
__device__ __forceinline__ SphereQuad sphere_quad(const ViewDev &c, const TilePix &tp, const DrawRec &d) {
  const double ifx = c.ifx, ify = c.ify;
  const double xc = ((double)tp.x0 + 8.0 - (double)c.cx) * ifx;     // tile-centre ray
  const double yc = ((double)tp.y0 + 8.0 - (double)c.cy) * ify;
  const double ax = d.u, ay = d.v, A = d.a;
  if (c.kind == SPLAT_CAM_ORTHOGRAPHIC) {
    // D = 1 - A ((xc - ax + X / fx)^2 + (yc - ay + Y / fy)^2)
    const double ex = xc - ax, ey = yc - ay;
    SphereQuad q;
    q.q01.x = 1.0 - A * (ex * ex + ey * ey);
    q.q01.y = -2.0 * A * ex * ifx;
    q.q23.x = -2.0 * A * ey * ify;
    q.q23.y = -A * ifx * ifx;
    q.q45.x = 0.0;
    q.q45.y = -A * ify * ify;
    return q;
  }
  // a x d = alpha + beta X + gamma Y, component by component
  const double al0 = ay - yc, ga0 = -ify;
  const double al1 = xc - ax, be1 = ifx;
  const double al2 = ax * yc - ay * xc, be2 = -ay * ifx, ga2 = ax * ify;
  SphereQuad q;
  q.q01.x = (1.0 + xc * xc + yc * yc) - A * (al0 * al0 + al1 * al1 + al2 * al2);
  q.q01.y = 2.0 * xc * ifx - 2.0 * A * (al1 * be1 + al2 * be2);
  q.q23.x = 2.0 * yc * ify - 2.0 * A * (al0 * ga0 + al2 * ga2);
  q.q23.y = ifx * ifx - A * (be1 * be1 + be2 * be2);
  q.q45.x = -2.0 * A * (be2 * ga2);
  q.q45.y = ify * ify - A * (ga0 * ga0 + ga2 * ga2);
  return q;
}

// D / g at the pixel.
__device__ __forceinline__ double sphere_num(const SphereRay &r, const double2 q01, const double2 q23,
                                             const double2 q45) {
  double t = __builtin_fma(q23.y, r.X, q01.y);
  t = __builtin_fma(q45.x, r.Y, t);
  double num = __builtin_fma(r.X, t, q01.x);
  const double v = __builtin_fma(q45.y, r.Y, q23.x);
  return __builtin_fma(r.Y, v, num);
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

// Staged conic: (a/2, b) and (c/2, opacity as fp32 bits) with power = (a dx^2 + 2 b dx dy + c dy^2) / 2.
struct Conic {
  double2 ab;
  double2 co;
};

__device__ __forceinline__ Conic stage_conic(const DrawRec &d) {
  Conic k;
  k.ab = make_double2(0.5 * d.a, d.b);
  // opacity as fp32 bits in the low half of the second slot: read back without
  // a conversion per entry
  k.co = make_double2(0.5 * d.c, __builtin_bit_cast(double, (unsigned long long)__float_as_uint(d.w)));
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
  if (LIDAR) {                                    // columns wrap: the nearer image of the centre
    const double half = 0.5 * (double)c.W;
    const double up = dx >= half ? (double)c.W : 0.0, dn = dx < -half ? (double)c.W : 0.0;
    dx = dx - up + dn;                              // selects, no branch; exact (one of them is 0)
  }
  const double power = __builtin_fma(dx, __builtin_fma(ab.x, dx, ab.y * dy), (co.x * dy) * dy);
  G = __expf(-(float)power);
  og = __uint_as_float((unsigned)__builtin_bit_cast(unsigned long long, co.y)) * G;
  return fminf(amax, og);
}

// Spherical views: a batch list entry carries LIST_SEAM when its staged centre
// (stage_uv: already the image of the centre nearest the tile centre) lies
// within 8 columns of half a turn from the tile centre. A pixel of the tile is
// at most 7.5 columns from that centre, so only for such an entry can the
// other image be the nearer one for some pixel; every other entry takes
// splat_alpha without the per-pixel wrap, which would leave it unchanged.
// Pinhole launches of at most SPLIT_TILES_MAX tiles (no more than the chip's
// 256 compute units) with up to four channels composite with the spherical
// views' split walk (four waves per quadrant list, the parts chained per
// pixel): at four waves per tile such a launch leaves most SIMDs idle. With
// more tiles the split costs more than it gains: its workgroup of 1024 threads
// fits once per CU, the parts composite their entries twice in the reverse pass,
// and in the forward pass a part cannot know that its pixels stopped in an
// earlier one (1024 tiles, 100k Gaussians at 512x512: forward 76 -> 273 us).
constexpr int SPLIT_TILES_MAX = 256;
template <int CM>
inline bool split_pinhole(int ntiles) { return CM <= 4 && ntiles <= SPLIT_TILES_MAX; }

constexpr int LIST_SEAM = 0x8000;
__device__ __forceinline__ int seam_flag(const ViewDev &c, double tu) {
  return fabs(tu - 8.0) >= 0.5 * (double)c.W - 8.0 ? LIST_SEAM : 0;
}
