// Forward compositor: one 256-thread workgroup (four wave64s) per 16x16 tile.
//
// Pulsar appendix B.1.2-B.1.4: pixel-parallel drawing over a per-block list of
// candidate primitives, loaded cooperatively and coalesced into shared memory,
// each pixel accumulating independently, a block-wide vote ending the block once
// every pixel is finished, and a per-pixel backward buffer (normalisation and the
// ids of the first contributing spheres). Gaussian splats use front-to-back alpha
// blending with transmittance termination (the NuRec rendering kernel).
//
// Batches of up to 256 list entries are staged into LDS as 16-byte records; every
// lane of a wave then reads the same LDS address (a broadcast) per entry.
// Positions are made tile-relative while staging and the per-pixel geometry runs
// in fp64 (full rate on CDNA4), so a footprint's rim and an elongated Gaussian's
// quadratic form keep their precision; weights and colours accumulate in fp32.
#include "splat_internal.h"

#include "render_common.h"

namespace {

// ---------------------------------------------------------------------------
// Spheres
// ---------------------------------------------------------------------------
struct __align__(16) SphereWgt {
  double A;      // qz^2 / r_eff^2
  float oe;      // opacity * exp(opacity * zhat / gamma)
  float bnd;     // weight bound of this and every later sphere
};

template <int CM>
__global__ __launch_bounds__(256) void k_fwd_sphere(ViewTable vt, FwdArgs A) {
  __shared__ double2 s_uv[256];     // tile-relative centre (pixels)
  __shared__ double2 s_ax[256];     // normalised centre
  __shared__ SphereWgt s_w[256];
  __shared__ int s_id[256];
  __shared__ float s_f[CM][256];
  if (*A.overflow) return;
  const int gtile = blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  const SphereRay ray = sphere_ray(c, tp);
  const float tau = A.tau;
  float N = A.bg_weight;
  float S[CM];
#pragma unroll
  for (int ch = 0; ch < CM; ch++) S[ch] = A.bg_weight * A.bg[ch];
  int top[SPLAT_TOPK_MAX];
#pragma unroll
  for (int k = 0; k < SPLAT_TOPK_MAX; k++) top[k] = -1;
  int ntop = 0;
  const int K = A.top_k;
  bool done = !tp.inside;
  const long long vbase = (long long)view * A.n;

  for (uint32_t b = start; b < end; b += 256) {
    const uint32_t e = b + threadIdx.x;
    if (e < end) {
      const uint32_t rid = A.vals[e];
      const DrawRec d = A.draw[rid];
      const int id = (int)((long long)rid - vbase);
      const SphereGeo sg = sphere_geo(c, tp, d);
      s_uv[threadIdx.x] = make_double2(sg.u, sg.v);
      s_ax[threadIdx.x] = make_double2(sg.ax, sg.ay);
      SphereWgt w;
      w.A = sg.A; w.oe = d.w; w.bnd = d.e;
      s_w[threadIdx.x] = w;
      s_id[threadIdx.x] = id;
#pragma unroll
      for (int ch = 0; ch < CM; ch++) s_f[ch][threadIdx.x] = ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
    }
    __syncthreads();
    const int cnt = (int)min(256u, end - b);
    if (!done) {
      for (int k = 0; k < cnt; k++) {
        const SphereWgt wg = s_w[k];
        if (wg.bnd < tau * N) { done = true; break; }       // no later sphere can matter
        const double2 uv = s_uv[k];
        const double2 ax = s_ax[k];
        double sx, sy;
        const double D = sphere_D_ex(ray, uv.x, uv.y, ax.x, ax.y, wg.A, sx, sy);
        if (D > 0.0) {
          const float w = wg.oe * (float)D;
          N += w;
#pragma unroll
          for (int ch = 0; ch < CM; ch++) S[ch] = __builtin_fmaf(w, s_f[ch][k], S[ch]);
          if (ntop < K) {
            const int id = s_id[k];
#pragma unroll
            for (int q = 0; q < SPLAT_TOPK_MAX; q++)
              if (q == ntop) top[q] = id;
            ntop++;
          }
        }
      }
    }
    if (__syncthreads_count(!done) == 0) break;
  }
  if (!tp.inside) return;
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  float *img = A.img + c.img_off + (size_t)tp.j * c.W + tp.i;
  const float inv = 1.0f / N;
#pragma unroll
  for (int ch = 0; ch < CM; ch++)
    if (ch < A.C) img[ch * plane] = S[ch] * inv;
  if (A.norm) A.norm[p] = N;
  if (A.topk)
#pragma unroll
    for (int q = 0; q < SPLAT_TOPK_MAX; q++)
      if (q < K) A.topk[p * K + q] = top[q];
}

// ---------------------------------------------------------------------------
// Gaussian splats (alpha blending); LIDAR = spherical view rendering
// expected depth and opacity.
// ---------------------------------------------------------------------------
template <int CM, bool LIDAR>
__global__ __launch_bounds__(256) void k_fwd_alpha(ViewTable vt, FwdArgs A) {
  __shared__ double2 s_uv[256];     // tile-relative centre
  __shared__ double2 s_ab[256];     // a/2, b
  __shared__ double2 s_co[256];     // c/2, opacity
  __shared__ float s_f[LIDAR ? 1 : CM][256];   // features, or depth for spherical views
  if (*A.overflow) return;
  const int gtile = blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  if ((c.kind == SPLAT_CAM_SPHERICAL) != LIDAR) return;
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  // Transmittance runs in fp64 (same issue rate as fp32 on CDNA4): it is the
  // product of every (1 - alpha) so far and the backward divides it back out.
  double T = 1.0;
  float S[LIDAR ? 1 : CM];
#pragma unroll
  for (int ch = 0; ch < (LIDAR ? 1 : CM); ch++) S[ch] = 0.0f;
  float dep = 0.0f;
  uint32_t last = 0;
  bool done = !tp.inside;
  const long long vbase = (long long)view * A.n;
  const float amin = A.alpha_min, amax = A.alpha_max;
  const double tmin = (double)A.T_min;

  const double pxr = tp.pxr, pyr = tp.pyr;

  for (uint32_t b = start; b < end; b += 256) {
    const uint32_t e = b + threadIdx.x;
    if (e < end) {
      const uint32_t rid = A.vals[e];
      const DrawRec d = A.draw[rid];
      s_uv[threadIdx.x] = stage_uv(c, tp, d, LIDAR);
      const Conic cn = stage_conic(d);
      s_ab[threadIdx.x] = cn.ab;
      s_co[threadIdx.x] = cn.co;
      if (LIDAR) {
        s_f[0][threadIdx.x] = A.aux[rid].depth;
      } else {
        const long long id = (long long)rid - vbase;
#pragma unroll
        for (int ch = 0; ch < CM; ch++) s_f[ch][threadIdx.x] = ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
      }
    }
    __syncthreads();
    const int cnt = (int)min(256u, end - b);
    if (!done) {
      for (int k = 0; k < cnt; k++) {
        float G, og;
        double dx, dy;
        const float al = splat_alpha<LIDAR>(c, pxr, pyr, s_uv[k], s_ab[k], s_co[k], amax, G, og, dx, dy);
        if (al < amin) continue;
        const float w = (float)(T * (double)al);
        if (LIDAR) {
          dep = __builtin_fmaf(w, s_f[0][k], dep);
        } else {
#pragma unroll
          for (int ch = 0; ch < CM; ch++) S[ch] = __builtin_fmaf(w, s_f[ch][k], S[ch]);
        }
        T = T * (1.0 - (double)al);
        last = b - start + (uint32_t)k + 1u;
        if (T < tmin) { done = true; break; }
      }
    }
    if (__syncthreads_count(!done) == 0) break;
  }
  if (!tp.inside) return;
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  float *img = A.img + c.img_off + (size_t)tp.j * c.W + tp.i;
  if (LIDAR) {
    img[0] = dep;
    img[plane] = (float)(1.0 - T);
  } else {
#pragma unroll
    for (int ch = 0; ch < CM; ch++)
      if (ch < A.C) img[ch * plane] = S[ch];
  }
  if (A.T_final) A.T_final[p] = (float)T;
  if (A.last) A.last[p] = last;
}

template <int CM>
int launch_fwd_cm(const ViewTable &vt, const FwdArgs &A, int kind, bool has_pin, bool has_sph, hipStream_t stream) {
  dim3 grid(vt.total_tiles), block(256);
  if (kind == SPLAT_PRIM_SPHERE) {
    hipLaunchKernelGGL(k_fwd_sphere<CM>, grid, block, 0, stream, vt, A);
  } else {
    if (has_pin) hipLaunchKernelGGL((k_fwd_alpha<CM, false>), grid, block, 0, stream, vt, A);
    if (has_sph) hipLaunchKernelGGL((k_fwd_alpha<1, true>), grid, block, 0, stream, vt, A);
  }
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}

}  // namespace

int launch_render_fwd(const ViewTable &vt, const FwdArgs &A, int kind, hipStream_t stream) {
  if (vt.total_tiles == 0) return SPLAT_OK;
  bool has_pin = false, has_sph = false;
  for (int v = 0; v < vt.n; v++) {
    if (vt.v[v].kind == SPLAT_CAM_SPHERICAL) has_sph = true;
    else has_pin = true;
  }
  switch (channel_bucket(A.C)) {
    case 1: return launch_fwd_cm<1>(vt, A, kind, has_pin, has_sph, stream);
    case 2: return launch_fwd_cm<2>(vt, A, kind, has_pin, has_sph, stream);
    case 3: return launch_fwd_cm<3>(vt, A, kind, has_pin, has_sph, stream);
    case 4: return launch_fwd_cm<4>(vt, A, kind, has_pin, has_sph, stream);
    case 8: return launch_fwd_cm<8>(vt, A, kind, has_pin, has_sph, stream);
    case 16: return launch_fwd_cm<16>(vt, A, kind, has_pin, has_sph, stream);
    case 32: return launch_fwd_cm<32>(vt, A, kind, has_pin, has_sph, stream);
    case 64: return launch_fwd_cm<64>(vt, A, kind, has_pin, has_sph, stream);
  }
  return SPLAT_ERR_UNSUPPORTED;
}
