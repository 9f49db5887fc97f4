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
#include <type_traits>

#include "splat_internal.h"

#include "render_common.h"

namespace {

// ---------------------------------------------------------------------------
// Spheres
// ---------------------------------------------------------------------------
// TOPD: record each pixel's top_k contributing spheres of smallest entry depth
// (sensor z where the ray enters the sphere) instead of the first top_k.
// MS: max-shifted blending. The records hold lambda = ln(o exp(o zhat / gamma))
// and beta = ln(bound); each pixel keeps its sums relative to exp(m), m the
// largest lambda so far (at least 0), rescaling them when a contributing sphere
// raises m, and tests the stop in the log domain: beta - ln tau < m + ln N.
template <int CM, bool TOPD, bool MS>
// (closest-K recording holds its list in registers and LDS: four waves per SIMD)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CM <= 4 ? (TOPD ? 4 : 6) : 1))) void k_fwd_sphere(
    ViewTable vt, FwdArgs A) {
  // One staged entry = NE 16-byte slots at a common stride, so every read of an
  // entry uses one LDS address with constant offsets: three slots of D / g
  // coefficients (fp64 pairs), then (o exp(o zhat / gamma), stop limit bound /
  // tau, features...) in fp32.
  constexpr int NF4 = (CM + 2 + 3) / 4;
  // closest-K recording adds one slot: (qz, ax, ay, r_eff), with a = 0 for
  // orthographic views, so that the entry depth is g (qz (a.d) - r_eff sqrt(D / g))
  constexpr int NE = 3 + NF4 + (TOPD ? 1 : 0);
  __shared__ float4 s_e[NE][256];
  __shared__ BlockLists<256> s_l;
  if ((int)blockIdx.x >= vt.total_tiles) {
    // one of FWD_CLEAR_BLOCKS workgroups after the tiles': clear the reverse
    // pass's sums (the reverse pass then skips its clearing). Dispatched last,
    // they run on the CUs that the longest tiles leave idle at the end. They
    // clear even after a pair overflow, so that the caller's word that the sums
    // are clear always holds.
    const int cb = (int)blockIdx.x - vt.total_tiles;
    const long long nthr = (long long)FWD_CLEAR_BLOCKS * blockDim.x;
    const long long t0 = (long long)cb * blockDim.x + threadIdx.x;
#pragma unroll
    for (int r = 0; r < 3; r++)
      for (long long k = t0; k < A.nclr[r]; k += nthr) A.clr[r][k] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  if (*A.overflow) return;
  const int gtile = blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  const SphereRay ray = sphere_ray(c, tp);
  const float gf = (float)ray.g;
  const int wq = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // this wave's quadrant
  const int sb = wq * 4 + (int)((threadIdx.x >> 4) & 3u);                  // this lane's 4x4 block
  const float tau = A.tau;
  float N = A.bg_weight;
  float msh = 0.0f;                              // MS: the shift m
  float lgn = MS ? __logf(A.bg_weight) : 0.0f;  // MS: m + ln N
  float S[CM];
#pragma unroll
  for (int ch = 0; ch < CM; ch++) S[ch] = A.bg_weight * A.bg[ch];
  const int K = A.top_k;
  int ntop = 0;
  // still recording contributing spheres (straight into the top-K buffer)
  bool need = K > 0 && A.topk != nullptr && tp.inside;
  int *my_top = need ? A.topk + (c.pix_off + (long long)tp.j * c.W + tp.i) * K : nullptr;
  // closest-K: the best top_k (entry depth, list position) so far, ascending;
  // slots from K on hold -inf and never change
  float bz[TOPD ? SPLAT_TOPK_MAX : 1];
  uint32_t bp[TOPD ? SPLAT_TOPK_MAX : 1];
  if constexpr (TOPD) {
#pragma unroll
    for (int j = 0; j < SPLAT_TOPK_MAX; j++) {
      bz[j] = j < K ? __builtin_huge_valf() : -__builtin_huge_valf();
      bp[j] = 0xffffffffu;
    }
  }
  const bool orth = c.kind == SPLAT_CAM_ORTHOGRAPHIC;
  bool active = tp.inside;
  const long long vbase = (long long)view * A.n;
  // list entries are read one batch ahead: the record gathers of a batch then
  // wait for one load, not two in a row
  uint32_t rid_next = start + threadIdx.x < end ? A.vals[start + threadIdx.x] : 0u;

  for (uint32_t b = start; b < end; b += 256) {
    const uint32_t e = b + threadIdx.x;
    const uint32_t rid_cur = rid_next;
    if (e + 256u < end) rid_next = A.vals[e + 256u];
    unsigned mask = 0;
    if (e < end) {
      const uint32_t rid = rid_cur;
      const DrawRec d = A.draw[rid];
      const long long id = (long long)rid - vbase;
      const SphereQuad q = sphere_quad(c, tp, d);
      s_e[0][threadIdx.x] = __builtin_bit_cast(float4, q.q01);
      s_e[1][threadIdx.x] = __builtin_bit_cast(float4, q.q23);
      s_e[2][threadIdx.x] = __builtin_bit_cast(float4, q.q45);
      float t[4 * NF4];
      // stop when bound < tau N, i.e. N > bound / tau (never when tau = 0);
      // MS: lambda, and beta - ln tau against m + ln N
      t[0] = d.w;
      if constexpr (MS)
        t[1] = tau > 0.0f ? d.e - __logf(tau) : __builtin_huge_valf();
      else
        t[1] = tau > 0.0f ? d.e / tau : __builtin_huge_valf();
#pragma unroll
      for (int ch = 0; ch < 4 * NF4 - 2; ch++) {
        if constexpr (CM <= SPLAT_REC_FEAT)
          t[2 + ch] = ch < CM ? rec_feat(d, ch) : 0.0f;       // here C = CM: features in the record
        else
          t[2 + ch] = ch < CM && ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
      }
#pragma unroll
      for (int f = 0; f < NF4; f++) s_e[3 + f][threadIdx.x] = make_float4(t[4 * f], t[4 * f + 1], t[4 * f + 2], t[4 * f + 3]);
      if constexpr (TOPD) {
        const AuxRec ax = A.aux[rid];
        s_e[3 + NF4][threadIdx.x] = make_float4(ax.z, orth ? 0.0f : (float)d.u, orth ? 0.0f : (float)d.v, ax.w);
      }
      mask = block_mask(tp, d);
    }
    build_block_lists(s_l, mask);
    // Each 16-lane group walks the list of its own 4x4 block, so one step of
    // the wave handles up to four different entries. cmin / cmax: shortest and
    // longest of the wave's four lists (uniform).
    const int cnt = s_l.cnt[sb];
    const int c0 = s_l.cnt[4 * wq], c1 = s_l.cnt[4 * wq + 1], c2 = s_l.cnt[4 * wq + 2], c3 = s_l.cnt[4 * wq + 3];
    const int cmin = __builtin_amdgcn_readfirstlane(min(min(c0, c1), min(c2, c3)));
    const int cmax = __builtin_amdgcn_readfirstlane(max(max(c0, c1), max(c2, c3)));
    const unsigned char *lst = s_l.idx[sb];
    // One pass over four entries; REC: some lane of the wave still records its
    // first contributing spheres (only the first few hits of each pixel do).
    // FULL: all four entries exist in every group's list; otherwise a lane past
    // its list's end reads staged slot 0 (always filled, finite) and is masked.
    auto four_entries = [&](auto REC, auto FULL, int k, uint32_t four) {
#pragma unroll
      for (int u = 0; u < 4; u++) {
        bool valid = true;
        int idx = (int)((four >> (8 * u)) & 0xffu);
        if constexpr (!decltype(FULL)::value) {
          if (k + u >= cmax) break;
          valid = k + u < cnt;
          idx = valid ? idx : 0;
        }
        float t[4 * NF4];
#pragma unroll
        for (int f = 0; f < NF4; f++) {
          const float4 x = s_e[3 + f][idx];
          t[4 * f] = x.x; t[4 * f + 1] = x.y; t[4 * f + 2] = x.z; t[4 * f + 3] = x.w;
        }
        // no later sphere can matter (& : no short-circuit branch)
        if constexpr (MS)
          active = active & !(valid & (t[1] < lgn));
        else
          active = active & !(valid & (N > t[1]));
        const double num = sphere_num(ray, __builtin_bit_cast(double2, s_e[0][idx]),
                                      __builtin_bit_cast(double2, s_e[1][idx]),
                                      __builtin_bit_cast(double2, s_e[2][idx]));
        // D / g past the five fp64 FMAs goes to fp32: the sign test and the
        // weight's product run at the fp32 rate (the sign is the fp64 one except
        // for 0 < D / g < 1.4e-45, which rounds to zero)
        float numf = (float)num;
        asm volatile("" : "+v"(numf));                    // keeps the compiler from testing num instead
        const bool hit = active & valid & (numf > 0.0f);
        if constexpr (MS) {
          if (ballot64(hit)) {
            const float sh = hit ? fmaxf(msh, t[0]) : msh;
            const float rs = __expf(msh - sh);             // 1 unless the shift rises
            // a select, not a 0/1 factor: a lane without a hit may hold lambda > m
            const float w = hit ? __expf(t[0] - sh) * (numf * gf) : 0.0f;
            N = __builtin_fmaf(N, rs, w);
#pragma unroll
            for (int ch = 0; ch < CM; ch++) S[ch] = __builtin_fmaf(w, t[2 + ch], S[ch] * rs);
            msh = sh;
            lgn = hit ? msh + __logf(N) : lgn;
          }
        } else {
          // the weight is formed on every lane (the empty asm keeps the compiler
          // from moving it under a branch) and selected: straight-line code
          float wx = t[0] * (numf * gf);
          asm volatile("" : "+v"(wx));
          const float w = hit ? wx : 0.0f;
          N += w;
#pragma unroll
          for (int ch = 0; ch < CM; ch++) S[ch] = __builtin_fmaf(w, t[2 + ch], S[ch]);
        }
        if constexpr (decltype(REC)::value) {
          const bool rec = hit & need;
          if constexpr (TOPD) {
            const float4 g4 = s_e[3 + NF4][idx];            // qz, ax, ay, r_eff
            if (ballot64(rec)) {
              if (rec) {
                const float ad = __builtin_fmaf(g4.y, (float)ray.x, __builtin_fmaf(g4.z, (float)ray.y, 1.0f));
                float z = (float)ray.g * (g4.x * ad - g4.w * sqrtf((float)num));
                uint32_t pz = b + (uint32_t)idx;
                // insertion: a strictly closer entry displaces (earlier positions win ties)
#pragma unroll
                for (int j = 0; j < SPLAT_TOPK_MAX; j++) {
                  const bool sw = z < bz[j];
                  const float tz = bz[j];
                  const uint32_t tq = bp[j];
                  bz[j] = sw ? z : tz;
                  bp[j] = sw ? pz : tq;
                  z = sw ? tz : z;
                  pz = sw ? tq : pz;
                }
              }
            }
            // no later entry can come closer once the K-th best lies in front of
            // this entry's front depth (later fronts are not nearer; margin for
            // the rounding of the key and of the entry depths)
            float kth = bz[0];
#pragma unroll
            for (int j = 1; j < SPLAT_TOPK_MAX; j++) kth = fmaxf(kth, bz[j]);
            need = need & !(valid & active & (kth < (g4.x - g4.w) * (1.0f - 1e-5f)));
          } else {
            if (ballot64(rec)) {                   // most entries record nothing
              if (rec) {
                my_top[ntop] = (int)(b + (uint32_t)idx);
                ntop++;
                need = ntop < K;
              }
            }
          }
        }
      }
    };
    if (ballot64(active)) {
      bool recording = ballot64(need && active) != 0;
      const int cmin4 = cmin & ~3;
      int k = 0;
      for (; k < cmin4; k += 4) {
        const uint32_t four = *reinterpret_cast<const uint32_t *>(lst + k);
        if (recording) {
          four_entries(std::true_type{}, std::true_type{}, k, four);
          recording = ballot64(need && active) != 0;
        } else {
          four_entries(std::false_type{}, std::true_type{}, k, four);
        }
        if (ballot64(active) == 0) break;
      }
      if (k == cmin4) {                          // the groups' remaining entries
        for (; k < cmax && ballot64(active); k += 4) {
          const uint32_t four = *reinterpret_cast<const uint32_t *>(lst + k);
          four_entries(std::true_type{}, std::false_type{}, k, four);
        }
      }
    }
    if (__syncthreads_count(active) == 0) break;
  }
  // the pixel again from the thread index: nothing of it stays live over the walk
  // (kept live, it spilled to scratch)
  const TilePix tq = tile_pixel(c, gtile, threadIdx.x);
  if (!tq.inside) return;
  const long long p = c.pix_off + (long long)tq.j * c.W + tq.i;
  const size_t plane = (size_t)c.W * c.H;
  float *img = A.img + c.img_off + (size_t)tq.j * c.W + tq.i;
  const float inv = 1.0f / N;
#pragma unroll
  for (int ch = 0; ch < CM; ch++)
    if (ch < A.C) img[ch * plane] = S[ch] * inv;
  if (A.norm) A.norm[p] = N;
  if constexpr (MS) {
    if (A.T_final) A.T_final[p] = msh;
  }
  if constexpr (TOPD) {
    if (A.topk) {
      // list order: sort the positions (empty slots, 0xffffffff, go last)
#pragma unroll
      for (int a = 0; a < SPLAT_TOPK_MAX; a++)
#pragma unroll
        for (int j = 0; j + 1 < SPLAT_TOPK_MAX - a; j++) {
          const uint32_t lo = min(bp[j], bp[j + 1]), hi = max(bp[j], bp[j + 1]);
          bp[j] = lo;
          bp[j + 1] = hi;
        }
#pragma unroll
      for (int q = 0; q < SPLAT_TOPK_MAX; q++)
        if (q < K) A.topk[p * K + q] = bp[q] == 0xffffffffu ? -1 : (int)bp[q];
    }
  } else if (A.topk) {
    for (int q = ntop; q < K; q++) A.topk[p * K + q] = -1;
  }
}

// ---------------------------------------------------------------------------
// Gaussian splats (alpha blending) in pinhole views.
// ---------------------------------------------------------------------------
template <int CM>
__global__ __launch_bounds__(256) void k_fwd_alpha(ViewTable vt, FwdArgs A, int tile_begin) {
  constexpr int NF = CM;
  // features [entry][channel], read as 16-byte pieces (one read per four
  // channels); from eight channels on the row stride has four floats more, so
  // that the staging writes of neighbouring entries spread over the banks
  constexpr int NF4 = (NF + 3) / 4;
  constexpr int FS = 4 * NF4 + (NF >= 8 ? 4 : 0);
  __shared__ double2 s_uv[256];     // tile-relative centre
  __shared__ double2 s_ab[256];     // a/2, b
  __shared__ double2 s_co[256];     // c/2, opacity
  __shared__ __align__(16) float s_f[256][FS];
  __shared__ QuadLists s_l;
  if (*A.overflow) return;
  const int gtile = tile_begin + (int)blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  if (c.kind == SPLAT_CAM_SPHERICAL) return;
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  const int wq = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // this wave's quadrant
  // Transmittance runs in fp64 (same issue rate as fp32 on CDNA4): it is the
  // product of every (1 - alpha) so far and the backward divides it back out.
  double T = 1.0;
  float S[NF];
#pragma unroll
  for (int ch = 0; ch < NF; ch++) S[ch] = 0.0f;
  uint32_t last = 0;
  bool active = tp.inside;
  const long long vbase = (long long)view * A.n;
  const float amin = A.alpha_min, amax = A.alpha_max;
  const double tmin = (double)A.T_min;
  const double pxr = tp.pxr, pyr = tp.pyr;

  for (uint32_t b = start; b < end; b += 256) {
    const uint32_t e = b + threadIdx.x;
    unsigned mask = 0;
    if (e < end) {
      const uint32_t rid = A.vals[e];
      const DrawRec d = A.draw[rid];
      s_uv[threadIdx.x] = stage_uv(c, tp, d, false);
      const Conic cn = stage_conic(d);
      s_ab[threadIdx.x] = cn.ab;
      s_co[threadIdx.x] = cn.co;
      const long long id = (long long)rid - vbase;
#pragma unroll
      for (int q = 0; q < NF4; q++) {
        float f[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const int ch = 4 * q + k;
          f[k] = ch < NF && ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
        }
        *reinterpret_cast<float4 *>(&s_f[threadIdx.x][4 * q]) = make_float4(f[0], f[1], f[2], f[3]);
      }
      mask = quadrant_mask(tp, d);
    }
    build_quad_lists(s_l, mask);
    // the list, its length and every index are the same for the whole wave
    const int cnt = __builtin_amdgcn_readfirstlane(s_l.cnt[wq]);
    // one entry: straight-line code (non-short-circuit tests, the weight a 0/1
    // factor times a finite product)
    auto one = [&](int idx) {
      float G, og;
      double dx, dy;
      const float al = splat_alpha<false>(c, pxr, pyr, s_uv[idx], s_ab[idx], s_co[idx], amax, G, og, dx, dy);
      const bool hit = active & (al >= amin);
      if (ballot64(hit) == 0) return;            // no pixel of the wave takes it: nothing changes
      const float w = (hit ? 1.0f : 0.0f) * (float)(T * (double)al);
#pragma unroll
      for (int q = 0; q < NF4; q++) {
        const float4 f = *reinterpret_cast<const float4 *>(&s_f[idx][4 * q]);
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (4 * q + k < NF) S[4 * q + k] = __builtin_fmaf(w, fv[k], S[4 * q + k]);
      }
      T = hit ? T * (1.0 - (double)al) : T;
      last = hit ? b - start + (uint32_t)idx + 1u : last;
      active = active & !(T < tmin);            // include, then stop
    };
    if (NF > 8) {
      // many channels: one entry per step keeps the staged features out of registers
      if (ballot64(active))
        for (int k = 0; k < cnt; k++) {
          one(__builtin_amdgcn_readfirstlane((int)s_l.idx[wq][k]));
          if ((k & 3) == 3 && ballot64(active) == 0) break;
        }
    } else if (ballot64(active)) {
      const int cnt4 = cnt & ~3;
      bool live = true;
      for (int k = 0; k < cnt4; k += 4) {
        const uint32_t four =
            __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t *>(&s_l.idx[wq][k]));
        one((int)(four & 0xffu));
        one((int)((four >> 8) & 0xffu));
        one((int)((four >> 16) & 0xffu));
        one((int)(four >> 24));
        if (ballot64(active) == 0) {
          live = false;
          break;
        }
      }
      if (live)
        for (int k = cnt4; k < cnt; k++) one(__builtin_amdgcn_readfirstlane((int)s_l.idx[wq][k]));
    }
    if (__syncthreads_count(active) == 0) break;
  }
  if (!tp.inside) return;
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  float *img = A.img + c.img_off + (size_t)tp.j * c.W + tp.i;
#pragma unroll
  for (int ch = 0; ch < CM; ch++)
    if (ch < A.C) img[ch * plane] = S[ch];
  if (A.T_final) A.T_final[p] = (float)T;
  if (A.last) A.last[p] = last;
}

// ---------------------------------------------------------------------------
// Spherical (lidar) views: long tile lists split four ways inside the tile.
// A range view's tiles hold lists tens of thousands of entries long, and a ray
// that sees sky walks thousands of them before (if ever) its transmittance
// stops it; with one wave per 8x8 quadrant the few longest tiles set the
// kernel's time. Here a workgroup of 1024 threads stages 1024 entries per
// batch, and four waves share each quadrant: the wave quadrant list is cut
// into four consecutive parts, each walked from T = 1 (partial colour S_j,
// transmittance T_j, last entry). The parts are then chained per pixel:
// S += T S_j, T *= T_j, as long as T T_j stays at or above T_min (T is
// non-increasing along a part, so no entry of it can have stopped the pixel).
// Otherwise the stop lies inside part j, and its wave walks that part again
// from the chained T and S with the ordinary per-entry stop.
// SPH = false: the same walk for pinhole views with up to four channels, for
// launches with few tiles (their four waves per tile left most SIMDs idle or
// waiting for the last tiles).
// ---------------------------------------------------------------------------
constexpr int LB = 1024;                 // threads and staged entries per batch

template <int CM, bool SPH>
__global__ __launch_bounds__(LB) void k_fwd_split(ViewTable vt, FwdArgs A, int tile_begin) {
  constexpr int NF = SPH ? 1 : CM;       // composited values: range, or the features
  __shared__ double2 s_uv[LB];           // tile-relative centre
  __shared__ double2 s_ab[LB];           // a/2, b
  __shared__ double2 s_co[LB];           // c/2, opacity
  __shared__ float s_f[NF][LB];          // range or features
  __shared__ uint16_t s_idx[4][LB];      // per-quadrant lists of the batch
  __shared__ int s_woff[16][4];          // per wave: first slot of its entries in each list
  __shared__ int s_cnt[4];
  __shared__ float s_pS[4][NF][256];     // per part and pixel: partial colour,
  __shared__ double s_pT[4][256];        //   transmittance,
  __shared__ uint32_t s_pL[4][256];      //   last composited entry (0: none)
  if (*A.overflow) return;
  const int gtile = tile_begin + (int)blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  if ((c.kind == SPLAT_CAM_SPHERICAL) != SPH) return;
  const unsigned tid = threadIdx.x, pix = tid & 255u;
  const int part = __builtin_amdgcn_readfirstlane((int)(tid >> 8));           // 0..3
  const int wq = __builtin_amdgcn_readfirstlane((int)((tid >> 6) & 3u));     // quadrant
  const unsigned lane = tid & 63u, sw = tid >> 6;
  const TilePix tp = tile_pixel(c, gtile, pix);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  // running state of this thread's pixel (the same in all four copies)
  double T = 1.0;
  float S[NF];
#pragma unroll
  for (int ch = 0; ch < NF; ch++) S[ch] = 0.0f;
  uint32_t last = 0;
  bool active = tp.inside;
  const float amin = A.alpha_min, amax = A.alpha_max;
  const double tmin = (double)A.T_min;
  const double pxr = tp.pxr, pyr = tp.pyr;
  const long long vbase = (long long)view * A.n;

  for (uint32_t b = start; b < end; b += LB) {
    const uint32_t e = b + tid;
    unsigned mask = 0;
    int seam = 0;
    if (e < end) {
      const uint32_t rid = A.vals[e];
      const DrawRec d = A.draw[rid];
      const double2 uv = stage_uv(c, tp, d, SPH);
      s_uv[tid] = uv;
      if constexpr (SPH) seam = seam_flag(c, uv.x);
      const Conic cn = stage_conic(d);
      s_ab[tid] = cn.ab;
      s_co[tid] = cn.co;
      if constexpr (SPH) {
        s_f[0][tid] = A.aux[rid].z;
      } else {
        const long long id = (long long)rid - vbase;
#pragma unroll
        for (int ch = 0; ch < NF; ch++) s_f[ch][tid] = ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
      }
      mask = quadrant_mask(tp, d);
    }
    // per-quadrant lists, in batch order
    const uint64_t below = lane ? (~0ull >> (64u - lane)) : 0ull;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint64_t bq = ballot64(((mask >> q) & 1u) != 0u);
      if (lane == 0) s_woff[sw][q] = __popcll(bq);
    }
    __syncthreads();
    if (tid < 4) {
      int run = 0;
      for (int w2 = 0; w2 < 16; w2++) {
        const int x = s_woff[w2][tid];
        s_woff[w2][tid] = run;
        run += x;
      }
      s_cnt[tid] = run;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint64_t bq = ballot64(((mask >> q) & 1u) != 0u);
      if ((mask >> q) & 1u) s_idx[q][s_woff[sw][q] + __popcll(bq & below)] = (uint16_t)((int)tid | seam);
    }
    __syncthreads();
    // this wave's part of its quadrant's list (entries: staged index | LIST_SEAM)
    const int L = __builtin_amdgcn_readfirstlane(s_cnt[wq]);
    const int k0 = (L * part) / 4, k1 = (L * (part + 1)) / 4;
    auto one = [&](int ie, double &Tx, float (&Sx)[NF], uint32_t &lx, bool &ax) {
      const int idx = ie & (LIST_SEAM - 1);
      float G, og, al;
      double dx, dy;
      if (SPH && (ie & LIST_SEAM))                     // wave-uniform
        al = splat_alpha<true>(c, pxr, pyr, s_uv[idx], s_ab[idx], s_co[idx], amax, G, og, dx, dy);
      else
        al = splat_alpha<false>(c, pxr, pyr, s_uv[idx], s_ab[idx], s_co[idx], amax, G, og, dx, dy);
      const bool hit = ax & (al >= amin);
      if (ballot64(hit) == 0) return;            // no pixel of the wave takes it: nothing changes
      const float w = (hit ? 1.0f : 0.0f) * (float)(Tx * (double)al);
#pragma unroll
      for (int ch = 0; ch < NF; ch++) Sx[ch] = __builtin_fmaf(w, s_f[ch][idx], Sx[ch]);
      Tx = hit ? Tx * (1.0 - (double)al) : Tx;
      lx = hit ? b - start + (uint32_t)idx + 1u : lx;
      ax = ax & !(Tx < tmin);
    };
    // the wave's walk over list positions [k0, k1): single entries up to a
    // multiple of four, then four indices per LDS read (their records are
    // read ahead of the dependent arithmetic), until no lane is left
    auto walk = [&](double &Tx, float (&Sx)[NF], uint32_t &lx, bool &ax) {
      int k = k0;
      for (; k < k1 && (k & 3); k++) one(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]), Tx, Sx, lx, ax);
      for (; k + 4 <= k1; k += 4) {
        if (ballot64(ax) == 0) return;
        const uint64_t four = *reinterpret_cast<const uint64_t *>(&s_idx[wq][k]);
        const uint32_t lo4 = __builtin_amdgcn_readfirstlane((uint32_t)four);
        const uint32_t hi4 = __builtin_amdgcn_readfirstlane((uint32_t)(four >> 32));
        one((int)(lo4 & 0xffffu), Tx, Sx, lx, ax);
        one((int)(lo4 >> 16), Tx, Sx, lx, ax);
        one((int)(hi4 & 0xffffu), Tx, Sx, lx, ax);
        one((int)(hi4 >> 16), Tx, Sx, lx, ax);
      }
      for (; k < k1; k++) one(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]), Tx, Sx, lx, ax);
    };
    // 1. the part from T = 1 (a local stop below T_min ends it: the chained T is smaller)
    {
      double Tj = 1.0;
      float Sj[NF];
#pragma unroll
      for (int ch = 0; ch < NF; ch++) Sj[ch] = 0.0f;
      uint32_t lj = 0;
      bool aj = active;
      walk(Tj, Sj, lj, aj);
#pragma unroll
      for (int ch = 0; ch < NF; ch++) s_pS[part][ch][pix] = Sj[ch];
      s_pT[part][pix] = Tj;
      s_pL[part][pix] = lj;
    }
    __syncthreads();
    // 2. chain the parts (every copy of the pixel computes the same)
    int stop_part = -1;
    if (active) {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (stop_part < 0) {
          const double Tj = s_pT[j][pix];
          if (T * Tj >= tmin) {
#pragma unroll
            for (int ch = 0; ch < NF; ch++) S[ch] = __builtin_fmaf((float)T, s_pS[j][ch][pix], S[ch]);
            const uint32_t lj = s_pL[j][pix];
            last = lj ? lj : last;
            T *= Tj;
          } else {
            stop_part = j;
          }
        }
      }
    }
    __syncthreads();                               // the partials are read before step 3 reuses them
    // 3. the part holding the stop, walked again from the chained state
    if (ballot64(stop_part == part)) {
      bool ax = stop_part == part;
      double Tx = T;
      float Sx[NF];
#pragma unroll
      for (int ch = 0; ch < NF; ch++) Sx[ch] = S[ch];
      uint32_t lx = last;
      walk(Tx, Sx, lx, ax);
      if (stop_part == part) {
#pragma unroll
        for (int ch = 0; ch < NF; ch++) s_pS[0][ch][pix] = Sx[ch];
        s_pT[0][pix] = Tx;
        s_pL[0][pix] = lx;
      }
    }
    __syncthreads();
    if (stop_part >= 0) {                          // stopped in this batch: final state
#pragma unroll
      for (int ch = 0; ch < NF; ch++) S[ch] = s_pS[0][ch][pix];
      T = s_pT[0][pix];
      last = s_pL[0][pix];
      active = false;
    }
    if (__syncthreads_count(active) == 0) break;
  }
  if (part != 0 || !tp.inside) return;
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  float *img = A.img + c.img_off + (size_t)tp.j * c.W + tp.i;
  if constexpr (SPH) {
    img[0] = S[0];
    img[plane] = (float)(1.0 - T);
  } else {
#pragma unroll
    for (int ch = 0; ch < NF; ch++)
      if (ch < A.C) img[ch * plane] = S[ch];
  }
  if (A.T_final) A.T_final[p] = (float)T;
  if (A.last) A.last[p] = last;
}

// Gaussians given the reverse workspace: the reverse pass's sums cleared with
// 16-byte stores, in a launch on the camera views' stream after their kernel.
// With a spherical view in the call it runs beside the lidar tiles, whose
// longest lists keep the caller's stream busy after the camera views are done.
__global__ __launch_bounds__(256) void k_fwd_clear(FwdArgs A) {
  const long long nthr = (long long)gridDim.x * blockDim.x;
  const long long t0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int r = 0; r < 3; r++)
    for (long long k = t0; k < A.nclr[r]; k += nthr) A.clr[r][k] = make_uint4(0u, 0u, 0u, 0u);
}

template <int CM>
int launch_fwd_cm(const ViewTable &vt, const FwdArgs &A, int kind, hipStream_t stream) {
  dim3 grid(vt.total_tiles), block(256);
  if (kind == SPLAT_PRIM_SPHERE && A.clear) grid.x += FWD_CLEAR_BLOCKS;
  if (kind == SPLAT_PRIM_SPHERE) {
    if (A.top_by_depth && A.max_shift)
      hipLaunchKernelGGL((k_fwd_sphere<CM, true, true>), grid, block, 0, stream, vt, A);
    else if (A.top_by_depth)
      hipLaunchKernelGGL((k_fwd_sphere<CM, true, false>), grid, block, 0, stream, vt, A);
    else if (A.max_shift)
      hipLaunchKernelGGL((k_fwd_sphere<CM, false, true>), grid, block, 0, stream, vt, A);
    else
      hipLaunchKernelGGL((k_fwd_sphere<CM, false, false>), grid, block, 0, stream, vt, A);
  } else {
    // one launch per run of consecutive views of one kind, over that run's
    // tiles only. With both kinds present the camera views run on the side
    // stream, which first waits for an event of the caller's stream: the
    // spherical views, launched on the caller's stream, are dispatched first
    // (all their workgroups are resident at once), so their long lists start
    // early and camera tiles fill the compute units they leave
    bool has_pin = false, has_sph = false;
    for (int v = 0; v < vt.n; v++) (vt.v[v].kind == SPLAT_CAM_SPHERICAL ? has_sph : has_pin) = true;
    hipStream_t side = stream;
    const bool fork = has_pin && has_sph && !A.serial_views;
    if (fork) {
      const int rc = side_begin(stream, &side);
      if (rc != SPLAT_OK) return rc;
    }
    for (int pass = 0; pass < 2; pass++) {
      for (int v0 = 0; v0 < vt.n;) {
        const int kind0 = vt.v[v0].kind;
        int v1 = v0 + 1;
        while (v1 < vt.n && vt.v[v1].kind == kind0) v1++;
        const int t0 = vt.v[v0].tile_off, t1 = v1 < vt.n ? vt.v[v1].tile_off : vt.total_tiles;
        if (t1 > t0) {
          if (pass == 0 && kind0 == SPLAT_CAM_SPHERICAL)
            hipLaunchKernelGGL((k_fwd_split<1, true>), dim3(t1 - t0), dim3(LB), 0, stream, vt, A, t0);
          else if (pass == 1 && kind0 != SPLAT_CAM_SPHERICAL && split_pinhole<CM>(t1 - t0))
            hipLaunchKernelGGL((k_fwd_split<CM <= 4 ? CM : 4, false>), dim3(t1 - t0), dim3(LB), 0, side, vt, A, t0);
          else if (pass == 1 && kind0 != SPLAT_CAM_SPHERICAL)
            hipLaunchKernelGGL(k_fwd_alpha<CM>, dim3(t1 - t0), block, 0, side, vt, A, t0);
        }
        v0 = v1;
      }
    }
    if (A.clear) hipLaunchKernelGGL(k_fwd_clear, dim3(FWD_CLEAR_GRID), dim3(256), 0, has_pin ? side : stream, A);
    if (fork) {
      const int rc = side_end(stream, side);
      if (rc != SPLAT_OK) return rc;
    }
  }
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}

}  // namespace

int launch_render_fwd(const ViewTable &vt, const FwdArgs &A, int kind, hipStream_t stream) {
  if (vt.total_tiles == 0) return SPLAT_OK;
  switch (channel_bucket(A.C)) {
    case 1: return launch_fwd_cm<1>(vt, A, kind, stream);
    case 2: return launch_fwd_cm<2>(vt, A, kind, stream);
    case 3: return launch_fwd_cm<3>(vt, A, kind, stream);
    case 4: return launch_fwd_cm<4>(vt, A, kind, stream);
    case 8: return launch_fwd_cm<8>(vt, A, kind, stream);
    case 16: return launch_fwd_cm<16>(vt, A, kind, stream);
    case 32: return launch_fwd_cm<32>(vt, A, kind, stream);
    case 64: return launch_fwd_cm<64>(vt, A, kind, stream);
  }
  return SPLAT_ERR_UNSUPPORTED;
}
