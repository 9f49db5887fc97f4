// Backward pass.
//
// Pulsar appendix B.2: pixel-wise backward parallelisation reading the forward
// pass's per-pixel buffer (no new intersection search), gradients only for the
// first few spheres of each pixel, then a sphere-wise pass for the camera
// gradient followed by a device-wide reduction. NuRec's renderBackward is split
// into camera and lidar versions; here the pinhole and spherical views run as
// separate kernel instantiations (different register and LDS budgets).
//
// Gradient accumulation per primitive: contributions of the lanes of a wave that
// touch the same primitive are summed in registers with DPP row shifts before
// any atomic (the DISTWAR observation, arXiv author page: most lanes of a warp
// update the same addresses). Alpha blending: every lane of a wave walks the same
// list entry, so each value is row-reduced and four lanes add into an LDS slot
// per entry; one global atomic per entry and value leaves the tile. Spheres:
// each pixel's first top_k spheres are tile-list positions, so contributions are
// added into an LDS table indexed by position and flushed once per tile.
#include "splat_internal.h"

#include "render_common.h"

namespace {

// Sum within each 16-lane row (inclusive scan); lanes 15, 31, 47, 63 hold the row sums.
__device__ __forceinline__ float row_sum_to_last(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
  return x;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// 1 / d and t / d for 0 < d <= 1 and normal t (here d = 1 - alpha, alpha at
// most alpha_max < 1): the hardware reciprocal refined by two Newton steps, and
// the quotient t r corrected once by its residual. Within an ulp or two of the
// rounded quotient, without the scaling and fix-up steps that IEEE division
// spends on the full exponent range.
__device__ __forceinline__ double recip_unit(double d) {
  double r = __builtin_amdgcn_rcp(d);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  return r;
}
__device__ __forceinline__ double div_unit(double t, double d, double r) {
  const double q = t * r;
  return __builtin_fma(__builtin_fma(-d, q, t), r, q);
}

// Pair sums through the gfx950 lane swaps (VALU; no LDS traffic).
// v_permlane32_swap exchanges the upper half of its first register with the
// lower half of its second, so the two results of swapping (x, y) add up to
// x[l] + x[l + 32] in lanes l < 32 and y[l - 32] + y[l] in lanes l >= 32.
// v_permlane16_swap exchanges the odd 16-lane rows of the first register with
// the even rows of the second: the sum holds x summed over rows (0, 1) and
// (2, 3) in rows 0 and 2, and y the same way in rows 1 and 3. The results are
// copied to plain integers before the bit casts: bit-casting an element of the
// returned pair directly read the first element for both.
__device__ __forceinline__ float swap_add32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned a = r[0], b = r[1];
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float swap_add16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned a = r[0], b = r[1];
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ double swap_add32(double x, double y) {
  const unsigned long long bx = __builtin_bit_cast(unsigned long long, x), by = __builtin_bit_cast(unsigned long long, y);
  const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)bx, (unsigned)by, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(bx >> 32), (unsigned)(by >> 32), false, false);
  const unsigned l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
  return __builtin_bit_cast(double, ((unsigned long long)h0 << 32) | l0) +
         __builtin_bit_cast(double, ((unsigned long long)h1 << 32) | l1);
}
__device__ __forceinline__ double swap_add16(double x, double y) {
  const unsigned long long bx = __builtin_bit_cast(unsigned long long, x), by = __builtin_bit_cast(unsigned long long, y);
  const auto lo = __builtin_amdgcn_permlane16_swap((unsigned)bx, (unsigned)by, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(bx >> 32), (unsigned)(by >> 32), false, false);
  const unsigned l0 = lo[0], l1 = lo[1], h0 = hi[0], h1 = hi[1];
  return __builtin_bit_cast(double, ((unsigned long long)h0 << 32) | l0) +
         __builtin_bit_cast(double, ((unsigned long long)h1 << 32) | l1);
}

template <int CTRL>
__device__ __forceinline__ double dpp_t(double x) { return dpp_f64<CTRL, 0xf, true>(x); }
template <int CTRL>
__device__ __forceinline__ float dpp_t(float x) { return dpp_f32<CTRL>(x); }

// Eight values per lane summed over the wave, transposed: every lane l ends with
// the total of v[l >> 3] (value q in the lanes of 8-lane group q). Each step
// halves the values a lane carries. The two lane swaps go first: a swap moves
// whole halves or rows between two registers, so which value a lane keeps
// follows from its lane id with no select (lane bit 5, then bit 4). Bit 3 takes
// a select and a row rotate by 8; three DPP steps then sum each 8-lane group.
template <typename T>
__device__ __forceinline__ T wave_sum8_transposed(const T (&v)[8]) {
  const bool b3 = lane_id() & 8u;
  T a[4], c[2];
#pragma unroll
  for (int j = 0; j < 4; j++) a[j] = swap_add32(v[j], v[j + 4]);     // value j + 4 b5
#pragma unroll
  for (int j = 0; j < 2; j++) c[j] = swap_add16(a[j], a[j + 2]);     // value j + 2 b4 + 4 b5
  T e = (b3 ? c[1] : c[0]) + dpp_t<0x128>(b3 ? c[0] : c[1]);         // row rotate by 8: lane ^ 8
  e += dpp_t<0xB1>(e);                                                // lane ^ 1
  e += dpp_t<0x4E>(e);                                                // lane ^ 2
  e += dpp_t<0x141>(e);                                               // 8-lane mirror: the other quad
  return e;
}

// Up to two fp64 and two fp32 ranges cleared by one launch.
struct ZeroRanges {
  double *d0, *d1;
  float *f0, *f1;
  uint32_t *u0;
  long long nd0, nd1, nf0, nf1, nu0;
};

constexpr int ZERO_GRID = 4096;

// Grid-stride over the ranges in order (at most ZERO_GRID workgroups).
__global__ __launch_bounds__(256) void k_zero(ZeroRanges z) {
  const long long n = z.nd0 + z.nd1 + z.nf0 + z.nf1 + z.nu0;
  for (long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x; i0 < n;
       i0 += (long long)gridDim.x * blockDim.x) {
    long long i = i0;
    if (i < z.nd0) { z.d0[i] = 0.0; continue; }
    i -= z.nd0;
    if (i < z.nd1) { z.d1[i] = 0.0; continue; }
    i -= z.nd1;
    if (i < z.nf0) { z.f0[i] = 0.0f; continue; }
    i -= z.nf0;
    if (i < z.nf1) { z.f1[i] = 0.0f; continue; }
    i -= z.nf1;
    if (i < z.nu0) z.u0[i] = 0u;
  }
}


// Four fp32 values per lane summed over the wave, transposed: value q ends in
// every lane of 16-lane row q. The lane swaps pair v_q with v_(q+2) across the
// halves, then the results across rows; four DPP adds sum each row.
__device__ __forceinline__ float wave_sum4_transposed(const float (&v)[4]) {
  const float a0 = swap_add32(v[0], v[2]), a1 = swap_add32(v[1], v[3]);   // value (lane bit 5) * 2 + 0 or 1
  float e = swap_add16(a0, a1);                                          // value = lane >> 4
  e += dpp_f32<0xB1>(e);                                                 // lane ^ 1
  e += dpp_f32<0x4E>(e);                                                 // lane ^ 2
  e += dpp_f32<0x141>(e);                                                // 8-lane mirror
  e += dpp_f32<0x140>(e);                                                // 16-lane mirror
  return e;
}

// ---------------------------------------------------------------------------
// Alpha blending backward: replay each pixel's list back to front from `last`,
// recovering T before entry k as T_after / (1 - alpha_k) (fp64).
// Per entry and pixel the gradient is a common factor d loss / d power times
// geometric terms of the offset (dx, dy); those terms and their sums are fp64,
// colour and opacity terms fp32.
// ---------------------------------------------------------------------------
template <int CM>
__global__ __launch_bounds__(256) void k_bwd_alpha(ViewTable vt, BwdArgs A, int tile_begin) {
  constexpr int NF = CM;                    // fp32 values per entry: features
  constexpr int NFP = NF | 1;               // odd row stride: lanes of one entry hit distinct banks
  constexpr int NG = (NF + 7) / 8;          // groups of eight for the transposed reduction
  static_assert(NG <= 8, "one lane of an 8-lane group per group of channels");
  // entries staged per batch: fewer with many channels, so that two or more
  // workgroups fit a CU's LDS
  constexpr int BT = NF >= 64 ? 64 : 128;
  __shared__ double2 s_uv[BT];
  __shared__ double2 s_ab[BT];
  __shared__ double2 s_co[BT];
  constexpr int NFS = (NF + 3) & ~3;        // 16-byte rows: vector reads of an entry's features
  __shared__ float s_f[BT][NFS];
  __shared__ uint32_t s_rid[BT];
  __shared__ double s_ag[BT][7];           // du, dv, d_ca, d_cb, d_cc, d_opac (odd stride)
  __shared__ float s_af[BT][NFP];          // d_feat
  __shared__ QuadLists s_l;
  __shared__ uint32_t s_maxlast;
  if (*A.overflow) return;
  const int gtile = tile_begin + blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  if (c.kind == SPLAT_CAM_SPHERICAL) return;
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile];
  const uint32_t len = A.ranges[2 * gtile + 1] - start;
  const unsigned lane = lane_id();
  const int wq = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  const size_t pofs = c.img_off + (size_t)tp.j * c.W + tp.i;
  const double pxr = tp.pxr, pyr = tp.pyr;
  uint32_t lastp = 0;
  double T = 1.0;      // transmittance after the current entry
  float g[CM];
  // behind the current entry: the composited colour projected on the pixel's
  // upstream gradient, sum_ch Sb_ch g_ch
  float Sb = 0.0f;
#pragma unroll
  for (int ch = 0; ch < CM; ch++) g[ch] = (tp.inside && ch < A.C) ? A.dimg[pofs + ch * plane] : 0.0f;
  if (tp.inside) {
    lastp = min(A.last[p], len);     // a forward buffer never exceeds the tile's list
    T = (double)A.T_final[p];
  }
  if (threadIdx.x == 0) s_maxlast = 0;
  __syncthreads();
  if (lastp) atomicMax(&s_maxlast, lastp);
  __syncthreads();
  const uint32_t maxlast = s_maxlast;
  // deepest list position any pixel of this wave replays
  uint32_t wlast = lastp;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) wlast = max(wlast, (uint32_t)__shfl_xor((int)wlast, d, WAVE));
  wlast = (uint32_t)__builtin_amdgcn_readfirstlane((int)wlast);
  const long long vbase = (long long)view * A.n;
  const float amin = A.alpha_min, amax = A.alpha_max;

  for (int hi = (int)maxlast; hi > 0; hi -= BT) {
    const int lo = hi > BT ? hi - BT : 0;
    const int cnt = hi - lo;
    unsigned mask = 0;
    if ((int)threadIdx.x < cnt) {
      const uint32_t rid = A.vals[start + lo + threadIdx.x];
      const DrawRec d = A.draw[rid];
      s_rid[threadIdx.x] = rid;
      s_uv[threadIdx.x] = stage_uv(c, tp, d, false);
      const Conic cn = stage_conic(d);
      s_ab[threadIdx.x] = cn.ab;
      s_co[threadIdx.x] = cn.co;
      const long long id = (long long)rid - vbase;
#pragma unroll
      for (int ch = 0; ch < CM; ch++) s_f[threadIdx.x][ch] = ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
#pragma unroll
      for (int q = 0; q < 6; q++) s_ag[threadIdx.x][q] = 0.0;
#pragma unroll
      for (int q = 0; q < NF; q++) s_af[threadIdx.x][q] = 0.0f;
      mask = quadrant_mask(tp, d);
    }
    build_quad_lists(s_l, mask);
    // One entry of the wave's list (uniform index), back to front.
    auto entry = [&](const int idx) {
      const uint32_t pos = (uint32_t)(lo + idx);
      if (pos >= wlast) return;                 // beyond every pixel of the wave
      const double2 ab = s_ab[idx], co = s_co[idx];
      float G, og;
      double dx, dy;
      const float al = splat_alpha<false>(c, pxr, pyr, s_uv[idx], ab, co, amax, G, og, dx, dy);
      const bool act = (pos < lastp) & (al >= amin);
      if (ballot64(act) == 0) return;
      // Straight-line code on every lane: a lane without this entry takes
      // alpha = 0, which leaves T and Sb as they are (a division by 1) and
      // zeroes its terms; only the clamp and the alpha gradient need selects.
      const float ala = act ? al : 0.0f;
      const float om = 1.0f - ala;
      const double dal = 1.0 - (double)ala;
      const double Tkd = div_unit(T, dal, recip_unit(dal));
      const float Tk = (float)Tkd;
      const float wk = Tk * ala;
      // d loss / d alpha = T_k sum_ch (f_ch - Sb_ch) g_ch, and sum_ch Sb_ch g_ch
      // follows the same blend as Sb: one dot product per entry
      float vf[NF];
      float fg = 0.0f;
#pragma unroll
      for (int ch = 0; ch < CM; ch++) {
        const float f = s_f[idx][ch];
        vf[ch] = wk * g[ch];
        fg = __builtin_fmaf(f, g[ch], fg);
      }
      const float da = Tk * (fg - Sb);
      Sb = __builtin_fmaf(ala, fg, om * Sb);
      T = Tkd;
      // alpha is the constant amax where clamped
      const bool geo = act & !(og > amax);
      double vg[6];
      vg[5] = geo ? (double)(G * da) : 0.0;
      {
        const double dp = geo ? -(double)ala * (double)da : 0.0;   // d loss / d power
        const double ha = ab.x, bb = ab.y, hc = co.x;                // a/2, b, c/2
        vg[0] = -dp * (2.0 * ha * dx + bb * dy);
        vg[1] = -dp * (bb * dx + 2.0 * hc * dy);
        vg[2] = dp * 0.5 * dx * dx;
        vg[3] = dp * dx * dy;
        vg[4] = dp * 0.5 * dy * dy;
      }
      {
        double v8[8];
#pragma unroll
        for (int q = 0; q < 8; q++) v8[q] = q < 6 ? vg[q] : 0.0;
        const double r = wave_sum8_transposed(v8);
        if (((lane & 7u) == 0u) & ((lane >> 3) < 6u)) atomicAdd(&s_ag[idx][lane >> 3], r);
      }
      if constexpr (NF >= 3 && NF <= 4) {
        // wave totals, transposed: channel q ends in the lanes of row q
        float v4[4];
#pragma unroll
        for (int q = 0; q < 4; q++) v4[q] = q < NF ? vf[q < NF ? q : 0] : 0.0f;
        const float x = wave_sum4_transposed(v4);
        if (((lane & 15u) == 0u) & ((lane >> 4) < (unsigned)NF)) atomicAdd(&s_af[idx][lane >> 4], x);
      } else if constexpr (NF >= 3) {
        // wave totals, transposed: group gq's channel 8 gq + q ends in the lanes
        // 8q..8q+7, and lane 8q + j adds that of group j
        float tot[NG];
#pragma unroll
        for (int gq = 0; gq < NG; gq++) {
          float v8[8];
#pragma unroll
          for (int j = 0; j < 8; j++) v8[j] = gq * 8 + j < NF ? vf[gq * 8 + j] : 0.0f;
          tot[gq] = wave_sum8_transposed(v8);
        }
        float x = tot[0];
#pragma unroll
        for (int gq = 1; gq < NG; gq++) x = (lane & 7u) == (unsigned)gq ? tot[gq] : x;
        const unsigned ch = 8u * (lane & 7u) + (lane >> 3);
        if (((lane & 7u) < (unsigned)NG) & (ch < (unsigned)NF)) atomicAdd(&s_af[idx][ch], x);
      } else {
#pragma unroll
        for (int q = 0; q < NF; q++) {
          const float r = row_sum_to_last(vf[q]);
          if ((lane & 15u) == 15u) atomicAdd(&s_af[idx][q], r);
        }
      }
        };
    {
      const int cnt_q = __builtin_amdgcn_readfirstlane(s_l.cnt[wq]);
      int k = cnt_q - 1;
      for (; k >= 0 && ((k + 1) & 3); k--) entry(__builtin_amdgcn_readfirstlane((int)s_l.idx[wq][k]));
      for (; k >= 3; k -= 4) {                  // four indices per list read
        const uint32_t four =
            __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t *>(&s_l.idx[wq][k - 3]));
        entry((int)(four >> 24));
        entry((int)((four >> 16) & 0xffu));
        entry((int)((four >> 8) & 0xffu));
        entry((int)(four & 0xffu));
      }
    }
    __syncthreads();
    // Flush: one wave per entry, its lanes over the entry's values, so that each
    // atomic instruction covers one or two cache lines of the record's rows.
    for (int e = wq; e < cnt; e += 4) {
      const uint32_t rid = s_rid[e];
      double *dg = A.accg + (size_t)rid * ACC_G;
      if (lane < 6u) {
        const double x = s_ag[e][lane];
        if (x != 0.0) atomicAdd(dg + lane, x);
      }
      double *df = A.accf + (size_t)rid * A.C;
#pragma unroll
      for (int q0 = 0; q0 < CM; q0 += WAVE) {
        const int q = q0 + (int)lane;
        if (q < CM && q < A.C) {
          const float x = s_af[e][q];
          if (x != 0.0f) atomicAdd(df + q, (double)x);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Spherical (lidar) views, reverse pass. A lidar tile's list can hold tens of
// thousands of entries, and one wave walking it back to front sets the
// kernel's length. Four waves share each quadrant's list of a batch of BL
// entries, one contiguous part each:
//  1. every wave composites its part front to back from T = 1 for its pixels
//     (only entries before the pixel's `last`): the part's transmittance P_j
//     and depth A_j;
//  2. the reverse pass through part j maps the state after it (T, Sb) to
//     (T / P_j, A_j + P_j Sb), so each wave chains the later parts' (P, A)
//     onto the state after the batch to get the state after its own part;
//  3. each wave replays its part back to front from that state, as the
//     single-wave replay does, and the chain through all four parts is the
//     state after the preceding batch.
// Sb is the depth composited behind the current entry, normalised by the
// transmittance before it. Gradients w.r.t. the entry's alpha: depth output
// T_k (depth_k - Sb) g_depth; opacity output 1 - T_final: T_final / (1 - alpha_k)
// g_opacity.
// ---------------------------------------------------------------------------
constexpr int BL = 512;                  // entries staged per batch

// SPH = false: pinhole views with up to four channels (launches with few
// tiles, as in the forward). There Sb is the blend of f . g over the channels
// (f the entry's features, g the pixel's upstream gradient), so the per-part
// state is still one value, and d loss / d alpha = T_k (f . g - Sb).
template <int CM, bool SPH>
__global__ __launch_bounds__(1024) void k_bwd_split(ViewTable vt, BwdArgs A, int tile_begin) {
  constexpr int NF = SPH ? 1 : CM;         // range, or the features
  constexpr int NFP = NF | 1;              // odd stride of the feature sums
  __shared__ double2 s_uv[BL];
  __shared__ double2 s_ab[BL];
  __shared__ double2 s_co[BL];
  __shared__ float s_f[BL][NF];
  __shared__ uint32_t s_rid[BL];
  __shared__ __align__(16) uint16_t s_idx[4][BL];  // per-quadrant lists of the batch
  __shared__ int s_woff[16][4];
  __shared__ int s_cnt[4];
  __shared__ double s_ag[BL][7];           // du, dv, d_ca, d_cb, d_cc, d_opac (odd stride)
  __shared__ float s_af[BL][NFP];          // d_depth, or d_feature
  __shared__ float s_pA[4][256];           // per part and pixel: Sb composited from T = 1,
  __shared__ double s_pT[4][256];          //   and the part's transmittance
  __shared__ uint32_t s_maxlast;
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
  const uint32_t start = A.ranges[2 * gtile];
  const uint32_t len = A.ranges[2 * gtile + 1] - start;
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  const size_t pofs = c.img_off + (size_t)tp.j * c.W + tp.i;
  const double pxr = tp.pxr, pyr = tp.pyr;
  uint32_t lastp = 0;
  double T = 1.0;                          // after the batch (the same in all four copies)
  float Sb = 0.0f;
  // upstream gradient: d loss / d (depth, opacity), or per channel
  float g[SPH ? 2 : NF];
#pragma unroll
  for (int ch = 0; ch < (SPH ? 2 : NF); ch++) g[ch] = tp.inside && (SPH || ch < A.C) ? A.dimg[pofs + ch * plane] : 0.0f;
  const long long vbase = (long long)view * A.n;
  if (tp.inside) {
    lastp = min(A.last[p], len);
    T = (double)A.T_final[p];
  }
  const double Tfin = T;
  if (tid == 0) s_maxlast = 0;
  __syncthreads();
  if (lastp) atomicMax(&s_maxlast, lastp);
  __syncthreads();
  const uint32_t maxlast = s_maxlast;
  uint32_t wlast = lastp;                  // deepest position a pixel of the wave replays
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) wlast = max(wlast, (uint32_t)__shfl_xor((int)wlast, d, WAVE));
  wlast = (uint32_t)__builtin_amdgcn_readfirstlane((int)wlast);
  const float amin = A.alpha_min, amax = A.alpha_max;
  const uint64_t below = lane ? (~0ull >> (64u - lane)) : 0ull;

  for (int hi = (int)maxlast; hi > 0; hi -= BL) {
    const int lo = hi > BL ? hi - BL : 0;
    const int cnt = hi - lo;
    unsigned mask = 0;
    int seam = 0;
    if ((int)tid < cnt) {
      const uint32_t rid = A.vals[start + lo + tid];
      const DrawRec d = A.draw[rid];
      s_rid[tid] = rid;
      const double2 uv = stage_uv(c, tp, d, SPH);
      s_uv[tid] = uv;
      if constexpr (SPH) seam = seam_flag(c, uv.x);
      const Conic cn = stage_conic(d);
      s_ab[tid] = cn.ab;
      s_co[tid] = cn.co;
      if constexpr (SPH) {
        s_f[tid][0] = A.aux[rid].z;
      } else {
        const long long id = (long long)rid - vbase;
#pragma unroll
        for (int ch = 0; ch < NF; ch++) s_f[tid][ch] = ch < A.C ? A.feat[(size_t)id * A.C + ch] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 7; q++) s_ag[tid][q] = 0.0;
#pragma unroll
      for (int q = 0; q < NF; q++) s_af[tid][q] = 0.0f;
      mask = quadrant_mask(tp, d);
    }
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
    // list entries: staged index | LIST_SEAM
    const int L = __builtin_amdgcn_readfirstlane(s_cnt[wq]);
    const int k0 = (L * part) / 4, k1 = (L * (part + 1)) / 4;

    // the value an entry blends into Sb: its range, or f . g
    auto blend_value = [&](const int idx) {
      if constexpr (SPH) {
        return s_f[idx][0];
      } else {
        float fg = 0.0f;
#pragma unroll
        for (int ch = 0; ch < NF; ch++) fg = __builtin_fmaf(s_f[idx][ch], g[ch], fg);
        return fg;
      }
    };
    // 1. the part front to back from T = 1
    {
      double Pt = 1.0;
      float Ax = 0.0f;
      auto fwd = [&](const int ie) {
        const int idx = ie & (LIST_SEAM - 1);
        const uint32_t pos = (uint32_t)(lo + idx);
        if (pos >= wlast) return;
        float G, og, al;
        double dx, dy;
        if (SPH && (ie & LIST_SEAM))                   // wave-uniform
          al = splat_alpha<true>(c, pxr, pyr, s_uv[idx], s_ab[idx], s_co[idx], amax, G, og, dx, dy);
        else
          al = splat_alpha<false>(c, pxr, pyr, s_uv[idx], s_ab[idx], s_co[idx], amax, G, og, dx, dy);
        const bool hit = (pos < lastp) & (al >= amin);
        if (ballot64(hit) == 0) return;          // no pixel of the wave takes it: nothing changes
        const float w = (hit ? 1.0f : 0.0f) * (float)(Pt * (double)al);
        Ax = __builtin_fmaf(w, blend_value(idx), Ax);
        Pt = hit ? Pt * (1.0 - (double)al) : Pt;
      };
      int k = k0;
      for (; k < k1 && (k & 3); k++) fwd(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]));
      for (; k + 4 <= k1; k += 4) {
        const uint64_t four = *reinterpret_cast<const uint64_t *>(&s_idx[wq][k]);
        const uint32_t lo4 = __builtin_amdgcn_readfirstlane((uint32_t)four);
        const uint32_t hi4 = __builtin_amdgcn_readfirstlane((uint32_t)(four >> 32));
        if ((uint32_t)lo + (lo4 & (LIST_SEAM - 1)) >= wlast) break;   // positions increase along the list
        fwd((int)(lo4 & 0xffffu));
        fwd((int)(lo4 >> 16));
        fwd((int)(hi4 & 0xffffu));
        fwd((int)(hi4 >> 16));
      }
      for (; k < k1; k++) fwd(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]));
      s_pT[part][pix] = Pt;
      s_pA[part][pix] = Ax;
    }
    __syncthreads();
    // 2. the state after this wave's part, and after the preceding batch
    double Te = T;
    float Se = Sb;
#pragma unroll
    for (int j = 3; j >= 0; j--) {
      if (j == part) {
        Te = T;
        Se = Sb;
      }
      const double Pj = s_pT[j][pix];
      T = T / Pj;
      Sb = __builtin_fmaf((float)Pj, Sb, s_pA[j][pix]);
    }
    // 3. the part back to front
    auto entry = [&](const int ie) {
      const int idx = ie & (LIST_SEAM - 1);
      const uint32_t pos = (uint32_t)(lo + idx);
      if (pos >= wlast) return;
      const double2 ab = s_ab[idx], co = s_co[idx];
      float G, og, al;
      double dx, dy;
      if (SPH && (ie & LIST_SEAM))                     // wave-uniform
        al = splat_alpha<true>(c, pxr, pyr, s_uv[idx], ab, co, amax, G, og, dx, dy);
      else
        al = splat_alpha<false>(c, pxr, pyr, s_uv[idx], ab, co, amax, G, og, dx, dy);
      const bool act = (pos < lastp) & (al >= amin);
      if (ballot64(act) == 0) return;
      // straight-line code on every lane, as in the camera pass: alpha = 0 for
      // a lane without this entry
      const float ala = act ? al : 0.0f;
      const float om = 1.0f - ala;
      const double dal = 1.0 - (double)ala, ral = recip_unit(dal);
      const double Tkd = div_unit(Te, dal, ral);
      const float Tk = (float)Tkd;
      float vf[NF], da;
      if constexpr (SPH) {
        // depth output T_k (depth_k - Sb) g_depth; opacity output 1 - T_final
        const float dep = s_f[idx][0];
        vf[0] = Tk * ala * g[0];
        da = Tk * (dep - Se) * g[0] + (float)div_unit(Tfin, dal, ral) * g[1];
        Se = __builtin_fmaf(ala, dep, om * Se);
      } else {
        const float wk = Tk * ala;
        const float fg = blend_value(idx);
#pragma unroll
        for (int ch = 0; ch < NF; ch++) vf[ch] = wk * g[ch];
        da = Tk * (fg - Se);
        Se = __builtin_fmaf(ala, fg, om * Se);
      }
      Te = Tkd;
      const bool geo = act & !(og > amax);    // alpha is the constant amax where clamped
      double vg[6];
      vg[5] = geo ? (double)(G * da) : 0.0;
      {
        const double dp = geo ? -(double)ala * (double)da : 0.0;   // d loss / d power
        const double ha = ab.x, bb = ab.y, hc = co.x;                // a/2, b, c/2
        vg[0] = -dp * (2.0 * ha * dx + bb * dy);
        vg[1] = -dp * (bb * dx + 2.0 * hc * dy);
        vg[2] = dp * 0.5 * dx * dx;
        vg[3] = dp * dx * dy;
        vg[4] = dp * 0.5 * dy * dy;
      }
      double v8[8];
#pragma unroll
      for (int q = 0; q < 8; q++) v8[q] = q < 6 ? vg[q] : 0.0;
      const double r = wave_sum8_transposed(v8);
      if (((lane & 7u) == 0u) & ((lane >> 3) < 6u)) atomicAdd(&s_ag[idx][lane >> 3], r);
      if constexpr (NF >= 3) {
        // transposed: channel q ends in the lanes of row q
        float v4[4];
#pragma unroll
        for (int q = 0; q < 4; q++) v4[q] = q < NF ? vf[q < NF ? q : 0] : 0.0f;
        const float rf = wave_sum4_transposed(v4);
        if (((lane & 15u) == 0u) & ((lane >> 4) < (unsigned)NF)) atomicAdd(&s_af[idx][lane >> 4], rf);
      } else {
#pragma unroll
        for (int q = 0; q < NF; q++) {
          const float rf = row_sum_to_last(vf[q]);
          if ((lane & 15u) == 15u) atomicAdd(&s_af[idx][q], rf);
        }
      }
    };
    {
      int k = k1 - 1;
      for (; k >= k0 && ((k + 1) & 3); k--) entry(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]));
      for (; k - 3 >= k0; k -= 4) {             // four indices per list read
        const uint64_t four = *reinterpret_cast<const uint64_t *>(&s_idx[wq][k - 3]);
        const uint32_t lo4 = __builtin_amdgcn_readfirstlane((uint32_t)four);
        const uint32_t hi4 = __builtin_amdgcn_readfirstlane((uint32_t)(four >> 32));
        entry((int)(hi4 >> 16));
        entry((int)(hi4 & 0xffffu));
        entry((int)(lo4 >> 16));
        entry((int)(lo4 & 0xffffu));
      }
      for (; k >= k0; k--) entry(__builtin_amdgcn_readfirstlane((int)s_idx[wq][k]));
    }
    __syncthreads();
    // flush: one wave per entry, lanes over the entry's values
    for (int e = (int)sw; e < cnt; e += 16) {
      const uint32_t rid = s_rid[e];
      double *dg = A.accg + (size_t)rid * ACC_G;
      if (lane < 6u) {
        const double x = s_ag[e][lane];
        if (x != 0.0) atomicAdd(dg + lane, x);
      } else if (SPH && lane == 6u) {
        const float x = s_af[e][0];
        if (x != 0.0f) atomicAdd(dg + 6, (double)x);
      } else if (!SPH && lane >= 8u && (int)lane - 8 < NF && (int)lane - 8 < A.C) {
        const float x = s_af[e][lane - 8];
        if (x != 0.0f) atomicAdd(A.accf + (size_t)rid * A.C + (lane - 8), (double)x);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Sphere backward over the first top_k contributing spheres of each pixel.
// The forward recorded each one as its index in the sorted pair list (ascending
// per pixel). Each wave (an 8x8 quadrant of the tile) visits only the entries
// its pixels recorded: the wave-wide minimum of the lanes' next recorded index
// picks the entry, the lanes that recorded it form their gradient terms, the
// wave sums them with a transposed reduction (value q ends in the lanes of
// 8-lane group q) and one lane per value adds the sum to the record's fp32 row
// (a row takes one sum per quadrant that recorded the sphere: a few at 1M
// spheres, hundreds for a sphere of 200 px radius, and the row's rounding stays
// below that of the wave sums).
// A step costs the same whether one lane or all 64 recorded the entry, so the
// number of steps is the number of distinct spheres the quadrant's pixels
// recorded (11 on average at 1M spheres, 1024x1024), not the length of the
// tile list up to the deepest recorded entry.
// The next entry's record is requested before the current one is processed.
// Records are read with vector loads of a wave-uniform address: their wait
// counter is in order and separate from the LDS one, so the LDS reads of the
// loop do not wait for the prefetch (scalar loads share a counter with LDS and
// return out of order, and every LDS wait would have waited for them too).
// ---------------------------------------------------------------------------
// Wave-wide minimum (uniform): butterflies within each 16-lane row leave every
// lane with its row's minimum; row_bcast:15 then folds row 0 into row 1 and row
// 2 into row 3, row_bcast:31 folds lane 31 into row 3, and lane 63 holds the
// minimum. Rows outside a step's row mask take the identity ~0.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, dpp_u32<0xB1>(x));     // lane ^ 1
  x = min(x, dpp_u32<0x4E>(x));     // lane ^ 2
  x = min(x, dpp_u32<0x141>(x));    // 8-lane mirror
  x = min(x, dpp_u32<0x140>(x));    // 16-lane mirror
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x142, 0xa, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// One recorded entry: what the gradient terms need (wave-uniform values).
template <int CM>
struct SphEntry {
  double u, v, a;        // normalised centre (orthographic: (qx, qy)), A = qz^2 / r_eff^2
  float oe;              // o exp(o zhat / gamma) (max-shift: its log)
  float qz, reff, opac;
  float flags;           // bit 0 floored, bit 1 gated (converted where used: a conversion here
                         // would wait for the load right after it is issued)
  float f[CM];
};

template <int CM>
__device__ __forceinline__ SphEntry<CM> sph_entry(uint32_t rid, long long vbase, int C, const DrawRec *draw,
                                                  const AuxRec *aux, const float *feat) {
  SphEntry<CM> e;
  const DrawRec &d = draw[rid];
  const AuxRec &ax = aux[rid];
  e.u = d.u;
  e.v = d.v;
  e.a = d.a;
  e.oe = d.w;
  e.qz = ax.z;
  e.reff = ax.w;
  e.opac = ax.opac;
  e.flags = ax.flags;
#pragma unroll
  for (int ch = 0; ch < CM; ch++) {
    if constexpr (CM <= SPLAT_REC_FEAT)
      e.f[ch] = rec_feat(d, ch);                                    // here C = CM: features in the record
    else
      e.f[ch] = ch < C ? feat[(size_t)((long long)rid - vbase) * C + ch] : 0.0f;
  }
  return e;
}

// Per-pixel values the terms of a recorded sphere need.
template <int CM>
struct SphPix {
  double x, y, g;          // the ray (x, y) and 1 / |d|^2 (orthographic: 1)
  double crs;              // 1 pinhole, 0 orthographic (no cross term)
  float gi[CM];            // g / N per channel
  float gC;                // (g / N) . C
  float msh;               // max-shifted blending: the pixel's shift m from the forward
  float rxf, ryf, rgf;     // the ray in fp32 (rgf = 0 orthographic)
  float inv_span, igam, zfar;
  bool orth, max_shift;
};

template <int CM>
__device__ __forceinline__ SphPix<CM> sph_pix(const ViewDev &c, const BwdArgs &A, const TilePix &tp,
                                              const SphereRay &ray, long long p, size_t plane, size_t pofs) {
  SphPix<CM> P;
  P.x = ray.x;
  P.y = ray.y;
  P.g = ray.g;
  // per pixel: g / N and (g / N) . C, for the feature and weight terms
  P.gC = 0.0f;
  const float invN = tp.inside ? 1.0f / A.norm[p] : 0.0f;
#pragma unroll
  for (int ch = 0; ch < CM; ch++) {
    const bool ok = tp.inside && ch < A.C;
    P.gi[ch] = ok ? A.dimg[pofs + ch * plane] * invN : 0.0f;
    P.gC = __builtin_fmaf(P.gi[ch], ok ? A.img[pofs + ch * plane] : 0.0f, P.gC);
  }
  // max-shifted blending: weights (and norm) relative to exp(m), m from the forward
  P.max_shift = A.max_shift != 0;
  P.msh = (A.max_shift && tp.inside) ? A.T_final[p] : 0.0f;
  P.inv_span = (float)c.ispan;
  P.igam = A.igamma;
  P.zfar = (float)c.zfar;
  // orthographic views: a = (qx, qy), the ray along +z through (x, y, 0); dist^2 =
  // |(x, y) - a|^2, whose gradient in q is -2 (sx, sy, 0) (no cross term, no qz scale)
  P.orth = c.kind == SPLAT_CAM_ORTHOGRAPHIC;
  P.crs = P.orth ? 0.0 : 1.0;
  P.rxf = (float)ray.x;
  P.ryf = (float)ray.y;
  P.rgf = (float)ray.g * (P.orth ? 0.0f : 1.0f);
  return P;
}

// The values one pixel adds for a recorded sphere, in row order (dq0, dq1, dq2,
// d_reff, d_opac, d_feat...; v holds zeros on entry); returns the weight w. EXT:
// the pixel's d loss / d (ray x, ray y) is added into (kgx, kgy).
template <int CM, bool EXT>
__device__ __forceinline__ float sph_terms(const SphPix<CM> &P, const SphEntry<CM> &e, float *v, float &kgx,
                                           float &kgy) {
  const int flags = (int)e.flags;
  const float oe = P.max_shift ? __expf(e.oe - P.msh) : e.oe;   // o exp(o zhat / gamma) [/ exp(m)]
  // t = dist^2 / r_eff^2 = A g |a x d|^2 (fp64: near the rim D = 1 - t is a
  // small difference), a x d from the offsets sx = x - ax, sy = y - ay
  const double sx = P.x - e.u, sy = P.y - e.v;
  const double cr = (e.u * sy - e.v * sx) * P.crs;
  const double t = e.a * P.g * (sx * sx + sy * sy + cr * cr);
  const float w = oe * (float)(1.0 - t);
  float dw = -P.gC;
#pragma unroll
  for (int ch = 0; ch < CM; ch++) {
    v[5 + ch] = P.gi[ch] * w;
    dw = __builtin_fmaf(P.gi[ch], e.f[ch], dw);
  }
  const float zhat = (P.zfar - e.qz) * P.inv_span;
  const float xz = __builtin_amdgcn_rcpf(e.opac) + zhat * P.igam;     // d ln w / d o (D fixed)
  v[4] = dw * w * xz;
  if (!(flags & 2)) {
    // dist^2 = |q|^2 - (q.d)^2 / |d|^2 has gradient 2 q_perp, with
    // q_perp = qz ((d.delta) g d - delta), delta = (sx, sy, 0)
    const float ir = __builtin_amdgcn_rcpf(e.reff);
    const float dD = dw * oe;
    const float dz = dw * w * (e.opac * P.igam);
    const float sxf = (float)sx, syf = (float)sy;
    const float c1 = (P.rxf * sxf + P.ryf * syf) * P.rgf;
    const float k2 = -2.0f * dD * ir * ir * (P.orth ? 1.0f : e.qz);
    const float gq0 = k2 * (c1 * P.rxf - sxf), gq1 = k2 * (c1 * P.ryf - syf);
    v[0] = gq0;
    v[1] = gq1;
    v[2] = k2 * c1 - dz * P.inv_span;
    if (!(flags & 1)) v[3] = 2.0f * dD * (float)t * ir;
    // the ray: d dist^2 / d d = -((q.d) / |d|^2) d dist^2 / d q, with
    // (q.d) / |d|^2 = qz (1 - c1); orthographic: d dist^2 / d (x, y) = -d dist^2 / d (qx, qy)
    if constexpr (EXT) {
      const float sc = P.orth ? 1.0f : e.qz * (1.0f - c1);
      kgx = kgx - sc * gq0;
      kgy = kgy - sc * gq1;
    }
  }
  return w;
}

// EXT: the call asks for intrinsic gradients or gradient normalisation (their
// per-contribution work is compiled out of the plain reverse pass). DIRECT:
// entries recorded by at most A.direct_max lanes of a wave skip the wave
// reduction and add lane by lane (a separate instance: in the default one no
// atomic is conditional on the lane count, which keeps its memory waits exact).
template <int CM, bool EXT, bool DIRECT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(CM <= 4 ? 6 : 1))) void k_bwd_sphere(
    ViewTable vt, BwdArgs A, int tile_begin) {
  constexpr int NV = 5 + CM;                  // dq0, dq1, dq2, d_reff, d_opac, d_feat...
  constexpr int NG = (NV + 7) / 8;            // groups of eight for the reduction
  constexpr int TKS = SPLAT_TOPK_MAX + 1;     // odd stride (in pairs) of the per-pixel recorded entries
  constexpr uint32_t NONE = 0xffffffffu;
  __shared__ uint2 s_top[256 * TKS];          // per pixel: (recorded index, record id), ascending
  if (*A.overflow) return;
  const int gtile = tile_begin + blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  const TilePix tp = tile_pixel(c, gtile, threadIdx.x);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  const SphereRay ray = sphere_ray(c, tp);
  const unsigned lane = lane_id();
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  const size_t pofs = c.img_off + (size_t)tp.j * c.W + tp.i;
  const int K = A.top_k;
  const long long vbase = (long long)view * A.n;
  // recorded entries (indices into the sorted pairs, ascending), this tile's only,
  // with their record ids (all loads in flight together)
  uint2 *my_top = s_top + threadIdx.x * TKS;
  int ntop = 0;
  {
    int t[SPLAT_TOPK_MAX];
#pragma unroll
    for (int s = 0; s < SPLAT_TOPK_MAX; s++) t[s] = (s < K && tp.inside) ? A.topk[p * K + s] : -1;
    bool go = true;
#pragma unroll
    for (int s = 0; s < SPLAT_TOPK_MAX; s++) {
      go = go && t[s] >= 0 && (uint32_t)t[s] >= start && (uint32_t)t[s] < end;
      ntop += go ? 1 : 0;
    }
    uint32_t r[SPLAT_TOPK_MAX];
#pragma unroll
    for (int s = 0; s < SPLAT_TOPK_MAX; s++) r[s] = s < ntop ? A.vals[t[s]] : 0u;
#pragma unroll
    for (int s = 0; s < SPLAT_TOPK_MAX; s++)
      if (s < ntop) my_top[s] = make_uint2((uint32_t)t[s], r[s]);
    my_top[ntop] = make_uint2(NONE, 0u);
  }
  const SphPix<CM> P = sph_pix<CM>(c, A, tp, ray, p, plane, pofs);
  // d loss / d (ray x, ray y) summed over the pixel's recorded spheres
  float kgx = 0.0f, kgy = 0.0f;
  const int rowlen = 5 + A.C;

  int nxt = 0;
  uint2 cur_t = my_top[0];
  uint32_t m = wave_min_u32(cur_t.x);
  // the record id of entry m, from the first lane whose next entry it is
  // (NONE: 0, the first record)
  auto rid_of = [&](uint32_t mm) {
    const int l = __builtin_amdgcn_readfirstlane((int)__ffsll((long long)ballot64(cur_t.x == mm)) - 1);
    const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)cur_t.y, l & 63);
    return mm != NONE ? r : 0u;
  };
  // One step: entry m (record e, id rid) is processed while the next entry's
  // record is requested into en / rid_n; m becomes the next entry.
  auto step = [&](const SphEntry<CM> &e, uint32_t rid, SphEntry<CM> &en, uint32_t &rid_n) {
    const bool mine = cur_t.x == m;
    if (mine) {
      nxt++;
      cur_t = my_top[nxt];
    }
    // requested unconditionally (record 0 after the last entry: any record is a
    // valid address), so that the number of loads in flight is the same on every
    // path and the wait for this step's record does not also wait for them
    const uint32_t mn = wave_min_u32(cur_t.x);
    rid_n = rid_of(mn);
    en = sph_entry<CM>(rid_n, vbase, A.C, A.draw, A.aux, A.feat);
    if constexpr (EXT)
      if (A.cnt) {
        const uint64_t bm = ballot64(mine);
        if (lane == 0u) atomicAdd(A.cnt + rid, (uint32_t)__popcll(bm));
      }
    float v[NG * 8];
#pragma unroll
    for (int q = 0; q < NG * 8; q++) v[q] = 0.0f;
    if (mine) sph_terms<CM, EXT>(P, e, v, kgx, kgy);
    float *row = A.accs + (size_t)rid * A.rs;
    bool reduce = true;
    if constexpr (DIRECT) {
      // few lanes recorded the entry: they add their values straight to the
      // row (global atomics resolved in L2) instead of the wave reduction
      // (DISTWAR's split between in-register reduction and atomic units)
      reduce = __popcll(ballot64(mine)) > A.direct_max;
      if (!reduce && mine) {
#pragma unroll
        for (int q = 0; q < NV; q++)
          if (q < rowlen) atomicAdd(row + q, v[q]);
      }
    }
    if (reduce) {
#pragma unroll
      for (int gq = 0; gq < NG; gq++) {
        const float (&vg)[8] = *reinterpret_cast<const float(*)[8]>(&v[8 * gq]);
        const float r = wave_sum8_transposed(vg);
        const int q = 8 * gq + (int)(lane >> 3);
        if (((lane & 7u) == 0u) & (q < rowlen) & (r != 0.0f)) atomicAdd(row + q, r);
      }
    }
    m = mn;
  };
  // two record buffers used in turn (no copy of the prefetched record per step)
  SphEntry<CM> e0, e1;
  uint32_t r0 = 0u, r1 = 0u;
  if (m != NONE) {
    r0 = rid_of(m);
    e0 = sph_entry<CM>(r0, vbase, A.C, A.draw, A.aux, A.feat);
  }
  while (m != NONE) {
    step(e0, r0, e1, r1);
    if (m == NONE) break;
    step(e1, r1, e0, r0);
  }
  if (EXT && A.kslot) {
    // intrinsics: the ray (x, y) = ((px - cx) / fx, (py - cy) / fy); per wave
    // the pixels' (d/dfx, d/dfy, d/dcx, d/dcy) are summed, lanes 0, 8, 16, 24 add them
    double v8[8];
    v8[0] = -(double)kgx * ray.x * c.ifx;
    v8[1] = -(double)kgy * ray.y * c.ify;
    v8[2] = -(double)kgx * c.ifx;
    v8[3] = -(double)kgy * c.ify;
#pragma unroll
    for (int q = 4; q < 8; q++) v8[q] = 0.0;
    const double r = wave_sum8_transposed(v8);
    if (((lane & 7u) == 0u) & ((lane >> 3) < 4u))
      atomicAdd(A.kslot + ((size_t)view * SPLAT_K_SLOTS + blockIdx.x % SPLAT_K_SLOTS) * 4 + (lane >> 3), r);
  }
}

// The plain reverse pass over spheres (no intrinsic gradients, normalisation or
// lane-by-lane atomics; at most SPH_DENSE_K recorded entries per pixel and three
// channels, eight values per entry) in two phases.
// Phase one: every lane forms the values of all its recorded entries, every lane
// busy, the records of three slots in flight together, and keeps them in LDS
// (24 bytes per slot, its own rows: the waves share nothing and need no barrier).
// Phase two: the wave walks the distinct entries as the kernel above does, but a
// step only takes the recording lanes' values, sums them over the wave and adds
// the sums: the arithmetic no longer runs once per distinct entry with only the
// lanes that recorded it active (29 of 64 on average at 1M spheres, 1024x1024).
// The walk goes in order of record id (each lane's ids sorted in registers), so
// that the wave minimum is the record itself and a step loads no record; the
// slot a lane is at after a step is read from LDS one step before it is needed.
// Five waves per SIMD (30 KB of LDS per workgroup) with 72 registers: with all
// five records in flight at once the kernel needed more registers and spilled.
constexpr int SPH_DENSE_K = 5;

__device__ __forceinline__ void sort2(uint32_t &a, uint32_t &b) {
  const uint32_t lo = min(a, b), hi = max(a, b);
  a = lo;
  b = hi;
}

template <int CM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void k_bwd_sphere_dense(ViewTable vt,
                                                                                           BwdArgs A,
                                                                                           int tile_begin) {
  static_assert(5 + CM <= 8, "eight values per entry");
  static_assert(SPH_DENSE_K == 5, "the sorting network below is for five ids");
  constexpr int KD = SPH_DENSE_K;
  constexpr uint32_t NONE = 0xffffffffu;
  // slot s of pixel tid: values 0..3, then value 4 and the weight w (the feature
  // values are g_ch / N w)
  __shared__ float4 s_va[KD][256];
  __shared__ float2 s_vb[KD][256];
  if (*A.overflow) return;
  const unsigned tid = threadIdx.x;
  const int gtile = tile_begin + blockIdx.x;
  const int view = view_of_tile(vt, gtile);
  const ViewDev &c = vt.v[view];
  const TilePix tp = tile_pixel(c, gtile, tid);
  const uint32_t start = A.ranges[2 * gtile], end = A.ranges[2 * gtile + 1];
  const SphereRay ray = sphere_ray(c, tp);
  const unsigned lane = lane_id();
  const long long p = c.pix_off + (long long)tp.j * c.W + tp.i;
  const size_t plane = (size_t)c.W * c.H;
  const size_t pofs = c.img_off + (size_t)tp.j * c.W + tp.i;
  const int K = A.top_k;
  const long long vbase = (long long)view * A.n;
  // record ids of this tile's recorded entries, ascending, NONE after the last
  int ntop = 0;
  uint32_t r[KD];
  {
    int t[KD];
#pragma unroll
    for (int s = 0; s < KD; s++) t[s] = (s < K && tp.inside) ? A.topk[p * K + s] : -1;
    bool go = true;
#pragma unroll
    for (int s = 0; s < KD; s++) {
      go = go && t[s] >= 0 && (uint32_t)t[s] >= start && (uint32_t)t[s] < end;
      ntop += go ? 1 : 0;
    }
#pragma unroll
    for (int s = 0; s < KD; s++) r[s] = s < ntop ? A.vals[t[s]] : NONE;
    // a sorting network for five (nine compare-exchanges)
    sort2(r[0], r[1]); sort2(r[3], r[4]); sort2(r[2], r[4]); sort2(r[2], r[3]); sort2(r[0], r[3]);
    sort2(r[0], r[2]); sort2(r[1], r[4]); sort2(r[1], r[3]); sort2(r[1], r[2]);
  }
  const SphPix<CM> P = sph_pix<CM>(c, A, tp, ray, p, plane, pofs);
  // phase one, over the slots some lane of the wave uses (record 0 stands in
  // for a lane's empty slots: a wave that reaches it has at least one record)
  int nmax = 0;
#pragma unroll
  for (int s = 0; s < KD; s++) nmax += ballot64(ntop > s) != 0 ? 1 : 0;
  // (in groups of PG slots, the group's records in flight together: all five at
  // once held more registers than five waves per SIMD allow)
  constexpr int PG = 3;
#pragma unroll
  for (int s0 = 0; s0 < KD; s0 += PG) {
    if (s0 >= nmax) break;
    SphEntry<CM> e[PG];
#pragma unroll
    for (int j = 0; j < PG; j++) {
      const int s = s0 + j;
      if (s < KD && s < nmax) e[j] = sph_entry<CM>(r[s] != NONE ? r[s] : 0u, vbase, A.C, A.draw, A.aux, A.feat);
    }
#pragma unroll
    for (int j = 0; j < PG; j++) {
      const int s = s0 + j;
      if (s >= KD || s >= nmax) break;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; q++) v[q] = 0.0f;
      float kx = 0.0f, ky = 0.0f;
      const float w = sph_terms<CM, false>(P, e[j], v, kx, ky);
      s_va[s][tid] = make_float4(v[0], v[1], v[2], v[3]);
      s_vb[s][tid] = make_float2(v[4], w);
    }
  }
  // phase two: a step takes the current slot's values from one register set and
  // reads the slot the lane is at after the step (the next one if the lane
  // recorded the entry, else the same) into the other; q0 is the lane's current
  // id (the ids q0..q4 move down a place when the lane recorded the entry)
  const int rowlen = 5 + A.C;
  int nxt = 0;
  float4 a0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), a1 = a0;
  float2 b0 = make_float2(0.0f, 0.0f), b1 = b0;
  if (nmax > 0) {
    a0 = s_va[0][tid];
    b0 = s_vb[0][tid];
  }
  uint32_t q0 = r[0], q1 = r[1], q2 = r[2], q3 = r[3], q4 = r[4];
  uint32_t m = wave_min_u32(q0);
  auto step = [&](const float4 &ca, const float2 &cb, float4 &na, float2 &nb) {
    const bool mine = q0 == m;
    float v[8];
    const float w = mine ? cb.y : 0.0f;
    v[0] = mine ? ca.x : 0.0f;
    v[1] = mine ? ca.y : 0.0f;
    v[2] = mine ? ca.z : 0.0f;
    v[3] = mine ? ca.w : 0.0f;
    v[4] = mine ? cb.x : 0.0f;
#pragma unroll
    for (int q = 5; q < 8; q++) v[q] = q - 5 < CM ? P.gi[q - 5 < CM ? q - 5 : 0] * w : 0.0f;
    q0 = mine ? q1 : q0;
    q1 = mine ? q2 : q1;
    q2 = mine ? q3 : q2;
    q3 = mine ? q4 : q3;
    q4 = mine ? NONE : q4;
    nxt += mine ? 1 : 0;
    const int sl = min(nxt, KD - 1);
    na = s_va[sl][tid];
    nb = s_vb[sl][tid];
    const uint32_t mn = wave_min_u32(q0);
    const float sum = wave_sum8_transposed(v);
    float *row = A.accs + (size_t)m * A.rs;
    if (((lane & 7u) == 0u) & ((int)(lane >> 3) < rowlen) & (sum != 0.0f)) atomicAdd(row + (lane >> 3), sum);
    m = mn;
  };
  while (m != NONE) {
    step(a0, b0, a1, b1);
    if (m == NONE) break;
    step(a1, b1, a0, b0);
  }
}

// Sum of the intrinsic-gradient slots of each view, in slot order.
__global__ __launch_bounds__(256) void k_cam_K_final(const double *kslot, float *gK, int vbeg, int vend,
                                                     int accumulate) {
  const int v = vbeg + (int)(threadIdx.x >> 2), a = (int)(threadIdx.x & 3u);
  if (v >= vend) return;
  const double *row = kslot + (size_t)v * SPLAT_K_SLOTS * 4 + a;
  double s = 0.0;
  for (int k = 0; k < SPLAT_K_SLOTS; k++) s += row[4 * k];
  if (accumulate) gK[4 * v + a] += (float)s;
  else gK[4 * v + a] = (float)s;
}

// ---------------------------------------------------------------------------
// Per-primitive chain rule (fp64), one thread per primitive, views summed.
// ---------------------------------------------------------------------------
struct ProjBwdArgs {
  int kind, n, C;
  const float *pos, *scale, *rot;
  BinArrays bin;
  const AuxRec *aux;
  const uint32_t *cnt;      // spheres, normalised gradients: pixels that recorded each record
  const double *accg;
  const double *accf;
  const float *accs;        // spheres: fp32 rows of 5 + C values, stride rs
  int rs;
  double *cam_part;
  float *gpos, *gscale, *grot, *gop, *gfeat, *gR, *gt;
  int accumulate;
  int cam_store;            // k_cam_final stores R, t instead of adding (nothing zeroed them)
};

__device__ __forceinline__ void put(float *p, size_t i, double x, int accumulate) {
  if (accumulate) p[i] += (float)x;
  else p[i] = (float)x;
}

__device__ __forceinline__ bool rec_live(const BinArrays &b, size_t rec) { return (b.rect[rec].x >> 16) != 0u; }

// Weight of a record's camera-gradient contribution: 1, or under Pulsar's
// normalisation (B.2) 1 / (projected area in pixels x 1e-3), the area
// pi (fx r_eff / qz)(fy r_eff / qz) (orthographic: pi (fx r_eff)(fy r_eff)).
__device__ __forceinline__ double cam_weight(const ViewDev &c, const ProjBwdArgs &P, size_t rec) {
  if (!P.cnt) return 1.0;
  if (!rec_live(P.bin, rec)) return 0.0;
  const AuxRec a = P.aux[rec];
  const double re = (double)a.w, iz = c.kind == SPLAT_CAM_ORTHOGRAPHIC ? 1.0 : 1.0 / (double)a.z;
  const double area = 3.141592653589793 * ((double)c.fx * re * iz) * ((double)c.fy * re * iz);
  return 1.0 / (area * 1e-3);
}

// Spheres, one fp32 accumulator row of 5 + C values per record. Grid-stride over
// spheres: the chain rule sums R^T dq, d_reff, d_opac and the features over the
// views; when the call covers one view, the same pass forms that view's camera
// gradient (Pulsar B.2: dL/dR = sum_k dq_k p_k^T, dL/dt = sum_k dq_k) in fp64
// registers. Each block stores its twelve sums and k_cam_final adds them up in
// a fixed order (deterministic, and no atomics contend on twelve outputs; a
// device-scope fence per block would write back the L2 of every XCD).
template <int CM>
__global__ __launch_bounds__(256) void k_sphere_grads(ViewTable vt, ProjBwdArgs P, int vbeg, int vend, int cam_view) {
  // Outputs of 256 spheres go through LDS and leave as contiguous runs: from
  // registers, the 3- (and C-) float rows of neighbouring lanes would be written
  // one float per instruction, a third of each line at a time.
  // Up to four channels (there C = CM) a thread reads its sphere's accumulator
  // row (RW floats, 16-byte aligned) with RW / 4 vector loads, all in flight
  // together; neighbouring lanes' rows are adjacent, so the loads of a wave
  // cover one contiguous run.
  constexpr int CS = CM <= 4 ? CM : 1;         // features staged up to four channels
  constexpr bool STAGE = CM <= 4;
  constexpr int RW = STAGE ? (5 + CM + 3) & ~3 : 4;   // row stride (floats) of the vector-load path
  __shared__ double s_red[12][4];
  __shared__ float s_pos[256 * 3];
  __shared__ float s_feat[256 * CS];
  const int S = P.rs;
  double cam[12];
#pragma unroll
  for (int q = 0; q < 12; q++) cam[q] = 0.0;
  for (int i0 = blockIdx.x * 256; i0 < P.n; i0 += gridDim.x * 256) {
    const int i = i0 + (int)threadIdx.x;
    const int nb = min(256, P.n - i0);
    double dp[3] = {0, 0, 0}, dr = 0, dop = 0, nrm = 1.0;
    double fs[CS];
#pragma unroll
    for (int ch = 0; ch < CS; ch++) fs[ch] = 0.0;
    for (int v = vbeg; v < vend; v++) {
      const ViewDev &c = vt.v[v];
      float A[STAGE ? RW : 5];
      if (i < P.n) {
        const float *row = P.accs + ((size_t)v * P.n + i) * S;   // zero for culled records
        if constexpr (STAGE) {
#pragma unroll
          for (int q = 0; q < RW / 4; q++) {
            const float4 x = reinterpret_cast<const float4 *>(row)[q];
            A[4 * q] = x.x; A[4 * q + 1] = x.y; A[4 * q + 2] = x.z; A[4 * q + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 5; q++) A[q] = row[q];
        }
      }
      if (i < P.n) {
        const double dq[3] = {A[0], A[1], A[2]};
#pragma unroll
        for (int a = 0; a < 3; a++)
          dp[a] += (double)c.R[a] * dq[0] + (double)c.R[3 + a] * dq[1] + (double)c.R[6 + a] * dq[2];   // R^T dq
        dr += A[3];
        dop += A[4];
        if constexpr (STAGE) {
#pragma unroll
          for (int ch = 0; ch < CS; ch++)
            if (ch < P.C) fs[ch] += A[5 + ch];
        }
        if (v == cam_view) {
          const double pp[3] = {P.pos[3 * i], P.pos[3 * i + 1], P.pos[3 * i + 2]};
          const double cw = cam_weight(c, P, (size_t)v * P.n + i);
#pragma unroll
          for (int a = 0; a < 3; a++) {
            const double dw = dq[a] * cw;
#pragma unroll
            for (int b = 0; b < 3; b++) cam[3 * a + b] = __builtin_fma(dw, pp[b], cam[3 * a + b]);
            cam[9 + a] += dw;
          }
        }
      }
    }
    if (i < P.n) {
      if (P.cnt) {
        // averaged over the pixels that recorded the sphere (all views of the call)
        uint32_t ct = 0;
        for (int v = vbeg; v < vend; v++) ct += P.cnt[(size_t)v * P.n + i];
        nrm = ct ? 1.0 / (double)ct : 0.0;
#pragma unroll
        for (int a = 0; a < 3; a++) dp[a] *= nrm;
        dr *= nrm;
        dop *= nrm;
      }
      if (P.gscale) put(P.gscale, i, dr, P.accumulate);
      if (P.gop) put(P.gop, i, dop, P.accumulate);
    }
    if (P.gpos) {
      if (i < P.n)
#pragma unroll
        for (int a = 0; a < 3; a++) s_pos[3 * threadIdx.x + a] = (float)dp[a];
      __syncthreads();
      float *out = P.gpos + 3 * (size_t)i0;
      for (int j = threadIdx.x; j < 3 * nb; j += 256) out[j] = P.accumulate ? out[j] + s_pos[j] : s_pos[j];
    }
    if (P.gfeat) {
      if constexpr (STAGE) {
        if (i < P.n)
#pragma unroll
          for (int ch = 0; ch < CS; ch++)
            if (ch < P.C) s_feat[P.C * threadIdx.x + ch] = (float)(fs[ch] * nrm);
        __syncthreads();
        float *out = P.gfeat + (size_t)P.C * i0;
        for (int j = threadIdx.x; j < P.C * nb; j += 256) out[j] = P.accumulate ? out[j] + s_feat[j] : s_feat[j];
      } else if (i < P.n) {
        for (int ch = 0; ch < P.C; ch++) {
          double f = 0;
          for (int v = vbeg; v < vend; v++) f += P.accs[((size_t)v * P.n + i) * S + 5 + ch];
          put(P.gfeat, (size_t)i * P.C + ch, f * nrm, P.accumulate);
        }
      }
    }
    __syncthreads();                           // LDS reuse by the next 256 spheres
  }
  if (cam_view < 0) return;
  const unsigned lane = lane_id(), w = threadIdx.x / WAVE;
#pragma unroll
  for (int q = 0; q < 12; q++) {
    const double t = wave_sum_f64(cam[q]);
    if (lane == 0) s_red[q][w] = t;
  }
  __syncthreads();
  if (threadIdx.x < 12) {
    const int q = threadIdx.x;
    P.cam_part[12 * blockIdx.x + q] = s_red[q][0] + s_red[q][1] + s_red[q][2] + s_red[q][3];
  }
}

// One block: the per-block camera sums of k_sphere_grads (nparts rows of twelve
// doubles) added in a fixed order. With 768 threads (a multiple of twelve),
// thread t reads the doubles e = t + 768 k, all of sum t mod 12: every wave
// load covers one contiguous 512-byte run (a row of twelve per thread touched
// ~48 cache lines per wave load) and the sixteen loads of a pass are
// independent, so they are in flight together. The 768 partial sums then fold
// in LDS by strides of 192, 48 and 12 (each a multiple of twelve).
constexpr int CAMF_THREADS = 768;
constexpr int CAMF_LOADS = 16;

__global__ __launch_bounds__(CAMF_THREADS) void k_cam_final(ProjBwdArgs P, int nparts, int cam_view) {
  __shared__ double s_acc[CAMF_THREADS];
  const int t = (int)threadIdx.x;
  const int ne = 12 * nparts;
  double acc = 0.0;
  for (int e0 = t; e0 < ne; e0 += CAMF_THREADS * CAMF_LOADS) {
    double x[CAMF_LOADS];
#pragma unroll
    for (int k = 0; k < CAMF_LOADS; k++) {
      const int e = e0 + CAMF_THREADS * k;
      x[k] = e < ne ? P.cam_part[e] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < CAMF_LOADS; k++) acc += x[k];
  }
  s_acc[t] = acc;
  __syncthreads();
#pragma unroll
  for (int h = CAMF_THREADS / 4; h >= 12; h /= 4) {
    double s = 0.0;
    if (t < h) s = s_acc[t] + s_acc[t + h] + s_acc[t + 2 * h] + s_acc[t + 3 * h];
    __syncthreads();
    if (t < h) s_acc[t] = s;
    __syncthreads();
  }
  if (t < 12) {
    const double tot = s_acc[t];
    float *o = t < 9 ? (P.gR ? P.gR + 9 * cam_view + t : nullptr) : (P.gt ? P.gt + 3 * cam_view + (t - 9) : nullptr);
    if (o) *o = P.cam_store ? (float)tot : *o + (float)tot;
  }
}

// Camera gradient of view vbeg + blockIdx.y when one call covers several views
// (same sums as above, one view per grid row).
__global__ __launch_bounds__(256) void k_cam_grad_sphere(ViewTable vt, ProjBwdArgs P, int vbeg) {
  __shared__ double s_red[12][4];
  const int v = vbeg + blockIdx.y;
  const int S = P.rs;
  double cam[12];
#pragma unroll
  for (int q = 0; q < 12; q++) cam[q] = 0.0;
  const ViewDev &c = vt.v[v];
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < P.n; i += gridDim.x * blockDim.x) {
    const float *A = P.accs + ((size_t)v * P.n + i) * S;
    const double cw = cam_weight(c, P, (size_t)v * P.n + i);
    const double dq[3] = {A[0] * cw, A[1] * cw, A[2] * cw};
    const double pp[3] = {P.pos[3 * i], P.pos[3 * i + 1], P.pos[3 * i + 2]};
#pragma unroll
    for (int a = 0; a < 3; a++) {
#pragma unroll
      for (int b = 0; b < 3; b++) cam[3 * a + b] = __builtin_fma(dq[a], pp[b], cam[3 * a + b]);
      cam[9 + a] += dq[a];
    }
  }
  const unsigned lane = lane_id(), w = threadIdx.x / WAVE;
#pragma unroll
  for (int q = 0; q < 12; q++) {
    const double t = wave_sum_f64(cam[q]);
    if (lane == 0) s_red[q][w] = t;
  }
  __syncthreads();
  if (threadIdx.x < 12) {
    const int q = threadIdx.x;
    const double t = s_red[q][0] + s_red[q][1] + s_red[q][2] + s_red[q][3];
    if (t != 0.0) {
      if (q < 9 && P.gR) atomicAdd(P.gR + 9 * v + q, (float)t);
      if (q >= 9 && P.gt) atomicAdd(P.gt + 3 * v + (q - 9), (float)t);
    }
  }
}

// Image-map Jacobian J (2x3) at sensor point m and its derivatives dJ[k][a] = dJ_k / dm_a.
__device__ void jacobian_and_derivs(const ViewDev &c, const double m[3], double J[6], double dJ[6][3]) {
#pragma unroll
  for (int k = 0; k < 6; k++)
#pragma unroll
    for (int a = 0; a < 3; a++) dJ[k][a] = 0.0;
  if (c.kind == SPLAT_CAM_PINHOLE) {
    const double fx = c.fx, fy = c.fy;
    const double iz = 1.0 / m[2], iz2 = iz * iz, iz3 = iz2 * iz;
    J[0] = fx * iz; J[1] = 0.0; J[2] = -fx * m[0] * iz2;
    J[3] = 0.0; J[4] = fy * iz; J[5] = -fy * m[1] * iz2;
    dJ[0][2] = -fx * iz2;
    dJ[2][0] = -fx * iz2;
    dJ[2][2] = 2.0 * fx * m[0] * iz3;
    dJ[4][2] = -fy * iz2;
    dJ[5][1] = -fy * iz2;
    dJ[5][2] = 2.0 * fy * m[1] * iz3;
  } else {
    const double kPi = 3.141592653589793;
    const double th_max = (double)c.el_max * (kPi / 180.0), th_min = (double)c.el_min * (kPi / 180.0);
    const double ka = (double)c.W / (2.0 * kPi), kb = (double)c.H / (th_max - th_min);
    const double x = m[0], y = m[1], z = m[2];
    const double rho2 = x * x + y * y, rho = sqrt(rho2), r2 = rho2 + z * z;
    const double rho4 = rho2 * rho2, r4 = r2 * r2;
    J[0] = ka * y / rho2; J[1] = -ka * x / rho2; J[2] = 0.0;
    const double h = 1.0 / (r2 * rho);
    J[3] = kb * x * z * h; J[4] = kb * y * z * h; J[5] = -kb * rho / r2;
    dJ[0][0] = -2.0 * ka * x * y / rho4;
    dJ[0][1] = ka * (x * x - y * y) / rho4;
    dJ[1][0] = ka * (x * x - y * y) / rho4;
    dJ[1][1] = 2.0 * ka * x * y / rho4;
    const double hx = -x * (2.0 * rho2 + r2) / (r4 * rho2 * rho);
    const double hy = -y * (2.0 * rho2 + r2) / (r4 * rho2 * rho);
    const double hz = -2.0 * z / (r4 * rho);
    dJ[3][0] = kb * z * (h + x * hx);
    dJ[3][1] = kb * x * z * hy;
    dJ[3][2] = kb * x * (h + z * hz);
    dJ[4][0] = kb * y * z * hx;
    dJ[4][1] = kb * z * (h + y * hy);
    dJ[4][2] = kb * y * (h + z * hz);
    dJ[5][0] = -kb * x * (r2 - 2.0 * rho2) / (rho * r4);
    dJ[5][1] = -kb * y * (r2 - 2.0 * rho2) / (rho * r4);
    dJ[5][2] = 2.0 * kb * rho * z / r4;
  }
}

// Geometry chain rule of one Gaussian (fp64), views summed.
__device__ __forceinline__ void gauss_prim_grads(const ViewTable &vt, const ProjBwdArgs &P, int vbeg, int vend, int i) {
  double gpos[3] = {0, 0, 0}, gs[3] = {0, 0, 0}, gq[4] = {0, 0, 0, 0}, gop = 0;
  if (P.kind == SPLAT_PRIM_GAUSS2D) {
    const double s = P.scale[i];
    for (int v = vbeg; v < vend; v++) {
      const long long rec = (long long)v * P.n + i;
      if (!rec_live(P.bin, rec)) continue;
      const double *A = P.accg + (size_t)rec * ACC_G;
      gpos[0] += A[0];
      gpos[1] += A[1];
      gs[0] += (A[2] + A[4]) * (-2.0 / (s * s * s));
      gop += A[5];
    }
  } else {
    // forward quantities shared by all views
    const double s[3] = {P.scale[3 * i], P.scale[3 * i + 1], P.scale[3 * i + 2]};
    const double q0[4] = {P.rot[4 * i], P.rot[4 * i + 1], P.rot[4 * i + 2], P.rot[4 * i + 3]};
    const double nq = sqrt(q0[0] * q0[0] + q0[1] * q0[1] + q0[2] * q0[2] + q0[3] * q0[3]);
    const double w = q0[0] / nq, x = q0[1] / nq, y = q0[2] / nq, z = q0[3] / nq;
    double Rq[9];
    Rq[0] = 1.0 - 2.0 * (y * y + z * z); Rq[1] = 2.0 * (x * y - w * z); Rq[2] = 2.0 * (x * z + w * y);
    Rq[3] = 2.0 * (x * y + w * z); Rq[4] = 1.0 - 2.0 * (x * x + z * z); Rq[5] = 2.0 * (y * z - w * x);
    Rq[6] = 2.0 * (x * z - w * y); Rq[7] = 2.0 * (y * z + w * x); Rq[8] = 1.0 - 2.0 * (x * x + y * y);
    double M[9], S3[9];
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++) M[3 * a + b] = Rq[3 * a + b] * s[b];
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++)
        S3[3 * a + b] = M[3 * a] * M[3 * b] + M[3 * a + 1] * M[3 * b + 1] + M[3 * a + 2] * M[3 * b + 2];
    double dS3sum[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
    for (int v = vbeg; v < vend; v++) {
      const long long rec = (long long)v * P.n + i;
      if (!rec_live(P.bin, rec)) continue;
      const ViewDev &c = vt.v[v];
      const double *A = P.accg + (size_t)rec * ACC_G;
      double W[9];
      for (int k = 0; k < 9; k++) W[k] = c.R[k];
      double m[3];
      for (int a = 0; a < 3; a++)
        m[a] = W[3 * a] * (double)P.pos[3 * i] + W[3 * a + 1] * (double)P.pos[3 * i + 1] +
               W[3 * a + 2] * (double)P.pos[3 * i + 2] + (double)c.t[a];
      double J[6], dJm[6][3];
      jacobian_and_derivs(c, m, J, dJm);
      double T[6];
      for (int a = 0; a < 2; a++)
        for (int b = 0; b < 3; b++) T[3 * a + b] = J[3 * a] * W[b] + J[3 * a + 1] * W[3 + b] + J[3 * a + 2] * W[6 + b];
      double TS[6];
      for (int a = 0; a < 2; a++)
        for (int b = 0; b < 3; b++) TS[3 * a + b] = T[3 * a] * S3[b] + T[3 * a + 1] * S3[3 + b] + T[3 * a + 2] * S3[6 + b];
      const double sxx = TS[0] * T[0] + TS[1] * T[1] + TS[2] * T[2];
      const double sxy = TS[0] * T[3] + TS[1] * T[4] + TS[2] * T[5];
      const double syy = TS[3] * T[3] + TS[4] * T[4] + TS[5] * T[5];
      const double det = sxx * syy - sxy * sxy;
      const double Q[4] = {syy / det, -sxy / det, -sxy / det, sxx / det};
      // dL/dQ as a symmetric matrix (the off-diagonal parameter appears twice)
      const double Gq[4] = {A[2], 0.5 * (double)A[3], 0.5 * (double)A[3], A[4]};
      double QG[4], dS2[4];
      QG[0] = Q[0] * Gq[0] + Q[1] * Gq[2]; QG[1] = Q[0] * Gq[1] + Q[1] * Gq[3];
      QG[2] = Q[2] * Gq[0] + Q[3] * Gq[2]; QG[3] = Q[2] * Gq[1] + Q[3] * Gq[3];
      dS2[0] = -(QG[0] * Q[0] + QG[1] * Q[2]); dS2[1] = -(QG[0] * Q[1] + QG[1] * Q[3]);
      dS2[2] = -(QG[2] * Q[0] + QG[3] * Q[2]); dS2[3] = -(QG[2] * Q[1] + QG[3] * Q[3]);
      // Sigma2 = T S3 T^T
      for (int a = 0; a < 3; a++)
        for (int b = 0; b < 3; b++) {
          double acc = 0.0;
          for (int pp = 0; pp < 2; pp++)
            for (int qq = 0; qq < 2; qq++) acc += T[3 * pp + a] * dS2[2 * pp + qq] * T[3 * qq + b];
          dS3sum[3 * a + b] += acc;
        }
      double dT[6];
      for (int a = 0; a < 2; a++)
        for (int b = 0; b < 3; b++) dT[3 * a + b] = 2.0 * (dS2[2 * a] * TS[b] + dS2[2 * a + 1] * TS[3 + b]);
      double dJ[6];
      for (int a = 0; a < 2; a++)
        for (int b = 0; b < 3; b++) dJ[3 * a + b] = dT[3 * a] * W[3 * b] + dT[3 * a + 1] * W[3 * b + 1] + dT[3 * a + 2] * W[3 * b + 2];
      double dm[3];
      for (int a = 0; a < 3; a++) {
        double t = (double)A[0] * J[a] + (double)A[1] * J[3 + a];
        for (int k = 0; k < 6; k++) t += dJ[k] * dJm[k][a];
        dm[a] = t;
      }
      if (c.kind == SPLAT_CAM_SPHERICAL) {
        const double rr = sqrt(m[0] * m[0] + m[1] * m[1] + m[2] * m[2]);
        for (int a = 0; a < 3; a++) dm[a] += (double)A[6] * m[a] / rr;
      }
      for (int a = 0; a < 3; a++) gpos[a] += W[a] * dm[0] + W[3 + a] * dm[1] + W[6 + a] * dm[2];
      gop += A[5];
    }
    // Sigma3 = M M^T, M = Rq diag(s)
    double dM[9], dRq[9];
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++)
        dM[3 * a + b] = 2.0 * (dS3sum[3 * a] * M[b] + dS3sum[3 * a + 1] * M[3 + b] + dS3sum[3 * a + 2] * M[6 + b]);
    for (int a = 0; a < 3; a++)
      for (int b = 0; b < 3; b++) {
        gs[b] += dM[3 * a + b] * Rq[3 * a + b];
        dRq[3 * a + b] = dM[3 * a + b] * s[b];
      }
    double dqn[4];
    dqn[0] = 2.0 * (-z * dRq[1] + y * dRq[2] + z * dRq[3] - x * dRq[5] - y * dRq[6] + x * dRq[7]);
    dqn[1] = 2.0 * (y * dRq[1] + z * dRq[2] + y * dRq[3] - 2.0 * x * dRq[4] - w * dRq[5] + z * dRq[6] + w * dRq[7] -
                    2.0 * x * dRq[8]);
    dqn[2] = 2.0 * (-2.0 * y * dRq[0] + x * dRq[1] + w * dRq[2] + x * dRq[3] + z * dRq[5] - w * dRq[6] + z * dRq[7] -
                    2.0 * y * dRq[8]);
    dqn[3] = 2.0 * (-2.0 * z * dRq[0] - w * dRq[1] + x * dRq[2] + w * dRq[3] - 2.0 * z * dRq[4] + y * dRq[5] +
                    x * dRq[6] + y * dRq[7]);
    const double qn[4] = {w, x, y, z};
    const double dot = qn[0] * dqn[0] + qn[1] * dqn[1] + qn[2] * dqn[2] + qn[3] * dqn[3];
    for (int a = 0; a < 4; a++) gq[a] = (dqn[a] - qn[a] * dot) / nq;
  }
  const int pd = P.kind == SPLAT_PRIM_GAUSS2D ? 2 : 3;
  const int sd = P.kind == SPLAT_PRIM_GAUSS3D ? 3 : 1;
  if (P.gpos)
    for (int a = 0; a < pd; a++) put(P.gpos, (size_t)pd * i + a, gpos[a], P.accumulate);
  if (P.gscale)
    for (int a = 0; a < sd; a++) put(P.gscale, (size_t)sd * i + a, gs[a], P.accumulate);
  if (P.grot && P.kind == SPLAT_PRIM_GAUSS3D)
    for (int a = 0; a < 4; a++) put(P.grot, 4 * (size_t)i + a, gq[a], P.accumulate);
  if (P.gop) put(P.gop, i, gop, P.accumulate);
}

// One thread per Gaussian for the geometry (fp64 chain rule, ~220 VGPRs: two
// waves per SIMD).
__global__ __launch_bounds__(256) void k_proj_bwd_gauss(ViewTable vt, ProjBwdArgs P, int vbeg, int vend) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < P.n) gauss_prim_grads(vt, P, vbeg, vend, i);
}

// Feature gradients of Gaussians ([primitive][channel], the call's pinhole views
// summed), element by element and coalesced. A kernel of their own: inside the
// geometry kernel this stream (fp64 sums in, fp32 gradients out; 768 MB for 2M
// primitives with 32 channels) ran at that kernel's two waves per SIMD.
__global__ __launch_bounds__(256) void k_feat_grads_gauss(ViewTable vt, ProjBwdArgs P, int vbeg, int vend) {
  const size_t plane = (size_t)P.n * P.C;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < plane; e += (size_t)gridDim.x * blockDim.x) {
    double sum = 0;
    for (int v = vbeg; v < vend; v++)
      if (vt.v[v].kind != SPLAT_CAM_SPHERICAL) sum += P.accf[(size_t)v * plane + e];
    put(P.gfeat, e, sum, P.accumulate);
  }
}

template <int CM>
int launch_bwd_cm(const ViewTable &vt, const BwdArgs &A, int kind, int tile_begin, int ntiles, int vbeg, int vend,
                   hipStream_t stream) {
  if (kind == SPLAT_PRIM_SPHERE) {
    if (A.kslot || A.cnt)
      hipLaunchKernelGGL((k_bwd_sphere<CM, true>), dim3(ntiles), dim3(256), 0, stream, vt, A, tile_begin);
    else if (CM <= 4 && A.direct_max > 0)
      hipLaunchKernelGGL((k_bwd_sphere<CM, false, CM <= 4>), dim3(ntiles), dim3(256), 0, stream, vt, A, tile_begin);
    else if (CM <= 3 && A.top_k <= SPH_DENSE_K)
      hipLaunchKernelGGL((k_bwd_sphere_dense<CM <= 3 ? CM : 3>), dim3(ntiles), dim3(256), 0, stream, vt, A,
                         tile_begin);
    else
      hipLaunchKernelGGL((k_bwd_sphere<CM, false>), dim3(ntiles), dim3(256), 0, stream, vt, A, tile_begin);
  } else {
    // one launch per run of consecutive views of one kind, over that run's
    // tiles only; with both kinds present the camera views run on the side
    // stream, the spherical views (dispatched first) on the caller's
    bool has_pin = false, has_sph = false;
    for (int v = vbeg; v < vend; v++) (vt.v[v].kind == SPLAT_CAM_SPHERICAL ? has_sph : has_pin) = true;
    hipStream_t side = stream;
    const bool fork = has_pin && has_sph && !A.serial_views;
    if (fork) {
      const int rc = side_begin(stream, &side);
      if (rc != SPLAT_OK) return rc;
    }
    for (int pass = 0; pass < 2; pass++) {
      for (int v0 = vbeg; v0 < vend;) {
        const int kind0 = vt.v[v0].kind;
        int v1 = v0 + 1;
        while (v1 < vend && vt.v[v1].kind == kind0) v1++;
        const int t0 = vt.v[v0].tile_off, t1 = v1 < vt.n ? vt.v[v1].tile_off : vt.total_tiles;
        if (t1 > t0) {
          if (pass == 0 && kind0 == SPLAT_CAM_SPHERICAL)
            hipLaunchKernelGGL((k_bwd_split<1, true>), dim3(t1 - t0), dim3(1024), 0, stream, vt, A, t0);
          else if (pass == 1 && kind0 != SPLAT_CAM_SPHERICAL && split_pinhole<CM>(t1 - t0))
            hipLaunchKernelGGL((k_bwd_split<CM <= 4 ? CM : 4, false>), dim3(t1 - t0), dim3(1024), 0, side, vt, A, t0);
          else if (pass == 1 && kind0 != SPLAT_CAM_SPHERICAL)
            hipLaunchKernelGGL(k_bwd_alpha<CM>, dim3(t1 - t0), dim3(256), 0, side, vt, A, t0);
        }
        v0 = v1;
      }
    }
    if (fork) return side_end(stream, side);
  }
  return SPLAT_OK;
}

}  // namespace

size_t bwd_workspace_bytes(long long nrec, int C) { return acc_bytes(nrec, C); }

int launch_render_bwd(const ViewTable &vt, int vbeg, int vend, BwdArgs A, const splat_prims *pr, BinArrays bin,
                      const splat_grads *gr, hipStream_t stream) {
  // accumulator rows of the requested views only (spheres: one row of 5 + C
  // values per record; Gaussians: ACC_G geometric values and C features)
  const bool sph = pr->kind == SPLAT_PRIM_SPHERE;
  const long long r0 = (long long)vbeg * A.n, r1 = (long long)vend * A.n;
  ZeroRanges z{};
  if (gr->sums_cleared) {
    // the forward before this call cleared every sum of the workspace
  } else if (sph) {
    // fp32 rows of a multiple of four floats: cleared as doubles
    z.d0 = reinterpret_cast<double *>(A.accs + r0 * A.rs);
    z.nd0 = (r1 - r0) * A.rs / 2;
    if (A.kslot) {
      z.d1 = A.kslot + (size_t)vbeg * SPLAT_K_SLOTS * 4;
      z.nd1 = (long long)(vend - vbeg) * SPLAT_K_SLOTS * 4;
    }
    if (A.cnt) {
      z.u0 = A.cnt + r0;
      z.nu0 = r1 - r0;
    }
  } else {
    z.d0 = A.accg + r0 * ACC_G;
    z.nd0 = (r1 - r0) * ACC_G;
    z.d1 = A.accf + r0 * A.C;
    z.nd1 = (r1 - r0) * A.C;
  }
  // one view, overwritten: the camera pass below stores R and t outright
  const bool cam_store = sph && !gr->accumulate && vt.n == 1;
  if (!gr->accumulate && !cam_store) {
    z.f0 = gr->cam_R;
    z.nf0 = gr->cam_R ? 9ll * vt.n : 0;
    z.f1 = gr->cam_t;
    z.nf1 = gr->cam_t ? 3ll * vt.n : 0;
  }

  const long long nz = z.nd0 + z.nd1 + z.nf0 + z.nf1 + z.nu0;
  if (nz > 0)
    hipLaunchKernelGGL(k_zero, dim3((unsigned)min((nz + 255) / 256, (long long)ZERO_GRID)), dim3(256), 0, stream, z);
  SPLAT_LAUNCH_CHECK();
  const int tile_begin = vt.v[vbeg].tile_off;
  const int tile_end = vend < vt.n ? vt.v[vend].tile_off : vt.total_tiles;
  const int ntiles = tile_end - tile_begin;
  if (ntiles > 0) {
    int rc = SPLAT_OK;
    switch (channel_bucket(A.C)) {
      case 1: rc = launch_bwd_cm<1>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 2: rc = launch_bwd_cm<2>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 3: rc = launch_bwd_cm<3>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 4: rc = launch_bwd_cm<4>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 8: rc = launch_bwd_cm<8>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 16: rc = launch_bwd_cm<16>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      case 32: rc = launch_bwd_cm<32>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
      default: rc = launch_bwd_cm<64>(vt, A, pr->kind, tile_begin, ntiles, vbeg, vend, stream); break;
    }
    if (rc != SPLAT_OK) return rc;
    if (sph && A.kslot)
      hipLaunchKernelGGL(k_cam_K_final, dim3(1), dim3(256), 0, stream, A.kslot, gr->cam_K, vbeg, vend,
                         gr->accumulate);
    SPLAT_LAUNCH_CHECK();
  }
  ProjBwdArgs P;
  P.kind = pr->kind; P.n = pr->n; P.C = A.C;
  P.pos = pr->pos; P.scale = pr->scale; P.rot = pr->rot;
  P.bin = bin; P.accg = A.accg; P.accf = A.accf; P.cam_part = A.cam_part;
  P.accs = A.accs; P.rs = A.rs;
  P.aux = A.aux; P.cnt = sph ? A.cnt : nullptr;
  P.gpos = gr->pos; P.gscale = gr->scale; P.grot = gr->rot; P.gop = gr->opacity; P.gfeat = gr->feat;
  P.gR = gr->cam_R; P.gt = gr->cam_t;
  P.accumulate = gr->accumulate;
  P.cam_store = cam_store ? 1 : 0;
  if (pr->n > 0) {
    dim3 grid((pr->n + 255) / 256);
    if (sph) {
      // a bounded grid keeps the camera atomics few; one view: camera in the same pass
      const bool cam = gr->cam_R || gr->cam_t;
      const unsigned nb = (unsigned)min((pr->n + 255) / 256, SPLAT_CAM_BLOCKS);
      const int cam_view = cam && vend - vbeg == 1 ? vbeg : -1;
      if (channel_bucket(A.C) <= 4) {
        switch (channel_bucket(A.C)) {
          case 1: hipLaunchKernelGGL(k_sphere_grads<1>, dim3(nb), dim3(256), 0, stream, vt, P, vbeg, vend, cam_view); break;
          case 2: hipLaunchKernelGGL(k_sphere_grads<2>, dim3(nb), dim3(256), 0, stream, vt, P, vbeg, vend, cam_view); break;
          case 3: hipLaunchKernelGGL(k_sphere_grads<3>, dim3(nb), dim3(256), 0, stream, vt, P, vbeg, vend, cam_view); break;
          default: hipLaunchKernelGGL(k_sphere_grads<4>, dim3(nb), dim3(256), 0, stream, vt, P, vbeg, vend, cam_view); break;
        }
      } else {
        hipLaunchKernelGGL(k_sphere_grads<8>, dim3(nb), dim3(256), 0, stream, vt, P, vbeg, vend, cam_view);
      }
      if (cam_view >= 0) hipLaunchKernelGGL(k_cam_final, dim3(1), dim3(CAMF_THREADS), 0, stream, P, (int)nb, cam_view);
      if (cam && vend - vbeg > 1)
        hipLaunchKernelGGL(k_cam_grad_sphere, dim3(min(nb, 512u), vend - vbeg), dim3(256), 0, stream, vt, P, vbeg);
    }
    else {
      hipLaunchKernelGGL(k_proj_bwd_gauss, grid, dim3(256), 0, stream, vt, P, vbeg, vend);
      if (P.gfeat) {
        const long long ne = (long long)pr->n * A.C;
        const unsigned fb = (unsigned)min((ne + 255) / 256, 8192ll);
        if (ne > 0) hipLaunchKernelGGL(k_feat_grads_gauss, dim3(fb), dim3(256), 0, stream, vt, P, vbeg, vend);
      }
    }
    SPLAT_LAUNCH_CHECK();
  }
  return SPLAT_OK;
}
