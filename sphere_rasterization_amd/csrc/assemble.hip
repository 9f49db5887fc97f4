// Per-frame parameter assembly, one fused kernel per direction.
//
// NuRec's profiling page ("Fusing small kernels and removing synchronizations")
// found the per-frame interpolate step of collect_gaussian_parameters spread over
// many tiny kernels and memory operations, and fused it into one. What is
// interpolated is not on the page; here every primitive carries its centre and
// its rotation quaternion at keyframe times, and a frame at time t blends the two
// bracketing keyframes with weight w: centre (1 - w) c_k + w c_k1, rotation
// (1 - w) q_k + w s q_k1 with s = -1 when q_k . q_k1 < 0 (the shorter arc; the
// projection normalises the quaternion).
//
// The work is a pure stream: per primitive 2 x 28 bytes read and 28 written
// forward, so the kernels are HBM-bound. One thread per primitive: the rotation
// as one 16-byte access (the sign needs the whole quaternion), the centre as three
// 4-byte accesses (contiguous across the wave's lanes).
#include "splat_internal.h"

namespace {

struct AsmArgs {
  const float *p0, *p1;       // key centres of frames k, k1 ([n][3] each)
  const float *q0, *q1;       // key rotations ([n][4] each)
  float *pos, *rot;           // outputs (either may be NULL)
  long long n;
  float w;                    // weight of frame k1
};

__global__ __launch_bounds__(256) void k_assemble(AsmArgs a) {
  const float u = 1.0f - a.w, w = a.w;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < a.n;
       i += (long long)gridDim.x * blockDim.x) {
    if (a.rot) {
      const float4 x = reinterpret_cast<const float4 *>(a.q0)[i];
      const float4 y = reinterpret_cast<const float4 *>(a.q1)[i];
      const float dot = x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
      const float ws = dot < 0.0f ? -w : w;
      reinterpret_cast<float4 *>(a.rot)[i] =
          make_float4(u * x.x + ws * y.x, u * x.y + ws * y.y, u * x.z + ws * y.z, u * x.w + ws * y.w);
    }
    if (a.pos) {
#pragma unroll
      for (int c = 0; c < 3; c++) a.pos[3 * i + c] = u * a.p0[3 * i + c] + w * a.p1[3 * i + c];
    }
  }
}

struct AsmBwdArgs {
  const float *q0, *q1;       // key rotations of frames k, k1
  const float *dpos, *drot;   // upstream gradients ([n][3], [n][4]; either may be NULL)
  float *gp0, *gp1;           // key-centre gradients of frames k, k1 (added into)
  float *gq0, *gq1;           // key-rotation gradients (added into)
  long long n;
  float w;
  int same;                   // k == k1 (t clamped to an end frame, or one keyframe)
};

__global__ __launch_bounds__(256) void k_assemble_bwd(AsmBwdArgs a) {
  const float u = 1.0f - a.w, w = a.w;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < a.n;
       i += (long long)gridDim.x * blockDim.x) {
    if (a.drot && a.gq0) {
      const float4 g = reinterpret_cast<const float4 *>(a.drot)[i];
      float4 *o0 = reinterpret_cast<float4 *>(a.gq0) + i;
      const float4 a0 = *o0;
      if (a.same) {
        *o0 = make_float4(a0.x + g.x, a0.y + g.y, a0.z + g.z, a0.w + g.w);
      } else {
        const float4 x = reinterpret_cast<const float4 *>(a.q0)[i];
        const float4 y = reinterpret_cast<const float4 *>(a.q1)[i];
        const float dot = x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        const float ws = dot < 0.0f ? -w : w;
        float4 *o1 = reinterpret_cast<float4 *>(a.gq1) + i;
        const float4 a1 = *o1;
        *o0 = make_float4(a0.x + u * g.x, a0.y + u * g.y, a0.z + u * g.z, a0.w + u * g.w);
        *o1 = make_float4(a1.x + ws * g.x, a1.y + ws * g.y, a1.z + ws * g.z, a1.w + ws * g.w);
      }
    }
    if (a.dpos && a.gp0) {
#pragma unroll
      for (int c = 0; c < 3; c++) {
        const float g = a.dpos[3 * i + c];
        if (a.same) {
          a.gp0[3 * i + c] += g;
        } else {
          a.gp0[3 * i + c] += u * g;
          a.gp1[3 * i + c] += w * g;
        }
      }
    }
  }
}

unsigned grid_for(long long items) {
  const long long b = (items + 255) / 256;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

int launch_assemble(const float *key_pos, const float *key_rot, int k, int k1, float w, long long n, float *pos,
                    float *rot, hipStream_t stream) {
  AsmArgs a;
  a.p0 = key_pos ? key_pos + (size_t)k * 3 * n : nullptr;
  a.p1 = key_pos ? key_pos + (size_t)k1 * 3 * n : nullptr;
  a.q0 = key_rot ? key_rot + (size_t)k * 4 * n : nullptr;
  a.q1 = key_rot ? key_rot + (size_t)k1 * 4 * n : nullptr;
  a.pos = key_pos ? pos : nullptr;
  a.rot = key_rot ? rot : nullptr;
  a.n = n;
  a.w = w;
  if (n == 0 || (!a.rot && !a.pos)) return SPLAT_OK;
  hipLaunchKernelGGL(k_assemble, dim3(grid_for(n)), dim3(256), 0, stream, a);
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}

int launch_assemble_bwd(const float *key_rot, int k, int k1, float w, long long n, const float *d_pos,
                        const float *d_rot, float *d_key_pos, float *d_key_rot, hipStream_t stream) {
  AsmBwdArgs a;
  a.q0 = key_rot ? key_rot + (size_t)k * 4 * n : nullptr;
  a.q1 = key_rot ? key_rot + (size_t)k1 * 4 * n : nullptr;
  a.dpos = d_pos;
  a.drot = d_rot;
  a.gp0 = d_key_pos ? d_key_pos + (size_t)k * 3 * n : nullptr;
  a.gp1 = d_key_pos ? d_key_pos + (size_t)k1 * 3 * n : nullptr;
  a.gq0 = d_key_rot ? d_key_rot + (size_t)k * 4 * n : nullptr;
  a.gq1 = d_key_rot ? d_key_rot + (size_t)k1 * 4 * n : nullptr;
  a.n = n;
  a.w = w;
  a.same = k == k1;
  if (n == 0 || (!(d_rot && d_key_rot) && !(d_pos && d_key_pos))) return SPLAT_OK;
  hipLaunchKernelGGL(k_assemble_bwd, dim3(grid_for(n)), dim3(256), 0, stream, a);
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}
