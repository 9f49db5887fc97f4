// Measurement kernels for the figures a roofline needs on the machine at
// hand: the shader clock under full VALU load (with the single-issue fp32 FMA
// rate it sustains), the HBM bandwidth of a plain copy, and the LDS bandwidth
// of broadcast reads in the compositors' pattern (each 16-lane group of a wave
// reads one 16-byte slot). The benchmark reports every stage against these as
// well as against the datasheet peaks. Nothing here is part of the
// rasterizer's path.
#include <hip/hip_runtime.h>

#include "splat_peaks.h"

namespace {

constexpr int PK_THREADS = 256;
constexpr int PK_CHAINS = 8;        // independent FMA chains per lane
constexpr int PK_LDS_SLOTS = 1024;  // 16 KiB of float4
constexpr int PK_LDS_UNROLL = 8;

__device__ __forceinline__ float fma_t(float x, float m, float a) { return __builtin_fmaf(x, m, a); }
__device__ __forceinline__ double fma_t(double x, double m, double a) { return __builtin_fma(x, m, a); }

// Every lane runs PK_CHAINS independent FMA chains (fp32 or fp64) of `iters`
// steps between two reads of the shader-clock counter and of the constant-rate
// wall clock; lane 0 of each workgroup's first wave stores the two differences.
template <typename T>
__global__ __launch_bounds__(PK_THREADS) void k_peak_valu(unsigned long long *clk, float *sink, int iters) {
  T x[PK_CHAINS];
#pragma unroll
  for (int j = 0; j < PK_CHAINS; j++) x[j] = (T)(threadIdx.x + j) * (T)1e-3;
  const T m = (T)0.999999, a = (T)1e-7;
  const unsigned long long c0 = clock64(), w0 = wall_clock64();
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int j = 0; j < PK_CHAINS; j++) x[j] = fma_t(x[j], m, a);
  }
  const unsigned long long c1 = clock64(), w1 = wall_clock64();
  T s = (T)0;
#pragma unroll
  for (int j = 0; j < PK_CHAINS; j++) s += x[j];
  sink[(size_t)blockIdx.x * PK_THREADS + threadIdx.x] = (float)s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = c1 - c0;
    clk[2 * blockIdx.x + 1] = w1 - w0;
  }
}

// dst = src over n4 16-byte words, four loads in flight per thread per round.
__global__ __launch_bounds__(PK_THREADS) void k_peak_copy(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                          size_t n4) {
  const size_t stride = (size_t)gridDim.x * PK_THREADS;
  size_t i = (size_t)blockIdx.x * PK_THREADS + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n4; i += stride) dst[i] = src[i];
}

// Broadcast LDS reads: per instruction the four 16-lane groups of a wave read
// four different 16-byte slots. Two integer adds per read keep the data live.
__global__ __launch_bounds__(PK_THREADS) void k_peak_lds(unsigned *sink, int iters) {
  __shared__ uint4 s[PK_LDS_SLOTS];
  for (int i = threadIdx.x; i < PK_LDS_SLOTS; i += PK_THREADS) s[i] = make_uint4(i, 3u * i, 5u * i, 7u * i);
  __syncthreads();
  const int g = (int)((threadIdx.x >> 4) & 3u), w = (int)(threadIdx.x >> 6);
  unsigned a = 0u, b = 0u;
  for (int k = 0; k < iters; k++) {
#pragma unroll
    for (int u = 0; u < PK_LDS_UNROLL; u++) {
      const uint4 v = s[(k * 64 + u * 8 + g * 2 + w * 256) & (PK_LDS_SLOTS - 1)];
      a = a + v.x + v.y;
      b = b + v.z + v.w;
    }
  }
  sink[(size_t)blockIdx.x * PK_THREADS + threadIdx.x] = a ^ b;
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : -2; }

}  // namespace

extern "C" {

int splat_peaks_valu(unsigned long long *clk, float *sink, int blocks, int iters, hipStream_t stream) {
  if (!clk || !sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(k_peak_valu<float>, dim3(blocks), dim3(PK_THREADS), 0, stream, clk, sink, iters);
  return launch_status();
}

int splat_peaks_valu64(unsigned long long *clk, float *sink, int blocks, int iters, hipStream_t stream) {
  if (!clk || !sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(k_peak_valu<double>, dim3(blocks), dim3(PK_THREADS), 0, stream, clk, sink, iters);
  return launch_status();
}

int splat_peaks_copy(const void *src, void *dst, size_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || blocks <= 0 || bytes % 16 != 0) return -1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(k_peak_copy, dim3(blocks), dim3(PK_THREADS), 0, stream, (const float4 *)src, (float4 *)dst,
                     bytes / 16);
  return launch_status();
}

int splat_peaks_lds(unsigned *sink, int blocks, int iters, hipStream_t stream) {
  if (!sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(k_peak_lds, dim3(blocks), dim3(PK_THREADS), 0, stream, sink, iters);
  return launch_status();
}

int splat_peaks_wall_clock_khz(int device, int *khz) {
  if (!khz) return -1;
  return hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, device) == hipSuccess ? 0 : -2;
}

int splat_peaks_lds_bytes_per_iter(void) { return PK_LDS_UNROLL * 16; }

int splat_peaks_fma_per_iter(void) { return PK_CHAINS; }

}  // extern "C"
