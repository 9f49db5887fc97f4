// Binning to 16x16 tiles and the per-tile depth sort.
//
// Pulsar appendix B.1.1 sorts spheres by their earliest possible intersection
// depth so that drawing can stop early; B.1.2 works on 16x16 pixel blocks.
// Here every (tile, record) overlap becomes one 64-bit key
//   (global tile << 32) | fp32 bits of the depth
// (depths are positive, so their bits order like the values), the pairs are
// emitted in record order and sorted with a stable LSD radix sort, which leaves
// each tile's list contiguous and ordered by (depth, record index).
//
// Pipeline (all on one stream, no host synchronisation):
//   k_scan_reduce / k_scan_top / k_emit   exclusive scan of pair counts, emit
//   per 8-bit digit: k_radix_hist, k_radix_scan, k_radix_scatter
//   k_fill + k_ranges                     per-tile [start, end)
// The pair count lives on the device; kernels are sized by the capacity and
// blocks past the live count exit at once.
#include "splat_internal.h"

namespace {

constexpr int SCAN_BLOCK = 256;
constexpr int SCAN_ITEMS = 1;
constexpr int SCAN_CHUNK = SCAN_BLOCK * SCAN_ITEMS;   // records per scan block
constexpr int SORT_BLOCK = 256;
constexpr int SORT_ROUNDS = 8;
constexpr int SORT_CHUNK = SORT_BLOCK * SORT_ROUNDS;   // pairs per sort block (many blocks per CU)
constexpr int RADIX = 256;

// Block-wide exclusive scan of one uint32 per thread (256 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ uint32_t block_exclusive_scan(uint32_t x, uint32_t *total) {
  __shared__ uint32_t s_w[SCAN_BLOCK / WAVE];
  unsigned lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  // wave inclusive scan with shuffles
  uint32_t inc = x;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    uint32_t y = __shfl_up(inc, d, WAVE);
    if (lane >= (unsigned)d) inc += y;
  }
  if (lane == WAVE - 1) s_w[w] = inc;
  __syncthreads();
  uint32_t wbase = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < SCAN_BLOCK / WAVE; k++) {
    uint32_t t = s_w[k];
    if ((unsigned)k < w) wbase += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wbase + inc - x;
}

// ---- pair-count scan -------------------------------------------------------

__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_reduce(const uint32_t *counts, long long nrec, uint32_t *block_sums) {
  long long base = (long long)blockIdx.x * SCAN_CHUNK;
  uint32_t s = 0;
#pragma unroll
  for (int r = 0; r < SCAN_ITEMS; r++) {
    long long k = base + r * SCAN_BLOCK + threadIdx.x;
    if (k < nrec) s += counts[k];
  }
  uint32_t tot;
  block_exclusive_scan(s, &tot);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
}

// Single workgroup: exclusive scan of the block sums in place, total and overflow.
// Each thread owns TOP_ITEMS consecutive sums per round (serial scan in registers).
constexpr int TOP_ITEMS = 16;
__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_top(uint32_t *block_sums, int nblocks, long long capacity,
                                                          int64_t *num_pairs, int32_t *overflow, uint32_t *live) {
  unsigned long long carry = 0;
  for (int base = 0; base < nblocks; base += SCAN_BLOCK * TOP_ITEMS) {
    const int k0 = base + (int)threadIdx.x * TOP_ITEMS;
    uint32_t x[TOP_ITEMS];
    uint32_t s = 0;
#pragma unroll
    for (int r = 0; r < TOP_ITEMS; r++) {
      x[r] = k0 + r < nblocks ? block_sums[k0 + r] : 0u;
      s += x[r];
    }
    uint32_t tot;
    uint32_t ex = block_exclusive_scan(s, &tot);
    uint32_t run = (uint32_t)carry + ex;
#pragma unroll
    for (int r = 0; r < TOP_ITEMS; r++) {
      if (k0 + r < nblocks) block_sums[k0 + r] = run;
      run += x[r];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) {
    *num_pairs = (int64_t)carry;
    int of = carry > (unsigned long long)capacity ? 1 : 0;
    *overflow = of;
    *live = of ? 0u : (uint32_t)carry;
  }
}

// Re-scan each block's counts with its base offset and write the pairs.
__global__ __launch_bounds__(SCAN_BLOCK) void k_emit(ViewTable vt, int n, const BinRec *bin, const uint32_t *counts,
                                                      const uint32_t *block_sums, const int32_t *overflow,
                                                      uint64_t *keys, uint32_t *vals) {
  if (*overflow) return;
  long long nrec = (long long)vt.n * n;
  long long base = (long long)blockIdx.x * SCAN_CHUNK + (long long)threadIdx.x * SCAN_ITEMS;
  uint32_t c[SCAN_ITEMS];
  uint32_t s = 0;
#pragma unroll
  for (int r = 0; r < SCAN_ITEMS; r++) {
    long long k = base + r;
    c[r] = k < nrec ? counts[k] : 0u;
    s += c[r];
  }
  uint32_t tot;
  uint32_t off = block_sums[blockIdx.x] + block_exclusive_scan(s, &tot);
#pragma unroll 1
  for (int r = 0; r < SCAN_ITEMS; r++) {
    long long k = base + r;
    if (c[r] == 0) continue;
    int view = (int)(k / n);
    const ViewDev &cv = vt.v[view];
    BinRec b = bin[k];
    uint64_t lo = (uint64_t)b.key;
    uint32_t o = off;
#pragma unroll 1
    for (int ty = b.ty0; ty <= b.ty1; ty++) {
      int tx = b.tx0;
#pragma unroll 1
      for (int a = 0; a < b.ntx; a++) {
        uint64_t gt = (uint64_t)(cv.tile_off + ty * cv.TW + tx);
        keys[o] = (gt << 32) | lo;
        vals[o] = (uint32_t)k;
        o++;
        if (++tx == cv.TW) tx = 0;
      }
    }
    off += c[r];
  }
}

// ---- LSD radix sort, one 8-bit digit per pass --------------------------------

// Digit histogram of each chunk, stored digit-major: hist[d * nblocks + block].
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_hist(const uint64_t *keys, const uint32_t *live,
                                                            const int32_t *overflow, int shift, int nblocks,
                                                            uint32_t *hist) {
  __shared__ uint32_t s_h[RADIX];
  uint32_t P = *overflow ? 0u : *live;
  long long base = (long long)blockIdx.x * SORT_CHUNK;
  if (base >= (long long)P) return;      // past the live pairs: nobody reads this column
  s_h[threadIdx.x] = 0;
  __syncthreads();
  const unsigned lane = threadIdx.x & (WAVE - 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  uint64_t kr[SORT_ROUNDS];
#pragma unroll
  for (int r = 0; r < SORT_ROUNDS; r++) {
    long long i = base + r * SORT_BLOCK + threadIdx.x;
    kr[r] = i < (long long)P ? keys[i] : 0ull;
  }
#pragma unroll
  for (int r = 0; r < SORT_ROUNDS; r++) {
    // one LDS add per distinct digit of the wave (few distinct values are common)
    const bool valid = base + r * SORT_BLOCK + threadIdx.x < (long long)P;
    const unsigned d = (unsigned)(kr[r] >> shift) & (RADIX - 1);
    uint64_t peers = ballot64(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = ballot64(bit);
      peers &= bit ? m : ~m;
    }
    if (valid && (peers & below) == 0) atomicAdd(&s_h[d], (uint32_t)__popcll(peers));
  }
  __syncthreads();
  hist[(size_t)threadIdx.x * nblocks + blockIdx.x] = s_h[threadIdx.x];
}

// One workgroup per digit: exclusive scan of its row over the chunks, row total out.
__global__ __launch_bounds__(SCAN_BLOCK) void k_radix_scan(uint32_t *hist, int nblocks, uint32_t *digit_total,
                                                            const uint32_t *live, const int32_t *overflow) {
  uint32_t *row = hist + (size_t)blockIdx.x * nblocks;
  const uint32_t P = *overflow ? 0u : *live;
  const int nlive = (int)((P + SORT_CHUNK - 1) / SORT_CHUNK);
  nblocks = nlive < nblocks ? nlive : nblocks;
  __shared__ uint32_t s_carry;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < nblocks; base += SCAN_BLOCK) {
    int k = base + threadIdx.x;
    uint32_t x = k < nblocks ? row[k] : 0u;
    uint32_t tot;
    uint32_t ex = block_exclusive_scan(x, &tot);
    uint32_t carry = s_carry;
    if (k < nblocks) row[k] = carry + ex;
    __syncthreads();
    if (threadIdx.x == 0) s_carry = carry + tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) digit_total[blockIdx.x] = s_carry;
}

// Stable scatter of one chunk. Ranks inside a wave come from 8 ballots (lanes with
// equal digits), across waves and rounds from LDS counters; the chunk is reordered
// by digit in LDS, then each digit's run is written to its global slot.
__global__ __launch_bounds__(SORT_BLOCK) void k_radix_scatter(const uint64_t *kin, const uint32_t *vin,
                                                               uint64_t *kout, uint32_t *vout,
                                                               const uint32_t *hist, const uint32_t *digit_total,
                                                               const uint32_t *live, const int32_t *overflow,
                                                               int shift, int nblocks) {
  __shared__ uint64_t s_key[SORT_CHUNK];
  __shared__ uint32_t s_val[SORT_CHUNK];
  __shared__ uint32_t s_gbase[RADIX];   // global output start of digit d for this chunk
  __shared__ uint32_t s_lstart[RADIX];  // chunk-local start of digit d
  __shared__ uint32_t s_run[RADIX];     // digit d items placed so far
  __shared__ uint32_t s_wcnt[SORT_BLOCK / WAVE][RADIX];
  if (*overflow) return;
  uint32_t P = *live;
  long long base = (long long)blockIdx.x * SORT_CHUNK;
  if (base >= (long long)P) return;
  int cnt = (int)min((long long)SORT_CHUNK, (long long)P - base);
  const unsigned tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;

  // digit totals -> exclusive digit bases (one digit per thread)
  uint32_t dt = digit_total[tid];
  uint32_t tot;
  uint32_t dbase = block_exclusive_scan(dt, &tot);
  const int nlive = (int)((P + SORT_CHUNK - 1) / SORT_CHUNK);
  uint32_t mine = hist[(size_t)tid * nblocks + blockIdx.x];
  uint32_t next = (int)blockIdx.x + 1 < nlive ? hist[(size_t)tid * nblocks + blockIdx.x + 1] : dt;
  uint32_t lcount = next - mine;
  s_gbase[tid] = dbase + mine;
  s_lstart[tid] = block_exclusive_scan(lcount, &tot);
  s_run[tid] = 0;
#pragma unroll
  for (int k = 0; k < SORT_BLOCK / WAVE; k++) s_wcnt[k][tid] = 0;
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (WAVE - lane));
  uint64_t keys_r[SORT_ROUNDS];
  uint32_t vals_r[SORT_ROUNDS];
#pragma unroll
  for (int r = 0; r < SORT_ROUNDS; r++) {        // every load in flight before ranking
    const int idx = r * SORT_BLOCK + (int)tid;
    keys_r[r] = idx < cnt ? kin[base + idx] : 0ull;
    vals_r[r] = idx < cnt ? vin[base + idx] : 0u;
  }
#pragma unroll
  for (int r = 0; r < SORT_ROUNDS; r++) {
    int idx = r * SORT_BLOCK + (int)tid;
    bool valid = idx < cnt;
    uint64_t key = keys_r[r];
    uint32_t val = vals_r[r];
    unsigned d = (unsigned)(key >> shift) & (RADIX - 1);
    uint64_t peers = ballot64(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
      bool bit = (d >> b) & 1u;
      uint64_t m = ballot64(bit);
      peers &= bit ? m : ~m;
    }
    unsigned rank = __popcll(peers & below);
    if (valid && rank == 0) s_wcnt[w][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      uint32_t off = s_run[d] + rank;
      for (unsigned k = 0; k < w; k++) off += s_wcnt[k][d];
      uint32_t pos = s_lstart[d] + off;
      s_key[pos] = key;
      s_val[pos] = val;
    }
    __syncthreads();
    uint32_t add = 0;
#pragma unroll
    for (int k = 0; k < SORT_BLOCK / WAVE; k++) {
      add += s_wcnt[k][tid];
      s_wcnt[k][tid] = 0;
    }
    s_run[tid] += add;
    __syncthreads();
  }
  for (int i = (int)tid; i < cnt; i += SORT_BLOCK) {
    uint64_t key = s_key[i];
    unsigned d = (unsigned)(key >> shift) & (RADIX - 1);
    uint32_t g = s_gbase[d] + (uint32_t)i - s_lstart[d];
    kout[g] = key;
    vout[g] = s_val[i];
  }
}

// ---- tile ranges -------------------------------------------------------------

__global__ void k_fill_u32(uint32_t *p, long long n, uint32_t v) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void k_ranges(const uint64_t *keys, const uint32_t *live, const int32_t *overflow,
                                                 uint32_t *ranges) {
  if (*overflow) return;
  uint32_t P = *live;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)P) return;
  uint32_t t = (uint32_t)(keys[i] >> 32);
  if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * (size_t)t] = (uint32_t)i;
  if (i == (long long)P - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * (size_t)t + 1] = (uint32_t)(i + 1);
}

struct SortWs {
  uint64_t *alt_keys;
  uint32_t *alt_vals;
  uint32_t *block_sums;
  uint32_t *hist;
  uint32_t *digit_total;
  uint32_t *live;
  size_t bytes;
};

SortWs sort_ws_layout(void *base, long long nrec, long long capacity) {
  SortWs w;
  char *p = (char *)base;
  long long nscan = (nrec + SCAN_CHUNK - 1) / SCAN_CHUNK;
  long long nsort = (capacity + SORT_CHUNK - 1) / SORT_CHUNK;
  if (nsort < 1) nsort = 1;
  w.alt_keys = (uint64_t *)p;  p += proj_align(sizeof(uint64_t) * (size_t)capacity);
  w.alt_vals = (uint32_t *)p;  p += proj_align(sizeof(uint32_t) * (size_t)capacity);
  w.block_sums = (uint32_t *)p; p += proj_align(sizeof(uint32_t) * (size_t)(nscan + 1));
  w.hist = (uint32_t *)p;      p += proj_align(sizeof(uint32_t) * (size_t)RADIX * (size_t)nsort);
  w.digit_total = (uint32_t *)p; p += proj_align(sizeof(uint32_t) * RADIX);
  w.live = (uint32_t *)p;      p += proj_align(sizeof(uint32_t) * 4);
  w.bytes = (size_t)(p - (char *)base);
  return w;
}

}  // namespace

size_t sort_workspace_bytes(long long nrec, long long capacity) {
  return sort_ws_layout(nullptr, nrec, capacity).bytes;
}

int sort_key_bits(int total_tiles) {
  int tb = 1;
  while ((1ll << tb) < (long long)total_tiles) tb++;
  return 32 + tb;
}

int launch_bin_sort(const ViewTable &vt, int n, const void *proj, const uint32_t *counts, long long capacity,
                    uint64_t *keys, uint32_t *vals, uint32_t *ranges, int64_t *num_pairs, int32_t *overflow,
                    void *workspace, hipStream_t stream) {
  long long nrec = (long long)vt.n * n;
  SortWs ws = sort_ws_layout(workspace, nrec, capacity);
  ProjLayout L = proj_layout(const_cast<void *>(proj), nrec);
  int nscan = (int)((nrec + SCAN_CHUNK - 1) / SCAN_CHUNK);
  int nsort = (int)((capacity + SORT_CHUNK - 1) / SORT_CHUNK);
  if (nsort < 1) nsort = 1;
  int passes = (sort_key_bits(vt.total_tiles) + 7) / 8;
  // emit into the buffer that makes the last pass land in the caller's arrays
  uint64_t *k_a = (passes % 2 == 0) ? keys : ws.alt_keys;
  uint32_t *v_a = (passes % 2 == 0) ? vals : ws.alt_vals;
  uint64_t *k_b = (passes % 2 == 0) ? ws.alt_keys : keys;
  uint32_t *v_b = (passes % 2 == 0) ? ws.alt_vals : vals;

  if (nscan > 0)
    hipLaunchKernelGGL(k_scan_reduce, dim3(nscan), dim3(SCAN_BLOCK), 0, stream, counts, nrec, ws.block_sums);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(SCAN_BLOCK), 0, stream, ws.block_sums, nscan, capacity, num_pairs,
                     overflow, ws.live);
  if (nscan > 0)
    hipLaunchKernelGGL(k_emit, dim3(nscan), dim3(SCAN_BLOCK), 0, stream, vt, n, L.bin, counts, ws.block_sums,
                       overflow, k_a, v_a);
  SPLAT_LAUNCH_CHECK();
  for (int p = 0; p < passes; p++) {
    int shift = 8 * p;
    hipLaunchKernelGGL(k_radix_hist, dim3(nsort), dim3(SORT_BLOCK), 0, stream, k_a, ws.live, overflow, shift, nsort,
                       ws.hist);
    hipLaunchKernelGGL(k_radix_scan, dim3(RADIX), dim3(SCAN_BLOCK), 0, stream, ws.hist, nsort, ws.digit_total, ws.live,
                       overflow);
    hipLaunchKernelGGL(k_radix_scatter, dim3(nsort), dim3(SORT_BLOCK), 0, stream, k_a, v_a, k_b, v_b, ws.hist,
                       ws.digit_total, ws.live, overflow, shift, nsort);
    SPLAT_LAUNCH_CHECK();
    uint64_t *tk = k_a; k_a = k_b; k_b = tk;
    uint32_t *tv = v_a; v_a = v_b; v_b = tv;
  }
  long long nr = 2ll * vt.total_tiles;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, stream, ranges, nr, 0u);
  hipLaunchKernelGGL(k_ranges, dim3((unsigned)((capacity + 255) / 256)), dim3(256), 0, stream, keys, ws.live,
                     overflow, ranges);
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}
