// Binning to 16x16 tiles and the per-tile depth sort.
//
// Pulsar appendix B.1.1 sorts spheres by their earliest possible intersection
// depth so that drawing can stop early; B.1.2 works on 16x16 pixel blocks.
// The output is every (tile, record) overlap as a 64-bit key
//   (global tile << 32) | fp32 bits of the depth
// (depths are positive, so their bits order like the values) with the record
// index as value, ordered by (tile, depth bits, record index).
//
// The sort is most-significant-digit first: the tile is a counting-sort digit
// taken in one pass, then every tile's segment is sorted on its own by the
// 64-bit word (depth bits << 32) | record index. That word is unique per pair,
// so the order inside a tile before the segment sort does not matter and the
// bucketing can use atomic cursors.
//
// Pipeline (one stream, no host synchronisation):
//   k_thist                       each workgroup counts the tiles of a chunk of
//                                 one view's records in LDS and stores the counts
//                                 as one row of the view's [chunk][tile] matrix
//                                 (rows in XCD-major chunk order)
//   k_col_scan                    per tile (column): for every row the
//                                 exclusive prefix over earlier rows, and the
//                                 tile's pair total (16 waves per 64 columns)
//   k_tile_scan1                  exclusive scan over tiles (one workgroup):
//                                 tile ranges, pair total, overflow, tile starts
//                                 (one-view calls: inside k_tscatter instead)
//   k_tscatter                    each pair's word into its tile's segment, at
//                                 tile start + chunk prefix + a rank from an LDS
//                                 atomic
//   k_seg_sort                    segments up to SEG_WAVE pairs: one wave each,
//                                 a bitonic network in registers (lane shuffles
//                                 for the low merge levels, layouts moved through
//                                 LDS for the top two); up to SEG_MED pairs: one
//                                 wave each, merge rounds in its LDS region; then
//                                 longer segments from a work queue, one
//                                 workgroup each: merge sort in LDS up to NV
//                                 pairs, an MSD split into LDS-sized buckets
//                                 beyond
// No global atomics on the counting path: device-wide atomics on a few thousand
// tile counters serialise. Views with more tiles than LDS_TILES take a fallback
// (k_tile_count, k_bucket) with global atomic counters and cursors; more than
// TILE_SCAN1_MAX tiles take a three-kernel scan (k_scan_reduce, k_scan_top,
// k_tile_ranges).
#include "splat_internal.h"

namespace {

constexpr int SCAN_BLOCK = 256;
constexpr int TH_THREADS = 1024;    // workgroup of the counting passes
constexpr int TH_RPT = 4;           // records per thread in the counting passes
constexpr int TH_CHUNK = TH_THREADS * TH_RPT;
constexpr int SEG_WAVE = 512;       // segments up to this length: one wave sorts them
constexpr int SEG_MED = 1024;       // up to this length: one wave merge-sorts them in LDS
constexpr int TILE_SCAN1_MAX = 1 << 16;   // tiles scanned by a single workgroup
constexpr int LDS_TILES = 16384;    // tiles of one view held as LDS counters (64 KiB)
constexpr int LT = 512;             // threads of the long-segment sort
constexpr int LE = 16;              // words per thread in the long-segment sort
constexpr int NV = LT * LE;         // words one workgroup sorts in LDS (64 KiB)
constexpr int NV_PHYS = NV + NV / LE;   // one pad word after every LE words
constexpr int MAXLVL = 8;           // MSD split levels (8 bits of the word range each)
constexpr int SORT_GRID = 512;      // workgroups of the segment sort (two per CU)

// Block-wide exclusive scan of one value per thread (NT threads); returns the
// exclusive prefix and writes the block total to *total.
template <typename T, int NT = SCAN_BLOCK>
__device__ T block_exclusive_scan(T x, T *total) {
  __shared__ T s_w[NT / WAVE];
  unsigned lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  T inc = x;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    T y = __shfl_up(inc, d, WAVE);
    if (lane >= (unsigned)d) inc += y;
  }
  if (lane == WAVE - 1) s_w[w] = inc;
  __syncthreads();
  T wbase = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NT / WAVE; k++) {
    T t = s_w[k];
    if ((unsigned)k < w) wbase += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wbase + inc - x;
}

__global__ void k_fill_u32(uint32_t *p, long long n, uint32_t v) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---- pairs per tile ----------------------------------------------------------

// Visit the global tile ids of one record's rectangle (tile columns wrap on
// spherical views), row by row.
template <typename F>
__device__ __forceinline__ void for_each_tile(const ViewDev &cv, const BinRec &b, F f) {
#pragma unroll 1
  for (int ty = b.ty0; ty <= b.ty1; ty++) {
    int tx = b.tx0;
#pragma unroll 1
    for (int a = 0; a < b.ntx; a++) {
      f((uint32_t)(cv.tile_off + ty * cv.TW + tx));
      if (++tx == cv.TW) tx = 0;
    }
  }
}

__global__ __launch_bounds__(256) void k_tile_count(ViewTable vt, int n, BinArrays bin, const uint32_t *counts,
                                                     uint32_t *tile_cnt) {
  const long long k = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (long long)vt.n * n || counts[k] == 0) return;
  const ViewDev &cv = vt.v[(int)(k / n)];
  for_each_tile(cv, bin_rect(bin, k), [&](uint32_t gt) { atomicAdd(&tile_cnt[gt], 1u); });
}

// ---- exclusive scan over tiles -------------------------------------------------

// Block totals in 64 bits (a total of 2^32 or more can only mean overflow).
__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_reduce(const uint32_t *cnt, long long m,
                                                             unsigned long long *block_sums) {
  const long long k = (long long)blockIdx.x * SCAN_BLOCK + threadIdx.x;
  unsigned long long tot;
  block_exclusive_scan<unsigned long long>(k < m ? cnt[k] : 0u, &tot);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = tot;
}

// Single workgroup: exclusive scan of the block sums in place; pair total,
// overflow flag and live pair count.
// Each thread owns TOP_ITEMS consecutive sums per round.
constexpr int TOP_ITEMS = 16;
__global__ __launch_bounds__(SCAN_BLOCK) void k_scan_top(unsigned long long *block_sums, int nblocks,
                                                          long long capacity, int64_t *num_pairs, int32_t *overflow,
                                                          uint32_t *live) {
  unsigned long long carry = 0;
  for (int base = 0; base < nblocks; base += SCAN_BLOCK * TOP_ITEMS) {
    const int k0 = base + (int)threadIdx.x * TOP_ITEMS;
    unsigned long long x[TOP_ITEMS];
    unsigned long long s = 0;
#pragma unroll
    for (int r = 0; r < TOP_ITEMS; r++) {
      x[r] = k0 + r < nblocks ? block_sums[k0 + r] : 0ull;
      s += x[r];
    }
    unsigned long long tot;
    unsigned long long run = carry + block_exclusive_scan<unsigned long long>(s, &tot);
#pragma unroll
    for (int r = 0; r < TOP_ITEMS; r++) {
      if (k0 + r < nblocks) block_sums[k0 + r] = run;
      run += x[r];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) {
    *num_pairs = (int64_t)carry;
    const int of = carry > (unsigned long long)capacity ? 1 : 0;
    *overflow = of;
    live[0] = of ? 0u : (uint32_t)carry;
    live[1] = live[2] = live[3] = 0u;          // long-segment lists, filled by k_tile_ranges
  }
}

// Append tile t to a work list when p holds: one global atomic per wave.
__device__ __forceinline__ void list_append(uint32_t *list, uint32_t *count, bool p, uint32_t t) {
  const uint64_t m = ballot64(p);
  if (m == 0) return;
  const unsigned lane = lane_id();
  const int leader = __builtin_ffsll((long long)m) - 1;
  uint32_t base = 0;
  if ((int)lane == leader) base = atomicAdd(count, (uint32_t)__popcll(m));
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  if (p) list[base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull))] = t;
}

// Per tile: [start, end) (0, 0 when empty) and the bucket cursor (in place of the count).
// Without overflow every prefix is below the capacity (< 2^32).
// Tiles with more than SEG_MED pairs also go on the work lists of the
// long-segment sort (unordered here): list[0..) those above NV, list[m..) the rest.
__global__ __launch_bounds__(SCAN_BLOCK) void k_tile_ranges(uint32_t *cnt_cursor, long long m,
                                                             const unsigned long long *block_sums,
                                                             const int32_t *overflow, uint32_t *ranges,
                                                             uint32_t *live, uint32_t *list) {
  if (*overflow) return;
  const long long t = (long long)blockIdx.x * SCAN_BLOCK + threadIdx.x;
  const uint32_t c = t < m ? cnt_cursor[t] : 0u;
  uint32_t tot;
  const uint32_t start = (uint32_t)block_sums[blockIdx.x] + block_exclusive_scan<uint32_t>(c, &tot);
  if (t < m) {
    cnt_cursor[t] = start;
    ranges[2 * t] = c ? start : 0u;
    ranges[2 * t + 1] = c ? start + c : 0u;
  }
  list_append(list, &live[1], c > (uint32_t)NV, (uint32_t)t);
  list_append(list + m, &live[2], c > (uint32_t)SEG_MED && c <= (uint32_t)NV, (uint32_t)t);
}

// Single workgroup, up to TILE_SCAN1_MAX tiles: pair total, overflow flag and
// live count first, then, without overflow, the exclusive scan that writes the
// tile ranges and turns the counts into tile starts. Every thread owns
// TS_ITEMS consecutive tiles per round, so one wave's loads and stores cover a
// contiguous 1-2 KiB span (with 16 tiles per thread each wave instruction
// touched 64 cache lines, and one CU issues them all); up to
// TS_THREADS * TS_ITEMS tiles in all keep their counts in registers between the
// two phases. The same scan (three
// fields packed in one 64-bit value) lists the tiles for the long-segment sort:
// list[0..) those with more than NV pairs in tile order, list[m..) those with
// SEG_MED < pairs <= NV; live[1], live[2] count them, live[3] = 0 is the queue
// head.
constexpr int TS_THREADS = 1024;
constexpr int TS_ITEMS = 4;

__device__ __forceinline__ void load_counts(const uint32_t *cnt, int m, int t0, uint32_t (&x)[TS_ITEMS]) {
#pragma unroll
  for (int r = 0; r < TS_ITEMS; r++) x[r] = t0 + r < m ? cnt[t0 + r] : 0u;
}

__global__ __launch_bounds__(TS_THREADS) void k_tile_scan1(uint32_t *cnt_start, int m, long long capacity,
                                                            int64_t *num_pairs, int32_t *overflow, uint32_t *live,
                                                            uint32_t *ranges, uint32_t *list) {
  __shared__ int s_of;
  constexpr int ROUND = TS_THREADS * TS_ITEMS;
  uint32_t x[TS_ITEMS];
  unsigned long long part = 0;
  for (int base = 0; base < m; base += ROUND) {
    load_counts(cnt_start, m, base + (int)threadIdx.x * TS_ITEMS, x);
#pragma unroll
    for (int r = 0; r < TS_ITEMS; r++) part += x[r];
  }
  unsigned long long total;
  block_exclusive_scan<unsigned long long, TS_THREADS>(part, &total);
  if (threadIdx.x == 0) {
    const int of = total > (unsigned long long)capacity ? 1 : 0;
    *num_pairs = (int64_t)total;
    *overflow = of;
    live[0] = of ? 0u : (uint32_t)total;
    s_of = of;
  }
  __syncthreads();
  if (s_of) return;
  // below the capacity (< 2^32) from here on; the list counts of one round are
  // at most ROUND < 2^16, so the packed fields never carry into each other
  uint32_t carry = 0, carry_h = 0, carry_m = 0;
  for (int base = 0; base < m; base += ROUND) {
    const int t0 = base + (int)threadIdx.x * TS_ITEMS;
    if (m > ROUND) load_counts(cnt_start, m, t0, x);   // one round: still in registers
    uint32_t sum = 0, nh = 0, nm = 0;
#pragma unroll
    for (int r = 0; r < TS_ITEMS; r++) {
      sum += x[r];
      nh += x[r] > (uint32_t)NV ? 1u : 0u;
      nm += ((x[r] > (uint32_t)SEG_MED) & (x[r] <= (uint32_t)NV)) ? 1u : 0u;
    }
    const unsigned long long packed =
        (unsigned long long)sum | ((unsigned long long)nh << 32) | ((unsigned long long)nm << 48);
    unsigned long long tot;
    const unsigned long long pre = block_exclusive_scan<unsigned long long, TS_THREADS>(packed, &tot);
    uint32_t run = carry + (uint32_t)pre;
    uint32_t ph = carry_h + (uint32_t)((pre >> 32) & 0xffffu), pm = carry_m + (uint32_t)(pre >> 48);
#pragma unroll
    for (int r = 0; r < TS_ITEMS; r++) {
      if (t0 + r < m) {
        cnt_start[t0 + r] = run;
        ranges[2 * (t0 + r)] = x[r] ? run : 0u;
        ranges[2 * (t0 + r) + 1] = x[r] ? run + x[r] : 0u;
        if (x[r] > (uint32_t)NV)
          list[ph++] = (uint32_t)(t0 + r);
        else if (x[r] > (uint32_t)SEG_MED)
          list[m + pm++] = (uint32_t)(t0 + r);
      }
      run += x[r];
    }
    carry += (uint32_t)tot;
    carry_h += (uint32_t)((tot >> 32) & 0xffffu);
    carry_m += (uint32_t)(tot >> 48);
  }
  if (threadIdx.x == 0) {
    live[1] = carry_h;
    live[2] = carry_m;
    live[3] = 0u;
  }
}

// ---- bucketing -------------------------------------------------------------------

__global__ __launch_bounds__(256) void k_bucket(ViewTable vt, int n, BinArrays bin, const uint32_t *counts,
                                                 const int32_t *overflow, uint32_t *cursor, uint64_t *words) {
  if (*overflow) return;
  const long long k = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= (long long)vt.n * n || counts[k] == 0) return;
  const ViewDev &cv = vt.v[(int)(k / n)];
  const BinRec b = bin_full(bin, k);
  const uint64_t w = ((uint64_t)b.key << 32) | (uint64_t)(uint32_t)k;
  for_each_tile(cv, b, [&](uint32_t gt) {
    const uint32_t pos = atomicAdd(&cursor[gt], 1u);
    words[pos] = w;
  });
}

// ---- counting in LDS -------------------------------------------------------------

// Matrix of per-chunk tile counts: view v holds nchunk rows of T_v counters at off[v].
struct MatTable {
  long long off[SPLAT_MAX_VIEWS];
};

__device__ __forceinline__ long long mat_index(const MatTable &mt, const ViewDev &cv, int v, int row, int t) {
  return mt.off[v] + (long long)row * (cv.TW * cv.TH) + t;
}

// Matrix row of a chunk: the rows hold the chunks in XCD-major order, chunks
// c = 0, 8, 16, ... first, then 1, 9, 17, ..., and so on. Workgroups go to the
// eight XCDs round-robin, so the k_tscatter workgroups of one residue class
// share an XCD (and its L2); with the prefix over rows in this order each XCD
// fills one contiguous run of every tile's segment. In plain chunk order
// neighbouring words of a segment came from different XCDs, each L2 wrote the
// line back partially and every 8-byte word cost a 32-byte sector. Any order is
// correct: the segment is sorted afterwards.
__device__ __forceinline__ int chunk_row(int chunk, int nchunk) {
  const int a = nchunk >> 3, b = nchunk & 7, g = chunk & 7;   // residues below b hold a + 1 chunks
  return g * a + min(g, b) + (chunk >> 3);
}

// Records of one chunk, loaded up front (every thread TH_RPT of them, coalesced).
// A record's pair count is its rectangle's tile count, ntx (ty1 - ty0 + 1), the
// value splat_project also stores in pair_counts (culled records are all zero):
// one load per record instead of the count and then the record.
struct ChunkRecs {
  uint32_t cnt[TH_RPT];
  BinRec b[TH_RPT];
};

template <bool KEYS>
__device__ __forceinline__ void load_chunk(const BinArrays &bin, long long rec0, int nvalid, ChunkRecs &cr) {
#pragma unroll
  for (int r = 0; r < TH_RPT; r++) {
    const int j = r * TH_THREADS + (int)threadIdx.x;
    if (j < nvalid) {
      cr.b[r] = KEYS ? bin_full(bin, rec0 + j) : bin_rect(bin, rec0 + j);
    } else {
      cr.b[r].key = 0u; cr.b[r].tx0 = 0; cr.b[r].ntx = 0; cr.b[r].ty0 = 0; cr.b[r].ty1 = 0;
    }
  }
#pragma unroll
  for (int r = 0; r < TH_RPT; r++)
    cr.cnt[r] = (uint32_t)cr.b[r].ntx * (uint32_t)((int)cr.b[r].ty1 - (int)cr.b[r].ty0 + 1);
}

// View-local tile ids of one record's rectangle.
template <typename F>
__device__ __forceinline__ void for_each_local_tile(const ViewDev &cv, const BinRec &b, F f) {
#pragma unroll 1
  for (int ty = b.ty0; ty <= b.ty1; ty++) {
    int tx = b.tx0;
#pragma unroll 1
    for (int a = 0; a < b.ntx; a++) {
      f((uint32_t)(ty * cv.TW + tx));
      if (++tx == cv.TW) tx = 0;
    }
  }
}

// Pairs of one chunk. A record with at most LIGHT tiles is walked by the thread
// that loaded it; the others are staged in LDS (HB per batch) and their pairs
// are cut into equal contiguous slices, one per thread, so that a record that
// covers thousands of tiles does not hold up its wave. f(local tile, record
// slot in the chunk, depth key) is called once per pair.
constexpr uint32_t LIGHT = 16;
constexpr int HB = 512;

struct HeavyLds {
  uint32_t pre[HB + 1];      // first pair of each staged record (chunk pair stream); [nb] = end
  uint32_t geo0[HB];         // tx0 | ntx << 16
  uint32_t geo1[HB];         // ty0 | record slot << 16
  uint32_t key[HB];
  uint64_t wsum[TH_THREADS / WAVE];
};

template <typename F>
__device__ __forceinline__ void chunk_pairs(const ViewDev &cv, const ChunkRecs &cr, HeavyLds &hl, F f) {
  const int tid = (int)threadIdx.x;
  const unsigned lane = (unsigned)tid & (WAVE - 1), w = (unsigned)tid / WAVE;
  uint32_t nh = 0, np = 0;
#pragma unroll      // constant indices keep the record arrays in registers
  for (int r = 0; r < TH_RPT; r++) {
    const uint32_t c = cr.cnt[r];
    if (c > LIGHT) {
      nh++;
      np += c;
    } else if (c) {
      for_each_local_tile(cv, cr.b[r], [&](uint32_t lt) { f(lt, (uint32_t)(r * TH_THREADS + tid), cr.b[r].key); });
    }
  }
  // exclusive scan of (pairs | records << 40) over the workgroup
  const uint64_t x = (uint64_t)np | ((uint64_t)nh << 40);
  uint64_t inc = x;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const uint64_t y = __shfl_up(inc, d, WAVE);
    if (lane >= (unsigned)d) inc += y;
  }
  if (lane == WAVE - 1) hl.wsum[w] = inc;
  __syncthreads();
  uint64_t pre = inc - x, tot = 0;
#pragma unroll
  for (int q = 0; q < TH_THREADS / WAVE; q++) {
    const uint64_t t = hl.wsum[q];
    pre += (unsigned)q < w ? t : 0ull;
    tot += t;
  }
  const uint32_t NP = (uint32_t)(tot & ((1ull << 40) - 1)), NH = (uint32_t)(tot >> 40);
  const uint32_t pbase = (uint32_t)(pre & ((1ull << 40) - 1)), hbase = (uint32_t)(pre >> 40);
  for (uint32_t b0 = 0; b0 < NH; b0 += HB) {
    __syncthreads();                                 // readers of the previous batch are done
    uint32_t e = hbase, q = pbase;
#pragma unroll
    for (int r = 0; r < TH_RPT; r++) {
      if (cr.cnt[r] > LIGHT) {
        if (e >= b0 && e < b0 + HB) {
          const uint32_t i = e - b0;
          hl.pre[i] = q;
          hl.geo0[i] = (uint32_t)cr.b[r].tx0 | ((uint32_t)cr.b[r].ntx << 16);
          hl.geo1[i] = (uint32_t)cr.b[r].ty0 | ((uint32_t)(r * TH_THREADS + tid) << 16);
          hl.key[i] = cr.b[r].key;
        }
        if (e == b0 + HB) hl.pre[HB] = q;
        e++;
        q += cr.cnt[r];
      }
    }
    const int nb = (int)min((uint32_t)HB, NH - b0);
    if (b0 + HB >= NH && tid == 0) hl.pre[nb] = NP;
    __syncthreads();
    const uint32_t q_lo = hl.pre[0], q_hi = hl.pre[nb];
    const uint32_t per = (q_hi - q_lo + TH_THREADS - 1) / TH_THREADS;
    const uint32_t q0 = q_lo + (uint32_t)tid * per, q1 = min(q0 + per, q_hi);
    if (q0 >= q1) continue;
    int lo = 0, hi = nb - 1;                          // last staged record starting at or before q0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (hl.pre[mid] <= q0)
        lo = mid;
      else
        hi = mid - 1;
    }
    int i = lo;
    uint32_t g0 = hl.geo0[i], g1 = hl.geo1[i], key = hl.key[i];
    uint32_t rem = hl.pre[i + 1] - q0;               // pairs left in record i
    uint32_t ntx = g0 >> 16, k = q0 - hl.pre[i];
    uint32_t row = k / ntx, col = k - row * ntx;
    int tx = (int)(g0 & 0xffffu) + (int)col;
    if (tx >= cv.TW) tx -= cv.TW;
    int ty = (int)(g1 & 0xffffu) + (int)row;
    for (uint32_t qq = q0; qq < q1; qq++) {
      f((uint32_t)(ty * cv.TW + tx), g1 >> 16, key);
      if (--rem == 0) {
        i = min(i + 1, nb - 1);
        g0 = hl.geo0[i];
        g1 = hl.geo1[i];
        key = hl.key[i];
        rem = hl.pre[i + 1] - hl.pre[i];
        ntx = g0 >> 16;
        col = 0;
        tx = (int)(g0 & 0xffffu);
        ty = (int)(g1 & 0xffffu);
      } else {
        col++;
        if (++tx == cv.TW) tx = 0;
        if (col == ntx) {
          col = 0;
          tx = (int)(g0 & 0xffffu);
          ty++;
        }
      }
    }
  }
}

// grid: n_views * nchunk workgroups of TH_THREADS; dynamic LDS: 4 * max tiles per view.
__global__ __launch_bounds__(TH_THREADS) void k_thist(ViewTable vt, MatTable mt, int n, int nchunk, BinArrays bin,
                                                uint32_t *M) {
  extern __shared__ uint32_t s_cnt[];
  __shared__ HeavyLds hl;
  const int v = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const ViewDev &cv = vt.v[v];
  const int T = cv.TW * cv.TH;
  ChunkRecs cr;
  const int nvalid = min(TH_CHUNK, n - chunk * TH_CHUNK);
  load_chunk<false>(bin, (long long)v * n + (long long)chunk * TH_CHUNK, nvalid, cr);   // the keys are not needed
  for (int t = threadIdx.x; t < T; t += TH_THREADS) s_cnt[t] = 0;
  __syncthreads();
  chunk_pairs(cv, cr, hl, [&](uint32_t lt, uint32_t, uint32_t) { atomicAdd(&s_cnt[lt], 1u); });
  __syncthreads();
  uint32_t *row = M + mat_index(mt, cv, v, chunk_row(chunk, nchunk), 0);
  for (int t = threadIdx.x; t < T; t += TH_THREADS) row[t] = s_cnt[t];
}

// Matrix entries become the exclusive prefix over earlier rows of the same
// tile, and tile_cnt gets each tile's pair count. One workgroup per 64 tiles:
// lane l of every wave owns tile 64 b + l, and the 16 waves split the rows into
// consecutive ranges; each wave sums its range, the waves' sums are scanned in
// LDS, then each wave rewrites its range as running prefixes.
constexpr int CS_WAVES = 16;
constexpr int CS_HOLD = 16;      // matrix entries a lane keeps in registers (nchunk <= 256)

__global__ __launch_bounds__(CS_WAVES * 64) void k_col_scan(ViewTable vt, MatTable mt, int nchunk, uint32_t *M,
                                                            uint32_t *tile_cnt) {
  __shared__ uint32_t s_part[CS_WAVES][64];
  const int w = (int)(threadIdx.x >> 6), l = (int)(threadIdx.x & 63u);
  const int gt = (int)blockIdx.x * 64 + l;
  const bool ok = gt < vt.total_tiles;
  const int q = (nchunk + CS_WAVES - 1) / CS_WAVES;
  const int c0 = w * q, c1 = min(c0 + q, nchunk);
  long long base = 0, stride = 0;
  if (ok) {
    const int v = view_of_tile(vt, gt);
    const ViewDev &cv = vt.v[v];
    base = mat_index(mt, cv, v, 0, gt - cv.tile_off);
    stride = (long long)cv.TW * cv.TH;
  }
  // up to CS_HOLD entries per lane stay in registers between the sum and the
  // rewrite (one read of the matrix); longer ranges are read twice
  uint32_t s = 0;
  uint32_t xs[CS_HOLD];
  const bool hold = q <= CS_HOLD;
  if (ok) {
    if (hold) {
#pragma unroll
      for (int j = 0; j < CS_HOLD; j++) {
        xs[j] = c0 + j < c1 ? M[base + (c0 + j) * stride] : 0u;
        s += xs[j];
      }
    } else {
#pragma unroll 8
      for (int c = c0; c < c1; c++) s += M[base + c * stride];
    }
  }
  s_part[w][l] = s;
  __syncthreads();
  uint32_t run = 0;
  for (int w2 = 0; w2 < w; w2++) run += s_part[w2][l];
  if (ok) {
    if (hold) {
#pragma unroll
      for (int j = 0; j < CS_HOLD; j++) {
        if (c0 + j < c1) M[base + (c0 + j) * stride] = run;
        run += xs[j];
      }
    } else {
#pragma unroll 8
      for (int c = c0; c < c1; c++) {
        const long long i = base + c * stride;
        const uint32_t x = M[i];
        M[i] = run;
        run += x;
      }
    }
    if (w == CS_WAVES - 1) tile_cnt[gt] = run;
  }
}

// Where the tile scan writes its results (see k_tile_scan1).
struct ScanOut {
  long long capacity;
  int64_t *num_pairs;
  int32_t *overflow;
  uint32_t *live;
  uint32_t *ranges;
  uint32_t *list;
};

constexpr int FS_MAX = 8;                       // tiles per thread in the fused tile scan (T <= 8192)

// The tile scan of k_tile_scan1 inside every scatter workgroup of a one-view
// call with T <= FS_MAX * TH_THREADS tiles (a one-workgroup kernel costs ~6 us
// of launch and latency; the counts come from L2). Every workgroup scans all T counts; s_base[t]
// gets tile start + this chunk's row entry; workgroup 0 writes the pair total,
// the overflow flag and the list counters, and workgroup w the tile ranges and
// long-segment list entries of tiles [w T / nw, (w + 1) T / nw). Every
// workgroup reaches the same overflow decision; returns false on overflow.
__device__ bool fused_tile_scan(const uint32_t *cnt, int T, const uint32_t *row, uint32_t *s_base, const ScanOut &so,
                                int w, int nw) {
  const int ipt = (T + TH_THREADS - 1) / TH_THREADS;
  const int t0 = (int)threadIdx.x * ipt;
  uint32_t x[FS_MAX];
  unsigned long long part = 0;
  uint32_t sum = 0, nh = 0, nm = 0;
#pragma unroll
  for (int r = 0; r < FS_MAX; r++) {
    x[r] = r < ipt && t0 + r < T ? cnt[t0 + r] : 0u;
    part += x[r];
    sum += x[r];
    nh += x[r] > (uint32_t)NV ? 1u : 0u;
    nm += ((x[r] > (uint32_t)SEG_MED) & (x[r] <= (uint32_t)NV)) ? 1u : 0u;
  }
  unsigned long long total;
  block_exclusive_scan<unsigned long long, TH_THREADS>(part, &total);
  const bool of = total > (unsigned long long)so.capacity;
  if (w == 0 && threadIdx.x == 0) {
    *so.num_pairs = (int64_t)total;
    *so.overflow = of ? 1 : 0;
    so.live[0] = of ? 0u : (uint32_t)total;
  }
  if (of) return false;
  // below the capacity (< 2^32) from here on, and the list counts are at most
  // T < 2^16: the packed fields never carry into each other
  const unsigned long long packed =
      (unsigned long long)sum | ((unsigned long long)nh << 32) | ((unsigned long long)nm << 48);
  unsigned long long tot;
  const unsigned long long pre = block_exclusive_scan<unsigned long long, TH_THREADS>(packed, &tot);
  uint32_t run = (uint32_t)pre, ph = (uint32_t)((pre >> 32) & 0xffffu), pm = (uint32_t)(pre >> 48);
  const int s0 = (int)((long long)w * T / nw), s1 = (int)((long long)(w + 1) * T / nw);
#pragma unroll
  for (int r = 0; r < FS_MAX; r++) {
    const int t = t0 + r;
    if (r < ipt && t < T) {
      s_base[t] = run + row[t];
      if (t >= s0 && t < s1) {
        so.ranges[2 * t] = x[r] ? run : 0u;
        so.ranges[2 * t + 1] = x[r] ? run + x[r] : 0u;
        if (x[r] > (uint32_t)NV)
          so.list[ph] = (uint32_t)t;
        else if (x[r] > (uint32_t)SEG_MED)
          so.list[T + pm] = (uint32_t)t;
      }
      ph += x[r] > (uint32_t)NV ? 1u : 0u;
      pm += ((x[r] > (uint32_t)SEG_MED) & (x[r] <= (uint32_t)NV)) ? 1u : 0u;
    }
    run += x[r];
  }
  if (w == 0 && threadIdx.x == 0) {
    so.live[1] = (uint32_t)((tot >> 32) & 0xffffu);
    so.live[2] = (uint32_t)(tot >> 48);
    so.live[3] = 0u;
  }
  return true;
}

// Same chunks as k_thist: words to tile start + chunk prefix + LDS rank.
// FUSED (one view): tile_start holds the tile counts and the tile scan runs
// here (fused_tile_scan); otherwise k_tile_scan1 has turned them into starts.
template <bool FUSED>
__global__ __launch_bounds__(TH_THREADS) void k_tscatter(ViewTable vt, MatTable mt, int n, int nchunk, BinArrays bin,
                                                   const uint32_t *M,
                                                   const uint32_t *tile_start, const int32_t *overflow,
                                                   uint64_t *words, ScanOut so) {
  extern __shared__ uint32_t s_base[];
  __shared__ HeavyLds hl;
  if constexpr (!FUSED) {
    if (*overflow) return;
  }
  const int v = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const ViewDev &cv = vt.v[v];
  const int T = cv.TW * cv.TH;
  const uint32_t *row = M + mat_index(mt, cv, v, chunk_row(chunk, nchunk), 0);
  // the chunk's records are requested first: their loads are in flight during
  // the tile scan
  ChunkRecs cr;
  const long long rec0 = (long long)v * n + (long long)chunk * TH_CHUNK;
  load_chunk<true>(bin, rec0, min(TH_CHUNK, n - chunk * TH_CHUNK), cr);
  if constexpr (FUSED) {
    if (!fused_tile_scan(tile_start, T, row, s_base, so, chunk, nchunk)) return;
  } else {
    for (int t = threadIdx.x; t < T; t += TH_THREADS) s_base[t] = tile_start[cv.tile_off + t] + row[t];
  }
  __syncthreads();
  chunk_pairs(cv, cr, hl, [&](uint32_t lt, uint32_t slot, uint32_t key) {
    words[atomicAdd(&s_base[lt], 1u)] = ((uint64_t)key << 32) | (uint64_t)(uint32_t)(rec0 + slot);
  });
}

// ---- segment sorts ---------------------------------------------------------------

__device__ __forceinline__ void write_pair(uint64_t *keys, uint32_t *vals, uint32_t pos, uint32_t tile, uint64_t w) {
  keys[pos] = ((uint64_t)tile << 32) | (w >> 32);
  vals[pos] = (uint32_t)w;
}

// Value of lane (lane ^ M) for a 32-bit value, M a power of two below 64 or
// one less than a power of two: DPP quad permutes for 1, 2 and 3, a half-row
// mirror for 7 (followed by a quad reversal for 4), a row mirror for 15, a row
// rotation by 8 for 8, swizzles for 16 and 31 and a lane permute through the
// LDS crossbar for 32 and 63.
template <int M>
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x, unsigned lane) {
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, false);
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, false);
  } else if constexpr (M == 3) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x1B, 0xf, 0xf, false);
  } else if constexpr (M == 4) {
    const int y = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xf, 0xf, false);
    return (uint32_t)__builtin_amdgcn_mov_dpp(y, 0x1B, 0xf, 0xf, false);
  } else if constexpr (M == 7) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xf, 0xf, false);
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);
  } else if constexpr (M == 15) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xf, 0xf, false);
  } else if constexpr (M == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);
  } else if constexpr (M == 31) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x7C1F);
  } else {
    static_assert(M == 32 || M == 63, "lane_xor32: unsupported lane mask");
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((lane ^ (unsigned)M) << 2), (int)x);
  }
}

template <int M>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v, unsigned lane) {
  const uint32_t lo = lane_xor32<M>((uint32_t)v, lane), hi = lane_xor32<M>((uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Pad word of the in-register sorts: above every sort word and, read as fp64,
// the largest finite number.
constexpr uint64_t SORT_PAD = 0x7FEFFFFFFFFFFFFFull;

// Ascending compare-exchange of two sort words inside one lane. A sort word's
// high half is the bit pattern of a non-negative, non-NaN fp32 depth (0 to
// 0x7F800000) and its top bit is clear, so read as fp64 every word, and the pad
// above, is a non-negative finite number, and fp64 order is the unsigned
// integer order (fp64 denormals are kept in these kernels, not flushed). One
// fp64 minimum and one maximum replace a 64-bit compare and four selects; both
// return one of their operands bit for bit.
__device__ __forceinline__ void ce_asc(uint64_t &x, uint64_t &y) {
  const double a = __longlong_as_double((long long)x), b = __longlong_as_double((long long)y);
  // written out: the compiler's fmin / fmax first quiet possible signalling
  // NaNs with an extra fp64 operation per operand, and no NaN ever reaches here
  double lo, hi;
  asm("v_min_f64 %0, %1, %2" : "=v"(lo) : "v"(a), "v"(b));
  asm("v_max_f64 %0, %1, %2" : "=v"(hi) : "v"(a), "v"(b));
  x = (uint64_t)__double_as_longlong(lo);
  y = (uint64_t)__double_as_longlong(hi);
}

// Compare-exchange of word a of this lane with the same position of the
// partner lane (value o): the lane keeps the smaller one when keep_min.
__device__ __forceinline__ uint64_t ce_lane(uint64_t mine, uint64_t o, bool keep_min) {
  return ((o < mine) == keep_min) ? o : mine;
}

// Bitonic sort of 512 words, lane l holding words 8 l .. 8 l + 7, in the form
// whose comparators all point the same way: merge level K opens with word x
// paired with x ^ (K - 1) (the upper half of each K-block mirrored onto the
// lower), then pairs x with x ^ J for J = K / 4 .. 1, the lower word of every
// pair keeping the smaller. Pairs more than eight words apart sit in different
// lanes: x ^ (K - 1) is word 7 - a of lane l ^ (K / 8 - 1), x ^ J word a of lane
// l ^ (J / 8), and the lower side is the lane with bit K / 16 (resp. J / 8)
// clear. Pairs closer than that sit in one lane and need no direction.
template <int K>
__device__ __forceinline__ void flip_stage(uint64_t (&e)[8], unsigned lane) {
  if constexpr (K <= 8) {
#pragma unroll
    for (int a = 0; a < 8; a++)
      if ((a & (K / 2)) == 0) ce_asc(e[a], e[a ^ (K - 1)]);
  } else {
    constexpr int M = K / 8 - 1;
    const bool keep_min = (lane & (unsigned)(K / 16)) == 0u;
    uint64_t o[8];
#pragma unroll
    for (int a = 0; a < 8; a++) o[a] = lane_xor64<M>(e[7 - a], lane);
#pragma unroll
    for (int a = 0; a < 8; a++) e[a] = ce_lane(e[a], o[a], keep_min);
  }
}

template <int J>
__device__ __forceinline__ void half_stage(uint64_t (&e)[8], unsigned lane) {
  if constexpr (J >= 8) {
    constexpr int M = J / 8;
    const bool keep_min = (lane & (unsigned)M) == 0u;
#pragma unroll
    for (int a = 0; a < 8; a++) e[a] = ce_lane(e[a], lane_xor64<M>(e[a], lane), keep_min);
  } else {
#pragma unroll
    for (int a = 0; a < 8; a++)
      if ((a & J) == 0) ce_asc(e[a], e[a | J]);
  }
  if constexpr (J > 1) half_stage<J / 2>(e, lane);
}

// From this merge level on, the wave sort moves its words between three
// layouts through the wave's LDS region instead of exchanging them between
// lanes, so that every compare-exchange pairs two registers of one lane:
//   A: word x = 8 l + a           (register index a = bits 0-2 of x)
//   B: word x = l + 64 a          (a = bits 6-8; also the global-memory layout)
//   C: word x = (l & 7) + 8 a + 64 (l >> 3)   (a = bits 3-5)
// A level's stages on bits 6-8 run in B, on bits 3-5 in C, on bits 0-2 in A.
// Its opening stage (x against x ^ (K - 1)) becomes a stage on the top bit
// alone, x against x ^ K / 2, once the upper half of every K-block is read in
// reverse order: the words then form a bitonic sequence per block, and the
// merge that follows keeps every comparator ascending.
constexpr int SORT_TR_LEVEL = 256;

// LDS slot (wslot) of the word that lane l, register a holds in a layout.
__device__ __forceinline__ int slot_a(unsigned l, int a) { return 9 * (int)l + a; }
__device__ __forceinline__ int slot_b(unsigned l, int a) { return (int)(l + (l >> 3)) + 72 * a; }
__device__ __forceinline__ int slot_c(unsigned l, int a) { return (int)((l & 7u) + 72u * (l >> 3)) + 9 * a; }

// Store the words from layout A.
__device__ __forceinline__ void lay_store_a(const uint64_t (&e)[8], unsigned lane, uint64_t *sw) {
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) sw[slot_a(lane, a)] = e[a];
  __builtin_amdgcn_wave_barrier();
}

// Read into layout B; with K > 0, the upper half of every K-block (K >= 128:
// bit K / 2 of x is a register bit here) in reverse order: word x ^ (K / 2 - 1).
template <int K>
__device__ __forceinline__ void lay_load_b(uint64_t (&e)[8], unsigned lane, const uint64_t *sw) {
#pragma unroll
  for (int a = 0; a < 8; a++) {
    if (K > 0 && ((64 * a) & (K / 2)) != 0)
      e[a] = sw[slot_b(lane ^ 63u, a ^ ((K / 2 - 1) >> 6))];
    else
      e[a] = sw[slot_b(lane, a)];
  }
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void lay_b_to_c(uint64_t (&e)[8], unsigned lane, uint64_t *sw) {
#pragma unroll
  for (int a = 0; a < 8; a++) sw[slot_b(lane, a)] = e[a];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) e[a] = sw[slot_c(lane, a)];
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void lay_c_to_a(uint64_t (&e)[8], unsigned lane, uint64_t *sw) {
#pragma unroll
  for (int a = 0; a < 8; a++) sw[slot_c(lane, a)] = e[a];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) e[a] = sw[slot_a(lane, a)];
  __builtin_amdgcn_wave_barrier();
}

// Stages on register bits R, R - 1, .. 0: the register with the bit clear
// keeps the smaller word.
template <int R>
__device__ __forceinline__ void reg_stages(uint64_t (&e)[8]) {
#pragma unroll
  for (int a = 0; a < 8; a++)
    if (((a >> R) & 1) == 0) ce_asc(e[a], e[a | (1 << R)]);
  if constexpr (R > 0) reg_stages<R - 1>(e);
}

template <int K>
__device__ __forceinline__ void bitonic512(uint64_t (&e)[8], unsigned lane, uint64_t *sw) {
  if constexpr (K >= SORT_TR_LEVEL) {
    static_assert(K >= 128, "layout B holds bits 6-8 only");
    constexpr int TOP = K == 128 ? 0 : K == 256 ? 1 : 2;   // register bit of x bit log2(K) - 1 in B
    lay_store_a(e, lane, sw);
    lay_load_b<K>(e, lane, sw);
    reg_stages<TOP>(e);
    lay_b_to_c(e, lane, sw);
    reg_stages<2>(e);
    lay_c_to_a(e, lane, sw);
    reg_stages<2>(e);
  } else {
    flip_stage<K>(e, lane);
    if constexpr (K >= 4) half_stage<K / 4>(e, lane);
  }
  if constexpr (K < 512) bitonic512<K * 2>(e, lane, sw);
}

// Segments of at most SEG_WAVE pairs: one wave per tile, padded to 512 words
// with the pad word (it sorts last), the whole network unrolled. The network
// wants lane l to hold words 8 l .. 8 l + 7; global memory is read and written
// with lane l on words l + 64 a instead (each wave access one contiguous run)
// and the wave transposes through its own 576 words of LDS, one pad word after
// every eight so that the blocked accesses (72-byte lane stride) spread over
// the banks. LDS operations of one wave complete in order, so no barrier is
// needed between a lane's write and another lane's read.
constexpr int WS_LDS = SEG_WAVE + SEG_WAVE / 8;

__device__ __forceinline__ int wslot(int x) { return x + (x >> 3); }

__device__ __forceinline__ void wave_sort_tile(const uint32_t *ranges, const uint64_t *words, uint64_t *keys,
                                               uint32_t *vals, int t, uint64_t *sw) {
  const uint32_t start = ranges[2 * t], len = ranges[2 * t + 1] - start;
  if (len == 0 || len > SEG_WAVE) return;
  const unsigned lane = lane_id();
  uint64_t e[8];
#pragma unroll
  for (int a = 0; a < 8; a++) {
    const uint32_t x = lane + 64u * a;
    e[a] = x < len ? words[start + x] : SORT_PAD;
  }
#pragma unroll
  for (int a = 0; a < 8; a++) sw[wslot((int)lane + 64 * a)] = e[a];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) e[a] = sw[wslot(8 * (int)lane + a)];
  bitonic512<2>(e, lane, sw);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) sw[wslot(8 * (int)lane + a)] = e[a];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int a = 0; a < 8; a++) {
    const uint32_t x = lane + 64u * a;
    const uint64_t w = sw[wslot((int)x)];
    if (x < len) write_pair(keys, vals, start + x, (uint32_t)t, w);
  }
  __builtin_amdgcn_wave_barrier();
}

// ---- long segments: merge sort in LDS, MSD split beyond NV -----------------------

// LDS slot of word x of the sort buffer: one pad word after every LE words, so
// that a thread's LE consecutive words start LE + 1 words after the previous
// thread's and the blocked reads and writes spread over the banks.
__device__ __forceinline__ int lslot(int x) { return x + x / LE; }

// Ascending sort of one thread's LE words: the bitonic network in the form
// with every comparator ascending (level k: a with a ^ (k - 1), then a with
// a ^ j for j = k / 4 .. 1), every index known at compile time.
__device__ __forceinline__ void sort_regs(uint64_t (&e)[LE]) {
#pragma unroll
  for (int k = 2; k <= LE; k <<= 1) {
#pragma unroll
    for (int a = 0; a < LE; a++)
      if ((a & (k >> 1)) == 0) ce_asc(e[a], e[a ^ (k - 1)]);
#pragma unroll
    for (int j = k >> 2; j > 0; j >>= 1) {
#pragma unroll
      for (int a = 0; a < LE; a++)
        if ((a & j) == 0) ce_asc(e[a], e[a | j]);
    }
  }
}

// One merge round: the LE outputs from position o of the merge of the two
// sorted runs of length R that contain o (the second run may be short or
// empty). The split of the outputs between the runs comes from a binary search
// along the cross diagonal (merge path); ties go to the first run, and the
// only equal words are the pad words, so every thread's split agrees with its
// neighbours'. An exhausted run reads as all-ones (above the pad).
template <int CAP = NV>
__device__ __forceinline__ void merge_round(const uint64_t *s, int R, int npad, int o, uint64_t (&e)[LE]) {
  const int a0 = o & ~(2 * R - 1), b0 = a0 + R;
  const int alen = min(R, npad - a0), blen = max(0, min(R, npad - b0));
  const int diag = o - a0;
  int lo = max(0, diag - blen), hi = min(diag, alen);
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[lslot(a0 + mid)] <= s[lslot(b0 + diag - 1 - mid)])
      lo = mid + 1;
    else
      hi = mid;
  }
  int ia = a0 + lo, ib = b0 + diag - lo;
  const int ea = a0 + alen, eb = b0 + blen;
  uint64_t a = s[lslot(min(ia, CAP - 1))], b = s[lslot(min(ib, CAP - 1))];
  a = ia < ea ? a : ~0ull;
  b = ib < eb ? b : ~0ull;
#pragma unroll
  for (int k = 0; k < LE; k++) {
    const bool ta = a <= b;
    e[k] = ta ? a : b;
    if (k == LE - 1) break;
    ia += ta ? 1 : 0;
    ib += ta ? 0 : 1;
    const int nx = ta ? ia : ib;
    const bool ok = nx < (ta ? ea : eb);
    uint64_t x = s[lslot(min(nx, CAP - 1))];
    x = ok ? x : ~0ull;
    a = ta ? x : a;
    b = ta ? b : x;
  }
}

// Sort len <= NV words of global memory in LDS by the whole workgroup and
// write the final (tile << 32 | depth bits, record) pairs. The words are padded
// to a multiple of LE with the pad word (it sorts last and is not written);
// every thread sorts its LE words in registers, then runs of LE, 2 LE, ... are
// merged pairwise until one run remains.
__device__ void lds_sort(const uint64_t *src, int len, uint64_t *kout, uint32_t *vout, uint32_t tile, uint64_t *s) {
  const int tid = (int)threadIdx.x;
  const int npad = (len + LE - 1) & ~(LE - 1);
  uint64_t e[LE];
#pragma unroll
  for (int r = 0; r < LE; r++) {
    const int i = r * LT + tid;
    e[r] = i < len ? src[i] : SORT_PAD;
  }
  __syncthreads();                                   // earlier readers of s are done
#pragma unroll
  for (int r = 0; r < LE; r++) {
    const int i = r * LT + tid;
    if (i < npad) s[lslot(i)] = e[r];
  }
  __syncthreads();
  const int o = tid * LE;
  const bool act = o < npad;
  if (act) {
#pragma unroll
    for (int k = 0; k < LE; k++) e[k] = s[tid * (LE + 1) + k];
    sort_regs(e);
  }
  for (int R = LE; R < npad; R <<= 1) {
    __syncthreads();
    if (act) {
#pragma unroll
      for (int k = 0; k < LE; k++) s[tid * (LE + 1) + k] = e[k];
    }
    __syncthreads();
    if (act) merge_round(s, R, npad, o, e);
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int k = 0; k < LE; k++) s[tid * (LE + 1) + k] = e[k];
  }
  __syncthreads();
  for (int i = tid; i < len; i += LT) {
    const uint64_t w = s[lslot(i)];
    kout[i] = ((uint64_t)tile << 32) | (w >> 32);
    vout[i] = (uint32_t)w;
  }
}

// Segments of SEG_WAVE < len <= SEG_MED words: one wave, LE words per lane, the
// register sort and merge rounds of lds_sort inside the wave's own LDS region
// (WS_REGION words), with no workgroup barrier: LDS operations of one wave
// complete in order. Eight such segments are sorted at once per workgroup,
// where the work queue would give each its own workgroup of LT threads.
constexpr int WS_REGION = SEG_MED + SEG_MED / LE;

__device__ __forceinline__ void wave_merge_sort_tile(const uint32_t *ranges, const uint64_t *words, uint64_t *keys,
                                                     uint32_t *vals, int t, uint64_t *sw) {
  const uint32_t start = ranges[2 * t];
  const int len = (int)(ranges[2 * t + 1] - start);
  const int lane = (int)lane_id();
  const int npad = (len + LE - 1) & ~(LE - 1);
  uint64_t e[LE];
#pragma unroll
  for (int r = 0; r < LE; r++) {
    const int i = r * WAVE + lane;
    e[r] = i < len ? words[start + i] : SORT_PAD;
  }
#pragma unroll
  for (int r = 0; r < LE; r++) {
    const int i = r * WAVE + lane;
    if (i < npad) sw[lslot(i)] = e[r];
  }
  __builtin_amdgcn_wave_barrier();
  const int o = lane * LE;
  const bool act = o < npad;
  if (act) {
#pragma unroll
    for (int k = 0; k < LE; k++) e[k] = sw[lane * (LE + 1) + k];
    sort_regs(e);
  }
  for (int R = LE; R < npad; R <<= 1) {
    __builtin_amdgcn_wave_barrier();
    if (act) {
#pragma unroll
      for (int k = 0; k < LE; k++) sw[lane * (LE + 1) + k] = e[k];
    }
    __builtin_amdgcn_wave_barrier();
    if (act) merge_round<SEG_MED>(sw, R, npad, o, e);
  }
  __builtin_amdgcn_wave_barrier();
  if (act) {
#pragma unroll
    for (int k = 0; k < LE; k++) sw[lane * (LE + 1) + k] = e[k];
  }
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < len; i += WAVE) write_pair(keys, vals, start + (uint32_t)i, (uint32_t)t, sw[lslot(i)]);
  __builtin_amdgcn_wave_barrier();
}

struct SplitLds {
  uint32_t off[MAXLVL][257];       // bucket starts of each open level (tile-relative), [256] = end
  uint32_t cur[256];               // histogram, then scatter cursors
  uint32_t wsum[4];
  unsigned long long mm[2];        // segment minimum and maximum
  int next[MAXLVL];                // first bucket still to visit on each open level
  int item;
};

// MSD split of src[0, len) into dst[0, len): bucket b holds the words whose
// offset from the minimum has b as its top 8 bits (of the offset range's bit
// length), so buckets are in value order and each spans less than 2^(bits-8).
// off[b] = base + start of bucket b, off[256] = base + len.
__device__ void msd_split(const uint64_t *src, uint64_t *dst, int len, uint32_t base, uint32_t *off, SplitLds &sl) {
  const int tid = (int)threadIdx.x;
  const unsigned lane = (unsigned)tid & (WAVE - 1);
  uint64_t mn = ~0ull, mx = 0ull;
  for (int i0 = 0; i0 < len; i0 += 4 * LT) {
    uint64_t x[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * LT + tid;
      x[r] = i < len ? src[i] : ~0ull;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * LT + tid;
      mn = x[r] < mn ? x[r] : mn;
      mx = ((i < len) & (x[r] > mx)) ? x[r] : mx;
    }
  }
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const uint64_t a = __shfl_xor(mn, d, WAVE), b = __shfl_xor(mx, d, WAVE);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  __syncthreads();                                   // earlier readers of sl are done
  if (tid == 0) {
    sl.mm[0] = ~0ull;
    sl.mm[1] = 0ull;
  }
  if (tid < 256) sl.cur[tid] = 0u;
  __syncthreads();
  if (lane == 0) {
    atomicMin(&sl.mm[0], (unsigned long long)mn);
    atomicMax(&sl.mm[1], (unsigned long long)mx);
  }
  __syncthreads();
  const uint64_t lo = sl.mm[0], range = sl.mm[1] - lo;
  const int bits = range ? 64 - __clzll((long long)range) : 0;
  const int sh = bits > 8 ? bits - 8 : 0;
  for (int i0 = 0; i0 < len; i0 += 4 * LT) {
    uint64_t x[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * LT + tid;
      x[r] = i < len ? src[i] : lo;
    }
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (i0 + r * LT + tid < len) atomicAdd(&sl.cur[(unsigned)((x[r] - lo) >> sh)], 1u);
  }
  __syncthreads();
  // exclusive scan of the 256 counts by threads 0..255
  const uint32_t c = tid < 256 ? sl.cur[tid] : 0u;
  uint32_t inc = c;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d, WAVE);
    if (lane >= (unsigned)d) inc += y;
  }
  if (tid < 256 && lane == WAVE - 1) sl.wsum[tid / WAVE] = inc;
  __syncthreads();
  if (tid < 256) {
    uint32_t pre = inc - c;
    for (int q = 0; q < tid / WAVE; q++) pre += sl.wsum[q];
    off[tid] = base + pre;
    sl.cur[tid] = pre;
  }
  if (tid == 0) off[256] = base + (uint32_t)len;
  __syncthreads();
  for (int i0 = 0; i0 < len; i0 += 4 * LT) {
    uint64_t x[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int i = i0 + r * LT + tid;
      x[r] = i < len ? src[i] : lo;
    }
#pragma unroll
    for (int r = 0; r < 4; r++)
      if (i0 + r * LT + tid < len) dst[atomicAdd(&sl.cur[(unsigned)((x[r] - lo) >> sh)], 1u)] = x[r];
  }
  __builtin_amdgcn_s_waitcnt(0);                     // the scattered words are written
  __syncthreads();                                   // before any thread reads them back
}

// Every segment sorted on its own. First each wave sorts the short segments
// (at most SEG_MED pairs) of its share of the tiles; then the workgroups take
// the longer segments one per workgroup from a work queue (the tiles above NV
// first). Up to NV pairs: lds_sort straight from the bucketed words. Beyond: MSD split into the key array (used as scratch), then every run
// of adjacent buckets that fits NV words is sorted as one segment; a bucket
// above NV is split again into the bucketed-word array, and so on, alternating.
// Words are unique, so the offset range loses 8 bits per level and a bucket on
// level MAXLVL - 1 holds at most one word: the split never goes deeper.
__global__ __launch_bounds__(LT) void k_seg_sort(const uint32_t *ranges, uint64_t *words, const int32_t *overflow,
                                                  uint64_t *keys, uint32_t *vals, uint32_t *live,
                                                  const uint32_t *list, int tiles) {
  __shared__ uint64_t s[NV_PHYS];
  __shared__ SplitLds sl;
  if (*overflow) return;
  {
    static_assert(WS_LDS <= WS_REGION && (LT / WAVE) * WS_REGION <= NV_PHYS,
                  "wave-sort LDS regions exceed the sort buffer");
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
    uint64_t *sw = s + wave * WS_REGION;
    for (int t = (int)blockIdx.x * (LT / WAVE) + wave; t < tiles; t += (int)gridDim.x * (LT / WAVE)) {
      const uint32_t len = ranges[2 * t + 1] - ranges[2 * t];
      if (len > (uint32_t)SEG_WAVE && len <= (uint32_t)SEG_MED)
        wave_merge_sort_tile(ranges, words, keys, vals, t, sw);
      else
        wave_sort_tile(ranges, words, keys, vals, t, sw);
    }
  }
  const int nh = (int)live[1], nall = nh + (int)live[2];
  if (nall == 0) return;
  const int tid = (int)threadIdx.x;
  for (;;) {
    __syncthreads();                                 // every thread has read sl.item
    if (tid == 0) sl.item = (int)atomicAdd(&live[3], 1u);
    __syncthreads();
    const int item = sl.item;
    if (item >= nall) break;
    const uint32_t t = item < nh ? list[item] : list[tiles + item - nh];
    const uint32_t start = ranges[2 * t];
    const int len = (int)(ranges[2 * t + 1] - start);
    uint64_t *W = words + start, *K = keys + start;
    uint32_t *V = vals + start;
    if (len <= NV) {
      lds_sort(W, len, K, V, t, s);
      continue;
    }
    msd_split(W, K, len, 0u, sl.off[0], sl);
    int L = 0, b = 0;
    for (;;) {
      if (b >= 256) {
        if (L == 0) break;
        L--;
        b = sl.next[L];
        continue;
      }
      const uint64_t *buf = (L & 1) ? W : K;         // level L buckets: K when L is even
      const uint32_t g0 = sl.off[L][b];
      const uint32_t blen = sl.off[L][b + 1] - g0;
      if (blen > (uint32_t)NV && L + 1 < MAXLVL) {
        __syncthreads();                             // every thread has read sl.next
        if (tid == 0) sl.next[L] = b + 1;
        msd_split(buf + g0, ((L & 1) ? K : W) + g0, (int)blen, g0, sl.off[L + 1], sl);
        L++;
        b = 0;
        continue;
      }
      int e = b + 1;
      while (e < 256 && sl.off[L][e + 1] - g0 <= (uint32_t)NV) e++;
      const int glen = (int)(sl.off[L][e] - g0);
      if (glen > 0 && glen <= NV) lds_sort(buf + g0, glen, K + g0, V + g0, t, s);
      b = e;
    }
  }
}

struct SortWs {
  uint64_t *words;      // [capacity] bucketed (depth << 32 | record) words
  uint32_t *cursor;     // [tiles] counts, then tile starts (and cursors in the fallback)
  unsigned long long *block_sums;  // [ceil(tiles / 256) + 1]
  uint32_t *live;       // [0] live pairs, [1] [2] long-segment list counts, [3] queue head
  uint32_t *list;       // [2 * tiles] long-segment work lists
  uint32_t *mat;        // per-chunk tile counts (LDS counting path)
  size_t bytes;
};

struct CountPlan {
  bool lds;             // every view's tiles fit the LDS counters
  int nchunk, max_tiles;
  long long mat_elems;
  MatTable mt;
};

CountPlan count_plan(const ViewTable &vt, int n) {
  CountPlan cp{};
  cp.nchunk = (n + TH_CHUNK - 1) / TH_CHUNK;
  cp.lds = n > 0;
  long long off = 0;
  for (int v = 0; v < vt.n; v++) {
    const int T = vt.v[v].TW * vt.v[v].TH;
    cp.max_tiles = T > cp.max_tiles ? T : cp.max_tiles;
    if (T > LDS_TILES) cp.lds = false;
    cp.mt.off[v] = off;
    off += (long long)cp.nchunk * T;
  }
  cp.mat_elems = cp.lds ? off : 0;
  return cp;
}

SortWs sort_ws_layout(void *base, const ViewTable &vt, int n, long long capacity) {
  SortWs w;
  char *p = (char *)base;
  const long long tiles = vt.total_tiles;
  const long long nscan = (tiles + SCAN_BLOCK - 1) / SCAN_BLOCK;
  const CountPlan cp = count_plan(vt, n);
  w.words = (uint64_t *)p;      p += proj_align(sizeof(uint64_t) * (size_t)(capacity > 0 ? capacity : 1));
  w.cursor = (uint32_t *)p;     p += proj_align(sizeof(uint32_t) * (size_t)tiles);
  w.block_sums = (unsigned long long *)p; p += proj_align(sizeof(unsigned long long) * (size_t)(nscan + 1));
  w.live = (uint32_t *)p;       p += proj_align(sizeof(uint32_t) * 4);
  w.list = (uint32_t *)p;       p += proj_align(sizeof(uint32_t) * 2 * (size_t)tiles);
  w.mat = (uint32_t *)p;        p += proj_align(sizeof(uint32_t) * (size_t)cp.mat_elems);
  w.bytes = (size_t)(p - (char *)base);
  return w;
}

}  // namespace

size_t sort_workspace_bytes(const ViewTable &vt, int n, long long capacity) {
  return sort_ws_layout(nullptr, vt, n, capacity).bytes;
}

int launch_bin_sort(const ViewTable &vt, int n, const void *proj, const uint32_t *counts, long long capacity,
                    uint64_t *keys, uint32_t *vals, uint32_t *ranges, int64_t *num_pairs, int32_t *overflow,
                    void *workspace, hipStream_t stream) {
  const long long nrec = (long long)vt.n * n;
  const long long tiles = vt.total_tiles;
  SortWs ws = sort_ws_layout(workspace, vt, n, capacity);
  const CountPlan cp = count_plan(vt, n);
  ProjLayout L = proj_layout(const_cast<void *>(proj), nrec);
  const unsigned rec_blocks = (unsigned)((nrec + 255) / 256);
  const int nscan = (int)((tiles + SCAN_BLOCK - 1) / SCAN_BLOCK);
  const unsigned tile_blocks = (unsigned)((tiles + 255) / 256);
  const size_t lds_bytes = sizeof(uint32_t) * (size_t)cp.max_tiles;

  if (cp.lds) {
    const unsigned grid = (unsigned)(vt.n * cp.nchunk);
    hipLaunchKernelGGL(k_thist, dim3(grid), dim3(TH_THREADS), lds_bytes, stream, vt, cp.mt, n, cp.nchunk, L.bin,
                       ws.mat);
    hipLaunchKernelGGL(k_col_scan, dim3((unsigned)((tiles + 63) / 64)), dim3(CS_WAVES * 64), 0, stream, vt, cp.mt,
                       cp.nchunk, ws.mat, ws.cursor);
  } else {
    hipLaunchKernelGGL(k_fill_u32, dim3(tile_blocks), dim3(256), 0, stream, ws.cursor, tiles, 0u);
    if (rec_blocks)
      hipLaunchKernelGGL(k_tile_count, dim3(rec_blocks), dim3(256), 0, stream, vt, n, L.bin, counts, ws.cursor);
  }
  // one view of at most FS_MAX * TH_THREADS tiles: the tile scan runs inside k_tscatter
  const bool fused = cp.lds && vt.n == 1 && tiles <= (long long)FS_MAX * TH_THREADS;
  const ScanOut so{capacity, num_pairs, overflow, ws.live, ranges, ws.list};
  if (fused) {
    // nothing here
  } else if (tiles <= TILE_SCAN1_MAX) {
    hipLaunchKernelGGL(k_tile_scan1, dim3(1), dim3(TS_THREADS), 0, stream, ws.cursor, (int)tiles, capacity, num_pairs,
                       overflow, ws.live, ranges, ws.list);
  } else {
    hipLaunchKernelGGL(k_scan_reduce, dim3(nscan), dim3(SCAN_BLOCK), 0, stream, ws.cursor, tiles, ws.block_sums);
    hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(SCAN_BLOCK), 0, stream, ws.block_sums, nscan, capacity, num_pairs,
                       overflow, ws.live);
    hipLaunchKernelGGL(k_tile_ranges, dim3(nscan), dim3(SCAN_BLOCK), 0, stream, ws.cursor, tiles, ws.block_sums,
                       overflow, ranges, ws.live, ws.list);
  }
  SPLAT_LAUNCH_CHECK();
  if (fused) {
    hipLaunchKernelGGL(k_tscatter<true>, dim3((unsigned)cp.nchunk), dim3(TH_THREADS), lds_bytes, stream, vt, cp.mt, n,
                       cp.nchunk, L.bin, ws.mat, ws.cursor, overflow, ws.words, so);
  } else if (cp.lds) {
    hipLaunchKernelGGL(k_tscatter<false>, dim3((unsigned)(vt.n * cp.nchunk)), dim3(TH_THREADS), lds_bytes, stream, vt,
                       cp.mt, n, cp.nchunk, L.bin, ws.mat, ws.cursor, overflow, ws.words, so);
  } else if (rec_blocks) {
    hipLaunchKernelGGL(k_bucket, dim3(rec_blocks), dim3(256), 0, stream, vt, n, L.bin, counts, overflow, ws.cursor,
                       ws.words);
  }
  hipLaunchKernelGGL(k_seg_sort, dim3(SORT_GRID), dim3(LT), 0, stream, ranges, ws.words, overflow, keys, vals, ws.live,
                     ws.list, (int)tiles);
  SPLAT_LAUNCH_CHECK();
  return SPLAT_OK;
}
