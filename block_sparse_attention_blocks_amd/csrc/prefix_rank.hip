// Historical KV ranking of S2O (Methodology 1, Historical KV Permutation): per KV head g and
// segment sigma >= 1, every key of the causal prefix [0, sigma*S) ordered by its dot product with a
// representative query of the segment (the mean of the segment's query rows over the G query heads
// of g), descending, ties by position.  Three steps:
//   seg_rep_*            fp64 representative queries (exact bf16 widening, fp64 sums)
//   prefix_score_kernel  fp64 scores r . k_j, rounded to fp32 and written as order-preserving keys
//   radix_*              stable least-significant-digit radix sort of every (g, sigma) list,
//                        8-bit digits, four passes
// Output layout: kv_rank[g][S*sigma*(sigma-1)/2 + r] = key of rank r for segment sigma.
// Also S2O's query permutation (query_guide_kernel + the segment sort of stage 1).
#include "estimate.h"

namespace pbsa {
namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int RK_THREADS = 256;
constexpr int RADIX_BITS = 8;
constexpr int DIGITS = 1 << RADIX_BITS;  // one bin per thread of a workgroup
constexpr int RADIX_PASSES = 32 / RADIX_BITS;
constexpr int NIB = 16;                  // a tile is reordered in LDS 4 bits at a time
static_assert(DIGITS == RK_THREADS, "one histogram bin per thread");

// List and tile geometry of the ranking.  The radix tile is the largest power of two <= 2048 that
// divides S, so every list (sigma*S keys) is a whole number of tiles.
struct PrefixGeom {
  int nseg;                // segments, ceil(N / S)
  int S;
  int64_t L;               // entries per KV head: S * nseg * (nseg - 1) / 2
  int tile;                // radix tile (elements)
  int tps;                 // tiles per S keys
  int64_t tiles_per_head;  // tps * nseg * (nseg - 1) / 2
};

PrefixGeom prefix_geom(const Geometry& g) {
  PrefixGeom p;
  p.S = g.S;
  p.nseg = (g.N + g.S - 1) / g.S;
  p.L = (int64_t)g.S * p.nseg * (p.nseg - 1) / 2;
  int t = 2048;
  while (g.S % t) t >>= 1;
  p.tile = t;
  p.tps = g.S / t;
  p.tiles_per_head = (int64_t)p.tps * p.nseg * (p.nseg - 1) / 2;
  return p;
}

constexpr int REP_ROWS = 256;  // query rows summed by one workgroup of seg_rep_partial_kernel

int rep_chunks(const Geometry& g) { return (g.G * g.S + REP_ROWS - 1) / REP_ROWS; }

struct RankWs {
  double* rep;      // [Hkv][nseg][d]
  double* rpart;    // [Hkv][nseg][rep_chunks][d] partial sums
  uint32_t* keysA;  // [Hkv][L]
  uint32_t* keysB;
  int32_t* valsA;
  int32_t* valsB;
  uint32_t* hist;   // [Hkv * tiles_per_head][DIGITS], per list digit-major
};

RankWs carve(const Geometry& g, const PrefixGeom& p, void* ws) {
  char* c = static_cast<char*>(ws);
  RankWs w;
  const size_t n = (size_t)g.Hkv * p.L;
  w.rep = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hkv * (size_t)p.nseg * g.d);
  w.rpart = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hkv * (size_t)p.nseg * rep_chunks(g) * g.d);
  w.keysA = reinterpret_cast<uint32_t*>(c);
  c += align256(4 * n);
  w.keysB = reinterpret_cast<uint32_t*>(c);
  c += align256(4 * n);
  w.valsA = reinterpret_cast<int32_t*>(c);
  c += align256(4 * n);
  w.valsB = reinterpret_cast<int32_t*>(c);
  c += align256(4 * n);
  w.hist = reinterpret_cast<uint32_t*>(c);
  return w;
}

// ---------------------------------------------------------------------------------------------
// Representative queries: r[g][sigma] = (1 / (G * rows)) * sum over the G heads of g and the rows
// of segment sigma of q.  The segment's G * rows query rows (head-major) are cut into chunks of
// REP_ROWS; one workgroup sums one chunk in fp64 (each thread 8 columns, one 16-byte load per row,
// its row group combined in LDS in a fixed order), and a second kernel adds the chunk sums in
// chunk order, so the result does not depend on scheduling.
template <int D>
__global__ __launch_bounds__(RK_THREADS) void seg_rep_partial_kernel(const uint16_t* q, int64_t qsh, int64_t qst,
                                                                     int N, int S, int G, int nseg, int nch,
                                                                     double* rpart) {
  constexpr int CPR = D / 8;              // threads per row
  constexpr int RP = RK_THREADS / CPR;    // rows per pass
  __shared__ double part[RP][D];
  const int ch = blockIdx.x, sigma = blockIdx.y, g = blockIdx.z, t = threadIdx.x;
  const int c8 = t % CPR, rg = t / CPR;
  const int i0 = sigma * S, len = min(S, N - i0);
  const int r0 = ch * REP_ROWS, r1 = min(r0 + REP_ROWS, G * len);
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = r0 + rg; r < r1; r += RP) {
    const int h = g * G + r / len, i = i0 + r % len;
    const u32x4 v = *reinterpret_cast<const u32x4*>(q + h * qsh + (int64_t)i * qst + c8 * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_bits_to_f32(v[e] & 0xffffu);
      acc[2 * e + 1] += (double)bf16_bits_to_f32(v[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][c8 * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int x = 0; x < RP; ++x) s += part[x][t];
    rpart[(((size_t)g * nseg + sigma) * nch + ch) * D + t] = s;
  }
}

template <int D>
__global__ __launch_bounds__(D) void seg_rep_combine_kernel(const double* rpart, int N, int S, int G, int nseg,
                                                            int nch, double* rep) {
  const int sigma = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int rows = G * min(S, N - sigma * S);
  const int used = (rows + REP_ROWS - 1) / REP_ROWS;
  const double* p = rpart + ((size_t)g * nseg + sigma) * nch * D + t;
  double s = 0.0;
  for (int c = 0; c < used; ++c) s += p[(size_t)c * D];
  rep[((size_t)g * nseg + sigma) * D + t] = s / (double)rows;
}

// Order-preserving key of a score: ascending key = descending score.  The fp64 score is rounded to
// fp32 first, so scores within one fp32 rounding of each other may come out tied (then the
// stable sort keeps them in position order).
__device__ __forceinline__ uint32_t desc_key32(double z) {
  const uint32_t b = __float_as_uint((float)z);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ~o;
}

// Scores of the keys that lie in some prefix (j < (nseg-1)*S), one key per lane (its row read in
// 16-byte chunks), against the representatives of every later segment, 16 at a time; fp64 FMAs.
template <int D>
__global__ __launch_bounds__(RK_THREADS) void prefix_score_kernel(const uint16_t* k, int64_t ksh, int64_t kst,
                                                                  const double* __restrict__ rep, int S, int nseg,
                                                                  int64_t L, uint32_t* keys) {
  constexpr int RG = 16;
  const int g = blockIdx.y, t = threadIdx.x;
  const int nh = (nseg - 1) * S;  // keys that belong to some prefix
  const int j0 = blockIdx.x * RK_THREADS, j = j0 + t;
  const bool live = j < nh;
  const int sj = (live ? j : j0) / S;
  const uint16_t* kp = k + g * ksh + (int64_t)(live ? j : j0) * kst;
  const double* rg_base = rep + (size_t)g * nseg * D;
  for (int s0 = j0 / S + 1; s0 < nseg; s0 += RG) {
    double acc[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) acc[r] = 0.0;
#pragma unroll 2
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 kc = *reinterpret_cast<const u32x4*>(kp + c * 8);  // this lane's key, 8 columns
      double kd[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kd[2 * e] = (double)bf16_bits_to_f32(kc[e] & 0xffffu);
        kd[2 * e + 1] = (double)bf16_bits_to_f32(kc[e] >> 16);
      }
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int sr = min(s0 + r, nseg - 1);  // rows past the last segment repeat it (not written)
        const double* rr = rg_base + (size_t)sr * D + c * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r] = fma(kd[e], rr[e], acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int sigma = s0 + r;
      if (live && sigma < nseg && sigma > sj)
        keys[(size_t)g * L + (size_t)S * sigma * (sigma - 1) / 2 + j] = desc_key32(acc[r]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Stable LSD radix sort of every (g, sigma) list, RADIX_BITS per pass.  A tile of `tile` elements
// is split into contiguous runs of E per thread (E = tile / 256, or one element for the first tile
// threads when tile < 256), so thread order then element order is position order.
struct RadixArgs {
  uint32_t* keys_in;
  uint32_t* keys_out;
  const int32_t* vals_in;  // NULL in the first pass: the value is the position in the list
  int32_t* vals_out;
  uint32_t* hist;
  int S, nseg, tile, tps;
  int64_t L, tiles_per_head;
  int shift;
  bool write_keys;
};

struct TileRef {
  int64_t elem;   // first element of the tile
  int64_t hbase;  // hist base of the tile's list
  int nt;         // tiles of the list
  int t;          // tile within the list
};

__device__ __forceinline__ TileRef tile_ref(const RadixArgs& a, int64_t f) {
  const int g = (int)(f / a.tiles_per_head);
  const int64_t r = f - (int64_t)g * a.tiles_per_head;
  int sigma = 1;
  while ((int64_t)a.tps * sigma * (sigma + 1) / 2 <= r) ++sigma;
  const int64_t first = (int64_t)a.tps * sigma * (sigma - 1) / 2;  // first tile of the list
  TileRef x;
  x.t = (int)(r - first);
  x.nt = a.tps * sigma;
  x.elem = (int64_t)g * a.L + (int64_t)a.S * sigma * (sigma - 1) / 2 + (int64_t)x.t * a.tile;
  x.hbase = (int64_t)DIGITS * ((int64_t)g * a.tiles_per_head + first);
  return x;
}

// LDS layouts padded by one word every 16 counts / every 8 elements, so that a thread walking its
// own 16 counts (or its run of up to 8 elements) and a wave walking consecutive entries both hit
// distinct banks.
__device__ __forceinline__ int cpad(int p) { return p + (p >> 4); }
__device__ __forceinline__ int epad(int i) { return i + (i >> 3); }
constexpr int CNT_WORDS = NIB * RK_THREADS + NIB * RK_THREADS / 16;

// Block-wide exclusive scan, in place, of the NIB x 256 counts in nibble-major order (entry
// p = nibble * 256 + thread at cpad(p)); thread t owns entries 16t .. 16t+15.  cnt then holds each
// (nibble, thread) start within the tile.
__device__ __forceinline__ void scan_counts(uint32_t* cnt, uint32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t v[16];
  uint32_t run = 0;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    v[x] = run;
    run += cnt[cpad(t * 16 + x)];
  }
  uint32_t inc = run;  // inclusive scan of the per-thread totals across the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t base = inc - run;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int x = 0; x < 16; ++x) cnt[cpad(t * 16 + x)] = base + v[x];
  __syncthreads();
}

__device__ __forceinline__ int run_len(int tile) { return tile >= RK_THREADS ? tile / RK_THREADS : 1; }

// Digit histogram of one tile (LDS counters, one per thread), into the list's (digit, tile) table.
__global__ __launch_bounds__(RK_THREADS) void radix_hist_kernel(RadixArgs a) {
  __shared__ uint32_t bins[DIGITS];
  const int t = threadIdx.x;
  const TileRef x = tile_ref(a, blockIdx.x);
  bins[t] = 0;
  __syncthreads();
  for (int i = t; i < a.tile; i += RK_THREADS) atomicAdd(&bins[(a.keys_in[x.elem + i] >> a.shift) & (DIGITS - 1)], 1u);
  __syncthreads();
  a.hist[x.hbase + (int64_t)t * x.nt + x.t] = bins[t];
}

// Exclusive scan over the workgroup of one value per thread (wsum: one word per wave).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t base = inc - v;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  __syncthreads();
  return base;
}

// Exclusive scan of one list's histogram in (digit, tile) order: the first output position of
// every (digit, tile) in the list.  Each thread scans one contiguous slice of the table.
constexpr int SCAN_THREADS = 1024;
__global__ __launch_bounds__(SCAN_THREADS) void radix_scan_kernel(RadixArgs a) {
  __shared__ uint32_t wsum[SCAN_THREADS / 64];
  const int t = threadIdx.x;
  const int g = blockIdx.x / (a.nseg - 1), sigma = blockIdx.x % (a.nseg - 1) + 1;
  const int64_t first = (int64_t)a.tps * sigma * (sigma - 1) / 2;
  uint32_t* h = a.hist + (int64_t)DIGITS * ((int64_t)g * a.tiles_per_head + first);
  const int n = DIGITS * a.tps * sigma;
  const int m = (n + SCAN_THREADS - 1) / SCAN_THREADS;
  const int b = min(t * m, n), e = min(b + m, n);
  uint32_t sum = 0;
  for (int i = b; i < e; ++i) sum += h[i];
  uint32_t run = block_exclusive_scan(sum, wsum);
  for (int i = b; i < e; ++i) {
    const uint32_t v = h[i];
    h[i] = run;
    run += v;
  }
}

// Stable reorder of the tile in LDS by the 4 key bits at `shift`: each thread ranks its run of E
// consecutive elements, the 16 x 256 counts are scanned block-wide.
__device__ __forceinline__ void lds_nibble_sort(uint32_t* skey, int32_t* sval, uint32_t* cnt, uint32_t* wsum, int E,
                                                int n, int shift) {
  const int t = threadIdx.x;
  uint32_t kv[8];
  int32_t vv[8];
  uint64_t c = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e < n) {
      kv[e] = skey[epad(t * E + e)];
      vv[e] = sval[epad(t * E + e)];
      c += 1ull << (4 * ((kv[e] >> shift) & (NIB - 1)));
    }
  }
#pragma unroll
  for (int d = 0; d < NIB; ++d) cnt[cpad(d * RK_THREADS + t)] = (uint32_t)(c >> (4 * d)) & 15u;
  __syncthreads();  // also: every run is in registers before the tile is reordered in place
  scan_counts(cnt, wsum);
  uint64_t seen = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e >= n) break;
    const uint32_t d = (kv[e] >> shift) & (NIB - 1);
    const int pos = (int)(cnt[cpad(d * RK_THREADS + t)] + ((uint32_t)(seen >> (4 * d)) & 15u));
    seen += 1ull << (4 * d);
    skey[epad(pos)] = kv[e];
    sval[epad(pos)] = vv[e];
  }
  __syncthreads();
}

// Scatter of one tile: the tile is read with striped loads into LDS, sorted there by its 8-bit
// digit (two stable 4-bit reorders), and stored with striped stores, so each digit's run lands
// contiguously at its offset in the list.
constexpr int MAX_TILE = 2048;
__global__ __launch_bounds__(RK_THREADS) void radix_scatter_kernel(RadixArgs a) {
  __shared__ uint32_t cnt[CNT_WORDS];
  __shared__ uint32_t wsum[RK_THREADS / 64];
  __shared__ uint32_t skey[MAX_TILE + MAX_TILE / 8];
  __shared__ int32_t sval[MAX_TILE + MAX_TILE / 8];
  __shared__ uint32_t bins[DIGITS];   // tile counts, then the tile-local start of each digit
  __shared__ uint32_t gofs[DIGITS];   // list offset of each digit's run from this tile
  const int t = threadIdx.x;
  const TileRef x = tile_ref(a, blockIdx.x);
  const int E = run_len(a.tile);
  const int n = (a.tile >= RK_THREADS || t < a.tile) ? E : 0;
  const int64_t lbase = x.elem - (int64_t)x.t * a.tile;  // first element of the list
  // this tile's count of digit t: the gap to the next (digit, tile) entry of the scanned table
  const int64_t hi = x.hbase + (int64_t)t * x.nt + x.t;
  const uint32_t o = a.hist[hi];
  const uint32_t next = (t == DIGITS - 1 && x.t == x.nt - 1) ? (uint32_t)(x.nt * a.tile) : a.hist[hi + 1];
  gofs[t] = o;
  for (int i = t; i < a.tile; i += RK_THREADS) {
    skey[epad(i)] = a.keys_in[x.elem + i];
    sval[epad(i)] = a.vals_in ? a.vals_in[x.elem + i] : (int32_t)(x.t * a.tile + i);
  }
  bins[t] = block_exclusive_scan(next - o, wsum);  // its barriers also publish skey, sval
  lds_nibble_sort(skey, sval, cnt, wsum, E, n, a.shift);
  lds_nibble_sort(skey, sval, cnt, wsum, E, n, a.shift + 4);
  for (int i = t; i < a.tile; i += RK_THREADS) {
    const uint32_t key = skey[epad(i)];
    const uint32_t d = (key >> a.shift) & (DIGITS - 1);
    const int64_t dst = lbase + gofs[d] + (i - bins[d]);
    if (a.write_keys) a.keys_out[dst] = key;
    a.vals_out[dst] = sval[epad(i)];
  }
}

// S2O query permutation (Methodology 1, Query Permutation): score of position i for KV head g =
// (1/G) * sum over the G query heads of q_{h,i} . u_g, u_g the mean key (the shared guide vector);
// one lane per position, u_g read through scalar loads, fp64.
template <int D>
__global__ __launch_bounds__(RK_THREADS) void query_guide_kernel(const uint16_t* q, int64_t qsh, int64_t qst, int N,
                                                                 int G, const double* __restrict__ u, double* score) {
  const int g = blockIdx.y, i = blockIdx.x * RK_THREADS + threadIdx.x;
  if (i >= N) return;
  const double* ug = u + (size_t)g * D;
  double tot = 0.0;
  for (int h = g * G; h < (g + 1) * G; ++h) {
    const uint16_t* qp = q + h * qsh + (int64_t)i * qst;
    double acc = 0.0;
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + c * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fma((double)bf16_bits_to_f32(v[e] & 0xffffu), ug[c * 8 + 2 * e], acc);
        acc = fma((double)bf16_bits_to_f32(v[e] >> 16), ug[c * 8 + 2 * e + 1], acc);
      }
    }
    tot += acc;
  }
  score[(size_t)g * N + i] = tot / (double)G;
}

}  // namespace

size_t query_perm_workspace_bytes(const Geometry& g) {
  const int nch = (g.N + REP_ROWS - 1) / REP_ROWS;
  return align256(sizeof(double) * g.Hkv * (size_t)nch * g.d) + align256(sizeof(double) * g.Hkv * g.d) +
         align256(sizeof(double) * g.Hkv * (size_t)g.N);
}

hipError_t launch_query_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* qperm, void* ws,
                                    hipStream_t st) {
  // the mean key of each KV head: the representative-query kernels over one "segment" of all N
  // key rows of one head (G = 1)
  const int nch = (g.N + REP_ROWS - 1) / REP_ROWS;
  char* c = static_cast<char*>(ws);
  double* upart = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hkv * (size_t)nch * g.d);
  double* u = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hkv * g.d);
  double* score = reinterpret_cast<double*>(c);
  const dim3 rgrid(nch, 1, g.Hkv), sgrid((g.N + RK_THREADS - 1) / RK_THREADS, g.Hkv);
  if (g.d == 128) {
    seg_rep_partial_kernel<128><<<rgrid, RK_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.N, 1, 1, nch, upart);
    seg_rep_combine_kernel<128><<<dim3(1, g.Hkv), 128, 0, st>>>(upart, g.N, g.N, 1, 1, nch, u);
    query_guide_kernel<128><<<sgrid, RK_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.G, u, score);
  } else {
    seg_rep_partial_kernel<64><<<rgrid, RK_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.N, 1, 1, nch, upart);
    seg_rep_combine_kernel<64><<<dim3(1, g.Hkv), 64, 0, st>>>(upart, g.N, g.N, 1, 1, nch, u);
    query_guide_kernel<64><<<sgrid, RK_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.G, u, score);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_segment_sort(g, score, qperm, st);
}

size_t prefix_rank_workspace_bytes(const Geometry& g) {
  const PrefixGeom p = prefix_geom(g);
  const size_t n = (size_t)g.Hkv * p.L;
  return align256(sizeof(double) * g.Hkv * (size_t)p.nseg * g.d) +
         align256(sizeof(double) * g.Hkv * (size_t)p.nseg * rep_chunks(g) * g.d) + 4 * align256(4 * n) +
         align256(sizeof(uint32_t) * DIGITS * (size_t)g.Hkv * p.tiles_per_head);
}

int64_t prefix_rank_length(const Geometry& g) { return prefix_geom(g).L; }

hipError_t launch_prefix_rank(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* kv_rank, void* ws,
                              hipStream_t st) {
  const PrefixGeom p = prefix_geom(g);
  if (p.nseg < 2) return hipSuccess;  // no segment has a prefix
  const RankWs w = carve(g, p, ws);
  const int nch = rep_chunks(g);
  const dim3 rgrid(nch, p.nseg, g.Hkv);
  if (g.d == 128) {
    seg_rep_partial_kernel<128><<<rgrid, RK_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.S, g.G, p.nseg, nch, w.rpart);
    seg_rep_combine_kernel<128><<<dim3(p.nseg, g.Hkv), 128, 0, st>>>(w.rpart, g.N, g.S, g.G, p.nseg, nch, w.rep);
  } else {
    seg_rep_partial_kernel<64><<<rgrid, RK_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.S, g.G, p.nseg, nch, w.rpart);
    seg_rep_combine_kernel<64><<<dim3(p.nseg, g.Hkv), 64, 0, st>>>(w.rpart, g.N, g.S, g.G, p.nseg, nch, w.rep);
  }
  const int nh = (p.nseg - 1) * g.S;
  const dim3 sgrid((nh + RK_THREADS - 1) / RK_THREADS, g.Hkv);
  if (g.d == 128)
    prefix_score_kernel<128><<<sgrid, RK_THREADS, 0, st>>>(k, g.kvsh, g.kvst, w.rep, g.S, p.nseg, p.L, w.keysA);
  else
    prefix_score_kernel<64><<<sgrid, RK_THREADS, 0, st>>>(k, g.kvsh, g.kvst, w.rep, g.S, p.nseg, p.L, w.keysA);
  RadixArgs a;
  a.hist = w.hist;
  a.S = g.S;
  a.nseg = p.nseg;
  a.tile = p.tile;
  a.tps = p.tps;
  a.L = p.L;
  a.tiles_per_head = p.tiles_per_head;
  const int64_t tiles = (int64_t)g.Hkv * p.tiles_per_head;
  const int lists = g.Hkv * (p.nseg - 1);
  for (int pass = 0; pass < RADIX_PASSES; ++pass) {
    const bool even = (pass & 1) == 0;
    a.keys_in = even ? w.keysA : w.keysB;
    a.keys_out = even ? w.keysB : w.keysA;
    a.vals_in = pass == 0 ? nullptr : (even ? w.valsA : w.valsB);
    a.vals_out = pass == RADIX_PASSES - 1 ? kv_rank : (even ? w.valsB : w.valsA);
    a.shift = pass * RADIX_BITS;
    a.write_keys = pass != RADIX_PASSES - 1;
    radix_hist_kernel<<<(unsigned)tiles, RK_THREADS, 0, st>>>(a);
    radix_scan_kernel<<<lists, SCAN_THREADS, 0, st>>>(a);
    radix_scatter_kernel<<<(unsigned)tiles, RK_THREADS, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pbsa
