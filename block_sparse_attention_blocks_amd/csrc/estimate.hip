// Stage 1 (key importance, segment sort) and stage 2 (pooling, block selection) on gfx950.
//
// Everything here is fp64: bf16 x bf16 products are exact in fp64, block means of bf16 rows are
// exact sums divided by a power of two, and the ranks and cumulative-mass cuts these kernels
// decide must agree with an fp64 evaluation of the same definitions bit for bit except at
// genuine near-ties.  fp32 accumulation would swap ranks whose gaps are far above the tie band.
#include "common.h"

#include <math.h>

namespace pbsa {

// =====================================================================================
// Stage 1a: key importance (Sparser Block-Sparse Attention via Token Permutation, section 3,
// "Proxy Scoring").  The proxy rows of KV head g are (h, i) with h in g's query-head group and
// i in [N - R1, N), R1 = min(B, N); there are R = G * R1 of them.  Row r maps to
// h = g*G + r / R1, i = N - R1 + r % R1.  Three launches:
//   imp_partial : per (key chunk, g) and row, the chunk's max logit and sum of exp(logit - max)
//   imp_lse     : per (row, g), combine the chunk partials into the row's log-sum-exp
//   imp_accum   : per (key chunk, g), sum over rows of exp(logit - lse), divided by R
// The logits are recomputed in imp_accum rather than stored.
// =====================================================================================

constexpr int IMP_CK = 64;       // keys per workgroup
constexpr int IMP_RT = 64;       // proxy rows per inner tile
constexpr int IMP_THREADS = 256;  // 16 row groups x 16 key groups, 4 x 4 logits per thread

struct ImpWs {
  double* part_m;  // [Hkv][nchunk][R]
  double* part_l;  // [Hkv][nchunk][R]
  double* lse;     // [Hkv][R]
  double* imp;     // [Hkv][N] (used when the caller passes no importance output)
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

static inline int imp_rows(const Geometry& g) { return g.G * (g.N < g.B ? g.N : g.B); }
static inline int imp_chunks(const Geometry& g) { return (g.N + IMP_CK - 1) / IMP_CK; }

static ImpWs carve_imp_ws(const Geometry& g, void* ws) {
  const size_t R = imp_rows(g), C = imp_chunks(g);
  char* p = static_cast<char*>(ws);
  ImpWs w;
  w.part_m = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * C * R);
  w.part_l = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * C * R);
  w.lse = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * R);
  w.imp = reinterpret_cast<double*>(p);
  return w;
}

size_t importance_workspace_bytes(const Geometry& g) {
  const size_t R = imp_rows(g), C = imp_chunks(g);
  return 2 * align256(sizeof(double) * g.Hkv * C * R) + align256(sizeof(double) * g.Hkv * R) +
         align256(sizeof(double) * g.Hkv * (size_t)g.N);
}

// Load a [rows][d] bf16 tile into LDS transposed as fp32 [d][IMP_CK] (zeros for invalid rows).
// Lane -> row mapping keeps LDS writes conflict-free; each lane reads 16 bytes of its row.
__device__ __forceinline__ void imp_load_tile_T(float* dst, const uint16_t* base, int64_t row_stride,
                                                const int* row_pos, int d) {
  const int t = threadIdx.x;
  const int row = t & (IMP_CK - 1);
  const int pos = row_pos[row];
  for (int dg = t >> 6; dg < d / 8; dg += IMP_THREADS / 64) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (pos >= 0) raw = *reinterpret_cast<const u32x4*>(base + (int64_t)pos * row_stride + dg * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(dg * 8 + 2 * e) * IMP_CK + row] = bf16_bits_to_f32(raw[e] & 0xffffu);
      dst[(dg * 8 + 2 * e + 1) * IMP_CK + row] = bf16_bits_to_f32(raw[e] >> 16);
    }
  }
}

// 4 x 4 fp64 logits of this thread: rows rg*4.., keys kg*4.. of the tile (unscaled dot products).
__device__ __forceinline__ void imp_tile_dots(const float* qT, const float* kT, int d, double acc[4][4]) {
  const int t = threadIdx.x;
  const int rg = t >> 4, kg = t & 15;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int dd = 0; dd < d; ++dd) {
    const f32x4 qv = *reinterpret_cast<const f32x4*>(qT + dd * IMP_CK + rg * 4);
    const f32x4 kv = *reinterpret_cast<const f32x4*>(kT + dd * IMP_CK + kg * 4);
    double qd[4], kd[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) { qd[a] = (double)qv[a]; kd[a] = (double)kv[a]; }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = fma(qd[a], kd[b], acc[a][b]);
  }
}

struct ImpArgs {
  const uint16_t* q;
  const uint16_t* k;
  int N, G, d, R1, R;
  int64_t qsh, qst, kvsh, kvst;
  double scale;
};

// Proxy row r of KV head g -> (query head, token position).
__device__ __forceinline__ void imp_row(const ImpArgs& a, int g, int r, int* h, int* i) {
  *h = g * a.G + r / a.R1;
  *i = a.N - a.R1 + r % a.R1;
}

__global__ __launch_bounds__(IMP_THREADS) void imp_partial_kernel(ImpArgs a, double* part_m, double* part_l) {
  __shared__ __align__(16) float qT[128 * IMP_CK];
  __shared__ __align__(16) float kT[128 * IMP_CK];
  __shared__ int kpos[IMP_CK];
  __shared__ int qpos[IMP_RT];
  __shared__ int qpos_i[IMP_RT];
  const int chunk = blockIdx.x, g = blockIdx.y, nchunk = gridDim.x;
  const int t = threadIdx.x, rg = t >> 4, kg = t & 15;
  const int j0 = chunk * IMP_CK;
  if (t < IMP_CK) kpos[t] = (j0 + t < a.N) ? j0 + t : -1;
  __syncthreads();
  imp_load_tile_T(kT, a.k + (int64_t)g * a.kvsh, a.kvst, kpos, a.d);
  for (int r0 = 0; r0 < a.R; r0 += IMP_RT) {
    __syncthreads();
    if (t < IMP_RT) {
      int h, i;
      const int r = r0 + t;
      if (r < a.R) {
        imp_row(a, g, r, &h, &i);
        qpos[t] = i;
        qpos_i[t] = i;
      } else {
        qpos[t] = -1;
        qpos_i[t] = -1;
      }
    }
    __syncthreads();
    // rows of one tile may span two query heads: load each row from its own head
    {
      const int row = t & (IMP_RT - 1);
      const int r = r0 + row;
      const int pos = qpos[row];
      int h = 0, i = 0;
      if (r < a.R) imp_row(a, g, r, &h, &i);
      const uint16_t* qrow = a.q + (int64_t)h * a.qsh + (int64_t)pos * a.qst;
      for (int dg = t >> 6; dg < a.d / 8; dg += IMP_THREADS / 64) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (pos >= 0) raw = *reinterpret_cast<const u32x4*>(qrow + dg * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qT[(dg * 8 + 2 * e) * IMP_CK + row] = bf16_bits_to_f32(raw[e] & 0xffffu);
          qT[(dg * 8 + 2 * e + 1) * IMP_CK + row] = bf16_bits_to_f32(raw[e] >> 16);
        }
      }
    }
    __syncthreads();
    double acc[4][4];
    imp_tile_dots(qT, kT, a.d, acc);
#pragma unroll
    for (int ra = 0; ra < 4; ++ra) {
      const int row = rg * 4 + ra;
      const int i = qpos_i[row];
      double s[4];
      double m = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = kpos[kg * 4 + b];
        const bool ok = (i >= 0) && (j >= 0) && (j <= i);
        s[b] = ok ? a.scale * acc[ra][b] : -INFINITY;
        m = fmax(m, s[b]);
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 16));
      double l = 0.0;
      if (m > -INFINITY) {
#pragma unroll
        for (int b = 0; b < 4; ++b) l += (s[b] > -INFINITY) ? exp(s[b] - m) : 0.0;
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) l += __shfl_xor(l, o, 16);
      const int r = r0 + row;
      if (kg == 0 && r < a.R) {
        const size_t o = ((size_t)g * nchunk + chunk) * a.R + r;
        part_m[o] = m;
        part_l[o] = l;
      }
    }
  }
}

__global__ __launch_bounds__(256) void imp_lse_kernel(const double* part_m, const double* part_l, int nchunk,
                                                      int R, double* lse) {
  __shared__ double sm[4], sl[4];
  const int r = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const double* pm = part_m + (size_t)g * nchunk * R + r;
  const double* pl = part_l + (size_t)g * nchunk * R + r;
  double m = -INFINITY;
  for (int c = t; c < nchunk; c += 256) m = fmax(m, pm[(size_t)c * R]);
  m = wave_max_f64(m);
  if ((t & 63) == 0) sm[t >> 6] = m;
  __syncthreads();
  m = fmax(fmax(sm[0], sm[1]), fmax(sm[2], sm[3]));
  double l = 0.0;
  for (int c = t; c < nchunk; c += 256) {
    const double mc = pm[(size_t)c * R];
    if (mc > -INFINITY) l += pl[(size_t)c * R] * exp(mc - m);
  }
  l = wave_sum_f64(l);
  if ((t & 63) == 0) sl[t >> 6] = l;
  __syncthreads();
  if (t == 0) lse[(size_t)g * R + r] = m + log((sl[0] + sl[1]) + (sl[2] + sl[3]));
}

__global__ __launch_bounds__(IMP_THREADS) void imp_accum_kernel(ImpArgs a, const double* lse, double* imp) {
  __shared__ __align__(16) float qT[128 * IMP_CK];
  __shared__ __align__(16) float kT[128 * IMP_CK];
  __shared__ int kpos[IMP_CK];
  __shared__ int qpos[IMP_RT];
  __shared__ double rlse[IMP_RT];
  __shared__ double red[16][IMP_CK];
  const int chunk = blockIdx.x, g = blockIdx.y;
  const int t = threadIdx.x, rg = t >> 4, kg = t & 15;
  const int j0 = chunk * IMP_CK;
  if (t < IMP_CK) kpos[t] = (j0 + t < a.N) ? j0 + t : -1;
  __syncthreads();
  imp_load_tile_T(kT, a.k + (int64_t)g * a.kvsh, a.kvst, kpos, a.d);
  double colsum[4] = {0.0, 0.0, 0.0, 0.0};
  for (int r0 = 0; r0 < a.R; r0 += IMP_RT) {
    __syncthreads();
    if (t < IMP_RT) {
      const int r = r0 + t;
      if (r < a.R) {
        int h, i;
        imp_row(a, g, r, &h, &i);
        qpos[t] = i;
        rlse[t] = lse[(size_t)g * a.R + r];
      } else {
        qpos[t] = -1;
        rlse[t] = 0.0;
      }
    }
    __syncthreads();
    {
      const int row = t & (IMP_RT - 1);
      const int r = r0 + row;
      const int pos = qpos[row];
      int h = 0, i = 0;
      if (r < a.R) imp_row(a, g, r, &h, &i);
      const uint16_t* qrow = a.q + (int64_t)h * a.qsh + (int64_t)pos * a.qst;
      for (int dg = t >> 6; dg < a.d / 8; dg += IMP_THREADS / 64) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (pos >= 0) raw = *reinterpret_cast<const u32x4*>(qrow + dg * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qT[(dg * 8 + 2 * e) * IMP_CK + row] = bf16_bits_to_f32(raw[e] & 0xffffu);
          qT[(dg * 8 + 2 * e + 1) * IMP_CK + row] = bf16_bits_to_f32(raw[e] >> 16);
        }
      }
    }
    __syncthreads();
    double acc[4][4];
    imp_tile_dots(qT, kT, a.d, acc);
#pragma unroll
    for (int ra = 0; ra < 4; ++ra) {
      const int row = rg * 4 + ra;
      const int i = qpos[row];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = kpos[kg * 4 + b];
        if (i >= 0 && j >= 0 && j <= i) colsum[b] += exp(a.scale * acc[ra][b] - rlse[row]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) red[rg][kg * 4 + b] = colsum[b];
  __syncthreads();
  if (t < IMP_CK) {
    double s = 0.0;
    for (int x = 0; x < 16; ++x) s += red[x][t];
    const int j = j0 + t;
    if (j < a.N) imp[(size_t)g * a.N + j] = s / (double)a.R;
  }
}

static hipError_t launch_key_importance(const Geometry& g, const uint16_t* q, const uint16_t* k, double* out,
                                        void* ws, hipStream_t st) {
  ImpWs w = carve_imp_ws(g, ws);
  ImpArgs a;
  a.q = q;
  a.k = k;
  a.N = g.N;
  a.G = g.G;
  a.d = g.d;
  a.R1 = g.N < g.B ? g.N : g.B;
  a.R = g.G * a.R1;
  a.qsh = g.qsh;
  a.qst = g.qst;
  a.kvsh = g.kvsh;
  a.kvst = g.kvst;
  a.scale = g.scale64;
  const int nchunk = imp_chunks(g);
  imp_partial_kernel<<<dim3(nchunk, g.Hkv), IMP_THREADS, 0, st>>>(a, w.part_m, w.part_l);
  imp_lse_kernel<<<dim3(a.R, g.Hkv), 256, 0, st>>>(w.part_m, w.part_l, nchunk, a.R, w.lse);
  imp_accum_kernel<<<dim3(nchunk, g.Hkv), IMP_THREADS, 0, st>>>(a, w.lse, out);
  return hipGetLastError();
}

// =====================================================================================
// Stage 1b: sort inside segments (section 3, "Sorting"): importance descending, ties by
// position ascending.  One workgroup per (segment, KV head); bitonic sort in LDS on the
// 64-bit key ~bits(imp) (imp >= 0, so the bit pattern orders like the value) with the
// position as the second key.
// =====================================================================================

constexpr int SORT_MAX = 8192;
constexpr int SORT_THREADS = 512;

__global__ __launch_bounds__(SORT_THREADS) void segment_sort_kernel(const double* imp, int32_t* perm, int N, int S) {
  __shared__ uint64_t key[SORT_MAX];
  __shared__ uint16_t off[SORT_MAX];
  const int seg = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int a = seg * S;
  const int L = min(S, N - a);
  int n = 1;
  while (n < L) n <<= 1;
  for (int x = t; x < n; x += SORT_THREADS) {
    if (x < L) {
      double v = imp[(size_t)g * N + a + x];
      uint64_t b = (v > 0.0) ? (uint64_t)__double_as_longlong(v) : 0ull;
      key[x] = ~b;
      off[x] = (uint16_t)x;
    } else {
      key[x] = ~0ull;
      off[x] = 0xffffu;
    }
  }
  __syncthreads();
  for (int kk = 2; kk <= n; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int x = t; x < n; x += SORT_THREADS) {
        const int y = x ^ j;
        if (y > x) {
          const uint64_t kx = key[x], ky = key[y];
          const uint16_t ox = off[x], oy = off[y];
          const bool gt = (kx > ky) || (kx == ky && ox > oy);
          const bool up = (x & kk) == 0;
          if (gt == up) {
            key[x] = ky;
            key[y] = kx;
            off[x] = oy;
            off[y] = ox;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int x = t; x < L; x += SORT_THREADS) perm[(size_t)g * N + a + x] = a + (int)off[x];
}

hipError_t launch_build_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* perm,
                                    double* imp, void* ws, hipStream_t st) {
  double* out = imp ? imp : carve_imp_ws(g, ws).imp;
  hipError_t e = launch_key_importance(g, q, k, out, ws, st);
  if (e != hipSuccess) return e;
  const int nseg = (g.N + g.S - 1) / g.S;
  segment_sort_kernel<<<dim3(nseg, g.Hkv), SORT_THREADS, 0, st>>>(out, perm, g.N, g.S);
  return hipGetLastError();
}

// =====================================================================================
// Stage 2a: mean pooling (section 4, "Block Selection": mean pooling on the permuted keys).
// dst[h][J][:] = mean over the rows of block J of src[h][row][:], where the rows are natural
// (rowmap == NULL) or rowmap[h][J*B + t].  Sums of bf16 values are exact in fp64.
// =====================================================================================

constexpr int POOL_THREADS = 256;

__global__ __launch_bounds__(POOL_THREADS) void pool_kernel(const uint16_t* src, int64_t sh, int64_t st_,
                                                            int N, int B, int d, const int32_t* rowmap,
                                                            double* dst, int NB) {
  __shared__ double part[32][128];
  const int J = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lanes = d / 8;                 // threads per row
  const int rp = POOL_THREADS / lanes;     // rows in flight
  const int c = t % lanes, rs = t / lanes;
  const int r0 = J * B;
  const int cnt = min(B, N - r0);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = src + (int64_t)h * sh;
  for (int r = rs; r < cnt; r += rp) {
    const int pos = rowmap ? rowmap[(size_t)h * N + r0 + r] : r0 + r;
    if (pos < 0 || pos >= N) continue;  // a corrupt index list contributes nothing
    const u32x4 raw = *reinterpret_cast<const u32x4*>(base + (int64_t)pos * st_ + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)bf16_bits_to_f32(raw[e] & 0xffffu);
      acc[2 * e + 1] += (double)bf16_bits_to_f32(raw[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rs][c * 8 + e] = acc[e];
  __syncthreads();
  if (t < d) {
    double s = 0.0;
    for (int x = 0; x < rp; ++x) s += part[x][t];
    dst[((size_t)h * NB + J) * d + t] = s / (double)cnt;
  }
}

// =====================================================================================
// Stage 2b: block selection.  One workgroup per (query block I, query head h):
// z_J = c * Qbar . Kbar_J (J <= I), p = softmax(z) in fp64, bitonic sort on (p desc, J asc),
// inclusive scan of the sorted p, k* = first prefix with mass >= tau, forced blocks, and an
// ascending compaction of the kept set.
// =====================================================================================

constexpr int SEL_THREADS = 256;
constexpr int SEL_MAX = 2048;

struct SelArgs {
  const double* qbar;   // [Hq][NB][d]
  const double* knat;   // [Hkv][NB][d]
  const double* kperm;  // [Hkv][NB][d] or NULL
  int NB, G, d, B, S;
  double scale, tau;
  uint32_t flags;
  int32_t* count;
  int32_t* idx;
  double* prob;
};

__device__ __forceinline__ double block_reduce_max(double x, double* sh) {
  x = wave_max_f64(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  return fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3]));
}

__device__ __forceinline__ double block_reduce_sum(double x, double* sh) {
  x = wave_sum_f64(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__global__ __launch_bounds__(SEL_THREADS) void block_select_kernel(SelArgs a) {
  __shared__ double qb[128];
  __shared__ double pv[SEL_MAX];     // z, then p (by J), then the inclusive scan (by rank)
  __shared__ uint64_t key[SEL_MAX];  // ~bits(p), sorted ascending
  __shared__ uint16_t jid[SEL_MAX];
  __shared__ uint8_t sel[SEL_MAX];
  __shared__ double red[4];
  __shared__ int kstar_sh;
  const int I = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int g = h / a.G;
  const int nJ = I + 1;
  const int sI = (a.S > 0) ? (I * a.B) / a.S : 0;
  if (t < a.d) qb[t] = a.qbar[((size_t)h * a.NB + I) * a.d + t];
  __syncthreads();
  // pooled logits, one wave per J
  for (int J = w; J < nJ; J += SEL_THREADS / 64) {
    const bool permuted = a.kperm && (((J * a.B) / a.S) < sI);
    const double* kb = (permuted ? a.kperm : a.knat) + ((size_t)g * a.NB + J) * a.d;
    double s = 0.0;
    for (int e = lane; e < a.d; e += 64) s = fma(qb[e], kb[e], s);
    s = wave_sum_f64(s);
    if (lane == 0) pv[J] = a.scale * s;
  }
  __syncthreads();
  double m = -INFINITY;
  for (int J = t; J < nJ; J += SEL_THREADS) m = fmax(m, pv[J]);
  m = block_reduce_max(m, red);
  double se = 0.0;
  for (int J = t; J < nJ; J += SEL_THREADS) {
    const double e = exp(pv[J] - m);
    pv[J] = e;
    se += e;
  }
  se = block_reduce_sum(se, red);
  int n = 1;
  while (n < nJ) n <<= 1;
  const size_t tri = (size_t)h * ((size_t)a.NB * (a.NB + 1) / 2) + (size_t)tri_offset(I);
  for (int J = t; J < n; J += SEL_THREADS) {
    if (J < nJ) {
      const double p = pv[J] / se;
      if (a.prob) a.prob[tri + J] = p;
      key[J] = ~(uint64_t)__double_as_longlong(p > 0.0 ? p : 0.0);
      jid[J] = (uint16_t)J;
      sel[J] = 0;
    } else {
      key[J] = ~0ull;
      jid[J] = 0xffffu;
    }
  }
  __syncthreads();
  for (int kk = 2; kk <= n; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int x = t; x < n; x += SEL_THREADS) {
        const int y = x ^ j;
        if (y > x) {
          const uint64_t kx = key[x], ky = key[y];
          const uint16_t ox = jid[x], oy = jid[y];
          const bool gt = (kx > ky) || (kx == ky && ox > oy);
          if (gt == ((x & kk) == 0)) {
            key[x] = ky;
            key[y] = kx;
            jid[x] = oy;
            jid[y] = ox;
          }
        }
      }
      __syncthreads();
    }
  }
  int kstar = nJ;
  if (a.tau < 1.0) {
    // inclusive scan of the sorted probabilities (Hillis-Steele, values staged in registers)
    constexpr int PER = SEL_MAX / SEL_THREADS;
    double vals[PER];
    for (int x = 0; x < PER; ++x) {
      const int r = t + x * SEL_THREADS;
      vals[x] = (r < nJ) ? __longlong_as_double((long long)~key[r]) : 0.0;
      if (r < n) pv[r] = vals[x];
    }
    __syncthreads();
    for (int o = 1; o < n; o <<= 1) {
      double add[PER];
      for (int x = 0; x < PER; ++x) {
        const int r = t + x * SEL_THREADS;
        add[x] = (r < n && r >= o) ? pv[r - o] : 0.0;
      }
      __syncthreads();
      for (int x = 0; x < PER; ++x) {
        const int r = t + x * SEL_THREADS;
        if (r < n) pv[r] += add[x];
      }
      __syncthreads();
    }
    if (t == 0) kstar_sh = nJ;
    __syncthreads();
    int first = nJ;
    for (int r = t; r < nJ; r += SEL_THREADS)
      if (pv[r] >= a.tau) first = min(first, r + 1);
    if (first < nJ) atomicMin(&kstar_sh, first);
    __syncthreads();
    kstar = kstar_sh;
  }
  for (int r = t; r < kstar; r += SEL_THREADS) sel[jid[r]] = 1;
  __syncthreads();
  if (t == 0) {
    if (a.flags & 1u) sel[I] = 1;
    if (a.flags & 2u) sel[0] = 1;
  }
  __syncthreads();
  if (w == 0) {
    int base = 0;
    for (int J0 = 0; J0 < nJ; J0 += 64) {
      const int J = J0 + lane;
      const bool f = (J < nJ) && sel[J];
      const unsigned long long bal = __ballot(f);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (f) a.idx[tri + pos] = J;
      base += __popcll(bal);
    }
    if (lane == 0) a.count[(size_t)h * a.NB + I] = base;
  }
}

size_t mask_workspace_bytes(const Geometry& g) {
  const size_t NB = g.NB;
  return align256(sizeof(double) * g.Hq * NB * g.d) + 2 * align256(sizeof(double) * g.Hkv * NB * g.d);
}

hipError_t launch_block_mask(const Geometry& g, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                             double tau, uint32_t flags, int32_t* count, int32_t* idx, double* prob,
                             void* ws, hipStream_t st) {
  char* p = static_cast<char*>(ws);
  double* qbar = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hq * (size_t)g.NB * g.d);
  double* knat = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)g.NB * g.d);
  double* kperm = reinterpret_cast<double*>(p);
  pool_kernel<<<dim3(g.NB, g.Hq), POOL_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.B, g.d, nullptr, qbar, g.NB);
  pool_kernel<<<dim3(g.NB, g.Hkv), POOL_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.B, g.d, nullptr, knat, g.NB);
  if (perm)
    pool_kernel<<<dim3(g.NB, g.Hkv), POOL_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.B, g.d, perm, kperm, g.NB);
  SelArgs a;
  a.qbar = qbar;
  a.knat = knat;
  a.kperm = perm ? kperm : nullptr;
  a.NB = g.NB;
  a.G = g.G;
  a.d = g.d;
  a.B = g.B;
  a.S = g.S;
  a.scale = g.scale64;
  a.tau = tau;
  a.flags = flags;
  a.count = count;
  a.idx = idx;
  a.prob = prob;
  block_select_kernel<<<dim3(g.NB, g.Hq), SEL_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace pbsa
