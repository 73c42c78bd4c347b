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
// h = g*G + r / R1, i = N - R1 + r % R1.  imp_j = (1/R) sum_r exp(s_rj - lse_r), s_rj = c q_r.k_j
// over causal j <= i.  Three launches:
//   imp_scores : per (64-key chunk c, g), the fp64 logits of all R rows on the fp64 matrix cores
//                (v_mfma_f64_16x16x4_f64); per row the chunk max m_cr and l_cr = sum exp(s - m_cr),
//                and e_rj = exp(s_rj - m_cr) stored to the workspace
//   imp_lse    : per (row, g), lse_r = M + log sum_c l_cr exp(m_cr - M)
//   imp_colsum : per key, imp_j = (1/R) sum_r e_rj exp(m_c(j)r - lse_r) in row order
// so every logit is computed once and exponentiated once.
// =====================================================================================

constexpr int IMP_CK = 64;        // keys per workgroup (4 MFMA tiles of 16)
constexpr int IMP_RT = 64;        // proxy rows per inner tile (4 waves x 16 rows)
constexpr int IMP_THREADS = 256;
constexpr int IMP_PITCH = 132;    // fp32 LDS row pitch: 16 rows x 4 k hit 64 distinct banks
constexpr int COL_KEYS = 256;     // keys per workgroup of imp_colsum
constexpr int COL_ROWS = 256;     // rows staged per pass of imp_colsum

typedef double f64x4 __attribute__((ext_vector_type(4)));

struct ImpWs {
  double* e;       // [Hkv][R][N] chunk-normalised exponentials
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
  w.e = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * R * (size_t)g.N);
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
  return align256(sizeof(double) * g.Hkv * R * (size_t)g.N) + 2 * align256(sizeof(double) * g.Hkv * C * R) +
         align256(sizeof(double) * g.Hkv * R) + align256(sizeof(double) * g.Hkv * (size_t)g.N);
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

// One bf16 row (d values, 16-byte chunks) widened to fp32 into LDS; zeros when src is null.
__device__ __forceinline__ void imp_row_to_lds(float* dst, const uint16_t* src, int cc) {
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (src) raw = *reinterpret_cast<const u32x4*>(src + cc * 8);
  f32x4 lo = {bf16_bits_to_f32(raw[0] & 0xffffu), bf16_bits_to_f32(raw[0] >> 16), bf16_bits_to_f32(raw[1] & 0xffffu),
              bf16_bits_to_f32(raw[1] >> 16)};
  f32x4 hi = {bf16_bits_to_f32(raw[2] & 0xffffu), bf16_bits_to_f32(raw[2] >> 16), bf16_bits_to_f32(raw[3] & 0xffffu),
              bf16_bits_to_f32(raw[3] >> 16)};
  *reinterpret_cast<f32x4*>(dst + cc * 8) = lo;
  *reinterpret_cast<f32x4*>(dst + cc * 8 + 4) = hi;
}

// v_mfma_f64_16x16x4_f64 layouts (lane l): A holds row l%16, k = l/16; B holds column l%16,
// k = l/16; D holds column l%16, rows l/16 + 4 r in its four doubles r = 0..3.
__global__ __launch_bounds__(IMP_THREADS) void imp_scores_kernel(ImpArgs a, double* E, double* part_m,
                                                                 double* part_l) {
  __shared__ __align__(16) float Kt[IMP_CK * IMP_PITCH];
  __shared__ __align__(16) float Qt[IMP_RT * IMP_PITCH];
  __shared__ int qi_s[IMP_RT];
  const int chunk = blockIdx.x, g = blockIdx.y, nchunk = gridDim.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int j0 = chunk * IMP_CK;
  const int cpr = a.d / 8;  // 16-byte chunks per row
  for (int c = t; c < IMP_CK * cpr; c += IMP_THREADS) {
    const int row = c / cpr, j = j0 + row;
    imp_row_to_lds(Kt + row * IMP_PITCH, j < a.N ? a.k + (int64_t)g * a.kvsh + (int64_t)j * a.kvst : nullptr,
                   c % cpr);
  }
  const int ksteps = a.d / 4;
  for (int r0 = 0; r0 < a.R; r0 += IMP_RT) {
    __syncthreads();  // previous Q tile consumed (and K tile written, first time)
    for (int c = t; c < IMP_RT * cpr; c += IMP_THREADS) {
      const int row = c / cpr, r = r0 + row;
      const uint16_t* src = nullptr;
      if (r < a.R) {
        int h, i;
        imp_row(a, g, r, &h, &i);
        src = a.q + (int64_t)h * a.qsh + (int64_t)i * a.qst;
        if (c % cpr == 0) qi_s[row] = i;
      } else if (c % cpr == 0) {
        qi_s[row] = -1;
      }
      imp_row_to_lds(Qt + row * IMP_PITCH, src, c % cpr);
    }
    __syncthreads();
    f64x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f64x4{0.0, 0.0, 0.0, 0.0};
    const float* qa = Qt + (16 * w + l16) * IMP_PITCH + lg;
    const float* kb = Kt + l16 * IMP_PITCH + lg;
    for (int ks = 0; ks < ksteps; ++ks) {
      const double av = (double)qa[ks * 4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const double bv = (double)kb[tt * 16 * IMP_PITCH + ks * 4];
        acc[tt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[tt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int row = 16 * w + lg + 4 * rr;
      const int i = qi_s[row];
      double s[4];
      double m = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int j = j0 + 16 * tt + l16;
        const bool ok = (i >= 0) && (j < a.N) && (j <= i);
        s[tt] = ok ? a.scale * acc[tt][rr] : -INFINITY;
        m = fmax(m, s[tt]);
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, 16));
      double l = 0.0;
      double e[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        e[tt] = (s[tt] > -INFINITY) ? exp(s[tt] - m) : 0.0;
        l += e[tt];
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) l += __shfl_xor(l, o, 16);
      const int r = r0 + row;
      if (r < a.R) {
        double* er = E + ((size_t)g * a.R + r) * a.N;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int j = j0 + 16 * tt + l16;
          if (j < a.N) er[j] = e[tt];
        }
        if (l16 == 0) {
          const size_t o = ((size_t)g * nchunk + chunk) * a.R + r;
          part_m[o] = m;
          part_l[o] = l;
        }
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

// imp_j = (1/R) sum_r e_rj * exp(m_c(j)r - lse_r), rows summed in order.
__global__ __launch_bounds__(COL_KEYS) void imp_colsum_kernel(const double* E, const double* part_m,
                                                              const double* lse, int N, int R, int nchunk,
                                                              double* imp) {
  constexpr int CPB = COL_KEYS / IMP_CK;  // chunks per workgroup
  __shared__ double wsh[CPB][COL_ROWS];
  const int g = blockIdx.y, t = threadIdx.x;
  const int j = blockIdx.x * COL_KEYS + t;
  const int c0 = blockIdx.x * CPB;
  double sum = 0.0;
  for (int rb = 0; rb < R; rb += COL_ROWS) {
    __syncthreads();
    for (int x = t; x < CPB * COL_ROWS; x += COL_KEYS) {
      const int cl = x / COL_ROWS, rr = x % COL_ROWS, r = rb + rr, c = c0 + cl;
      double wv = 0.0;
      if (r < R && c < nchunk) {
        const double mc = part_m[((size_t)g * nchunk + c) * R + r];
        if (mc > -INFINITY) wv = exp(mc - lse[(size_t)g * R + r]);
      }
      wsh[cl][rr] = wv;
    }
    __syncthreads();
    if (j < N) {
      const double* col = E + ((size_t)g * R + rb) * N + j;
      const int nr = min(COL_ROWS, R - rb);
      const double* wc = wsh[t / IMP_CK];
      for (int rr = 0; rr < nr; ++rr) sum = fma(col[(size_t)rr * N], wc[rr], sum);
    }
  }
  if (j < N) imp[(size_t)g * N + j] = sum / (double)R;
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
  imp_scores_kernel<<<dim3(nchunk, g.Hkv), IMP_THREADS, 0, st>>>(a, w.e, w.part_m, w.part_l);
  imp_lse_kernel<<<dim3(a.R, g.Hkv), 256, 0, st>>>(w.part_m, w.part_l, nchunk, a.R, w.lse);
  imp_colsum_kernel<<<dim3((g.N + COL_KEYS - 1) / COL_KEYS, g.Hkv), COL_KEYS, 0, st>>>(w.e, w.part_m, w.lse, g.N,
                                                                                       a.R, nchunk, out);
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
