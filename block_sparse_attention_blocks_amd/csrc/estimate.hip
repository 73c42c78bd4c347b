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

constexpr int IMP_CK = 64;        // keys per chunk (4 MFMA column tiles of 16)
constexpr int IMP_RT = 64;        // proxy rows per workgroup (4 waves x 16 rows)
constexpr int IMP_THREADS = 256;
constexpr int IMP_KR = 16;        // chunks per workgroup
constexpr int COL_KEYS = 256;     // keys per workgroup of imp_colsum
constexpr int COL_ROWS = 256;     // rows staged per pass of imp_colsum

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

struct ImpWs {
  double* e;       // [Hkv][R][N] chunk-normalised exponentials
  double* part_m;  // [Hkv][nchunk][R]
  double* part_l;  // [Hkv][nchunk][R]
  double* lse;     // [Hkv][R]
  double* imp;     // [Hkv][N] (used when the caller passes no importance output)
};

static inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workgroup barrier that waits for this wave's LDS operations only (__syncthreads() would also wait
// for every outstanding global store).
__device__ __forceinline__ void lds_barrier_est() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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
  int trunk_c;    // 0: proxy rows are the last R1 positions; > 0: trunk-sampled rows (chunk length)
  int rpt;        // trunk sampling: rows per trunk
  int first_row;  // smallest proxy position (every key j <= first_row is visible to every proxy row)
};

// Proxy row r of KV head g -> (query head, token position): the last R1 positions, or with trunk
// sampling the last rpt positions of every trunk of trunk_c positions.
__device__ __forceinline__ void imp_row(const ImpArgs& a, int g, int r, int* h, int* i) {
  *h = g * a.G + r / a.R1;
  const int r1 = r % a.R1;
  if (a.trunk_c > 0) {
    const int t = r1 / a.rpt;
    *i = min((t + 1) * a.trunk_c, a.N) - a.rpt + r1 % a.rpt;
  } else {
    *i = a.N - a.R1 + r1;
  }
}

// DPP row rotation of a double (16-lane rows): all-reduce helpers for the 16 lanes of one row.
template <int N>
__device__ __forceinline__ double row_ror_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x120 + N, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x120 + N, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double row_max_f64(double x) {
  x = fmax(x, row_ror_f64<1>(x));
  x = fmax(x, row_ror_f64<2>(x));
  x = fmax(x, row_ror_f64<4>(x));
  return fmax(x, row_ror_f64<8>(x));
}
__device__ __forceinline__ double row_sum_f64(double x) {  // exact on lane 0 of the row's order
  x += row_ror_f64<1>(x);
  x += row_ror_f64<2>(x);
  x += row_ror_f64<4>(x);
  return x + row_ror_f64<8>(x);
}


// exp(x) for the logits of the importance pass (x <= 0, -inf allowed), written out in fp64:
// Cody-Waite reduction x = n ln2 + r with |r| <= ln2/2 (ln2 split into a 32-significant-bit head,
// so n * head is exact, and the rounded remainder), exp(r) by its Taylor series to degree 11
// (truncation below 1e-14 relative on that interval; 8.8e-15 worst case measured against the math
// library on [-60, 0]), then the exact scaling by 2^n.  Below -745 the result is 0.
__device__ __forceinline__ double exp_nonpos(double x) {
  constexpr double kLog2e = 1.4426950408889634, kLn2Hi = 0.6931471803691238, kLn2Lo = 1.9082149292705877e-10;
  const double n = rint(x * kLog2e);
  double r = fma(-n, kLn2Hi, x);
  r = fma(-n, kLn2Lo, r);
  double q = 2.505210838544172e-08;  // 1/11!
  q = fma(q, r, 2.755731922398589e-07);
  q = fma(q, r, 2.7557319223985893e-06);
  q = fma(q, r, 2.48015873015873e-05);
  q = fma(q, r, 0.0001984126984126984);
  q = fma(q, r, 0.001388888888888889);
  q = fma(q, r, 0.008333333333333333);
  q = fma(q, r, 0.041666666666666664);
  q = fma(q, r, 0.16666666666666666);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  q = fma(q, r, 1.0);
  const double y = ldexp(q, (int)n);
  return x < -745.0 ? 0.0 : y;
}

// v_mfma_f64_16x16x4_f64 (lane l): A holds row l%16 and B column l%16 at contraction slot l/16; D
// holds column l%16, rows l/16 + 4 r in its four doubles r = 0..3.  The contraction index of lane
// group lg at MFMA step ks is k = 4 ks + lg.  Each wave keeps its 16 proxy rows (all of d) in
// registers as doubles; every key chunk is widened to doubles once, by the staging threads, into
// LDS rows padded to D + 4 doubles, so a B operand is one 8-byte read at a fixed offset from the
// lane's base address and the 64 lanes of a read fall on distinct bank pairs two at a time.  The
// next chunk's bf16 rows are loaded into registers while the current one is multiplied.
template <int D>
__global__ __launch_bounds__(IMP_THREADS) void imp_scores_kernel(ImpArgs a, double* E, double* part_m,
                                                                 double* part_l) {
  constexpr int KS = D / 4;         // MFMA k-steps
  constexpr int PITCH = D + 4;      // doubles per staged key row
  constexpr int cpr = D / 8;        // 16-byte bf16 chunks per key row
  constexpr int NLD = IMP_CK * cpr / IMP_THREADS;  // chunks per thread per stage
  __shared__ __align__(16) double Kf[IMP_CK * PITCH];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int r0 = blockIdx.x * IMP_RT, g = blockIdx.z;
  const int nchunk = (a.N + IMP_CK - 1) / IMP_CK;
  const int c0 = blockIdx.y * IMP_KR, c1 = min(c0 + IMP_KR, nchunk);
  const uint16_t* kbase = a.k + (int64_t)g * a.kvsh;

  // A operand: proxy row r0 + 16 w + l16, slots k = 4 ks + lg
  const int ra = r0 + 16 * w + l16;
  double av[KS];
  {
    const uint16_t* src = nullptr;
    if (ra < a.R) {
      int h, i;
      imp_row(a, g, ra, &h, &i);
      src = a.q + (int64_t)h * a.qsh + (int64_t)i * a.qst;
    }
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {  // 32 elements (8 k-steps) at a time
      u32x4 raw[4] = {};
      if (src)
#pragma unroll
        for (int c = 0; c < 4; ++c) raw[c] = *reinterpret_cast<const u32x4*>(src + 32 * p + 8 * c);
#pragma unroll
      for (int kl = 0; kl < 8; ++kl) {
        // element 4 kl + lg of these 32: 16-byte chunk kl / 2, word 2 (kl % 2) + lg / 2, half lg % 2
        const u32x4 v = raw[kl >> 1];
        const uint32_t wd = (lg >> 1) ? v[2 * (kl & 1) + 1] : v[2 * (kl & 1)];
        av[8 * p + kl] = (double)bf16_bits_to_f32((lg & 1) ? (wd >> 16) : (wd & 0xffffu));
      }
    }
  }
  // this lane's D rows (proxy rows r0 + 16 w + lg + 4 rr) and their query positions
  int qi[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = r0 + 16 * w + lg + 4 * rr;
    int h, i;
    imp_row(a, g, r, &h, &i);
    qi[rr] = r < a.R ? i : -1;
  }
  const int first_proxy = a.first_row;  // every key j <= first_proxy is visible to every proxy row

  auto prefetch = [&](int c, u32x4* pf) {
    const int j0 = c * IMP_CK;
#pragma unroll
    for (int x = 0; x < NLD; ++x) {
      const int idx = t + x * IMP_THREADS;
      const int row = idx / cpr, ch = idx % cpr;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (j0 + row < a.N) v = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(j0 + row) * a.kvst + ch * 8);
      pf[x] = v;
    }
  };
  // widen the prefetched bf16 rows to doubles into the padded LDS rows
  auto stage = [&](const u32x4* pf) {
#pragma unroll
    for (int x = 0; x < NLD; ++x) {
      const int idx = t + x * IMP_THREADS;
      const int row = idx / cpr, ch = idx % cpr;
      double* dst = Kf + row * PITCH + ch * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t wd = pf[x][e];
        const f64x2 two = {(double)bf16_bits_to_f32(wd & 0xffffu), (double)bf16_bits_to_f32(wd >> 16)};
        *reinterpret_cast<f64x2*>(dst + 2 * e) = two;
      }
    }
  };
  const double* bbase = Kf + l16 * PITCH + lg;  // B operand of column tile tt, step ks: bbase[16 tt PITCH + 4 ks]

  u32x4 pf[NLD];
  prefetch(c0, pf);
  for (int c = c0; c < c1; ++c) {
    stage(pf);
    __syncthreads();
    if (c + 1 < c1) prefetch(c + 1, pf);
    f64x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], bbase[16 * tt * PITCH + 4 * ks], acc[tt], 0, 0, 0);
    // per proxy row: chunk max, sum of exponentials, and the exponentials themselves
    const int j0 = c * IMP_CK;
    const bool open = j0 + IMP_CK - 1 <= first_proxy && j0 + IMP_CK <= a.N;  // no key of the chunk is masked
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      double sv[4];
      double m;
      if (open) {
        double mx = fmax(fmax(acc[0][rr], acc[1][rr]), fmax(acc[2][rr], acc[3][rr]));
        m = a.scale * row_max_f64(mx);  // scale > 0 keeps the max
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sv[tt] = exp_nonpos(fma(a.scale, acc[tt][rr], -m));
      } else {
        const int i = qi[rr];
        m = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int j = j0 + 16 * tt + l16;
          const bool ok = (i >= 0) && (j < a.N) && (j <= i);
          sv[tt] = ok ? a.scale * acc[tt][rr] : -INFINITY;
          m = fmax(m, sv[tt]);
        }
        m = row_max_f64(m);
        const double mm = m > -INFINITY ? m : 0.0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sv[tt] = exp_nonpos(sv[tt] - mm);
      }
      double l = (sv[0] + sv[1]) + (sv[2] + sv[3]);
      l = row_sum_f64(l);
      const int r = r0 + 16 * w + lg + 4 * rr;
      if (r < a.R) {
        double* er = E + ((size_t)g * a.R + r) * a.N;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int j = j0 + 16 * tt + l16;
          if (j < a.N) er[j] = sv[tt];
        }
        if (l16 == 0) {
          const size_t o = ((size_t)g * nchunk + c) * a.R + r;
          part_m[o] = m;
          part_l[o] = l;
        }
      }
    }
    __syncthreads();  // every wave is done with this chunk's rows before they are replaced
  }
}

// lse_r = M + log sum_c l_cr exp(m_cr - M) for 8 proxy rows per workgroup: thread t takes row
// r0 + t % 8 and every 32nd chunk from t / 8, so one load instruction reads 8 consecutive rows of
// 32 chunks; four chunks are loaded before any is used.
constexpr int LSE_ROWS = 8, LSE_CG = 32;
__global__ __launch_bounds__(256) void imp_lse_kernel(const double* part_m, const double* part_l, int nchunk,
                                                      int R, double* lse) {
  __shared__ double sm[LSE_CG][LSE_ROWS], sl[LSE_CG][LSE_ROWS];
  const int t = threadIdx.x, rl = t % LSE_ROWS, cg = t / LSE_ROWS;
  const int r = blockIdx.x * LSE_ROWS + rl, g = blockIdx.y;
  const bool ok = r < R;
  const double* pm = part_m + (size_t)g * nchunk * R + r;
  const double* pl = part_l + (size_t)g * nchunk * R + r;
  constexpr int U = 4;
  double m = -INFINITY;
  if (ok)
    for (int c0 = cg; c0 < nchunk; c0 += U * LSE_CG) {
      double x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * LSE_CG;
        x[u] = c < nchunk ? pm[(size_t)c * R] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) m = fmax(m, x[u]);
    }
  sm[cg][rl] = m;
  __syncthreads();
  m = -INFINITY;
#pragma unroll 8
  for (int k = 0; k < LSE_CG; ++k) m = fmax(m, sm[k][rl]);
  double l = 0.0;
  if (ok)
    for (int c0 = cg; c0 < nchunk; c0 += U * LSE_CG) {
      double x[U], y[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * LSE_CG;
        x[u] = c < nchunk ? pm[(size_t)c * R] : -INFINITY;
        y[u] = c < nchunk ? pl[(size_t)c * R] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (x[u] > -INFINITY) l += y[u] * exp(x[u] - m);
    }
  sl[cg][rl] = l;
  __syncthreads();
  if (cg == 0 && ok) {
    double tot = 0.0;
    for (int k = 0; k < LSE_CG; ++k) tot += sl[k][rl];
    lse[(size_t)g * R + r] = m + log(tot);
  }
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
  a.trunk_c = 0;
  a.rpt = 0;
  a.first_row = g.N - a.R1;
  const int nchunk = imp_chunks(g);
  const dim3 grid((a.R + IMP_RT - 1) / IMP_RT, (nchunk + IMP_KR - 1) / IMP_KR, g.Hkv);
  if (g.d == 128) {
    imp_scores_kernel<128><<<grid, IMP_THREADS, 0, st>>>(a, w.e, w.part_m, w.part_l);
  } else {
    imp_scores_kernel<64><<<grid, IMP_THREADS, 0, st>>>(a, w.e, w.part_m, w.part_l);
  }
  imp_lse_kernel<<<dim3((a.R + LSE_ROWS - 1) / LSE_ROWS, g.Hkv), 256, 0, st>>>(w.part_m, w.part_l, nchunk, a.R,
                                                                                 w.lse);
  imp_colsum_kernel<<<dim3((g.N + COL_KEYS - 1) / COL_KEYS, g.Hkv), COL_KEYS, 0, st>>>(w.e, w.part_m, w.lse, g.N,
                                                                                       a.R, nchunk, out);
  return hipGetLastError();
}

// =====================================================================================
// Stage 1b: sort inside segments (section 3, "Sorting"): importance descending, ties by
// position ascending.  One workgroup per (segment, KV head); bitonic sort in LDS on a 64-bit key
// that orders like the negated value (sign-folded bit pattern), with the position as the second
// key.  The same sort orders S2O's query guide scores, which may be negative.
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
      const uint64_t b = (uint64_t)__double_as_longlong(imp[(size_t)g * N + a + x]);
      const uint64_t o = (b >> 63) ? ~b : (b | 0x8000000000000000ull);  // ascending in the value
      key[x] = ~o;
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

// Exact causal softmax rows of trunk-sampled queries (SampleAttention, stage 1): the importance
// kernels with the trunk row map; per KV head its G * n_trunks * rpt rows, head-major.
size_t sampled_softmax_workspace_bytes(const Geometry& g, int n_trunks, int rpt) {
  const size_t R = (size_t)g.G * n_trunks * rpt, C = imp_chunks(g);
  return align256(sizeof(double) * g.Hkv * R * (size_t)g.N) + 2 * align256(sizeof(double) * g.Hkv * C * R) +
         align256(sizeof(double) * g.Hkv * R);
}

hipError_t launch_sampled_softmax(const Geometry& g, const uint16_t* q, const uint16_t* k, int n_trunks, int rpt,
                                  void* ws, SampledRows* out, hipStream_t st) {
  const int R = g.G * n_trunks * rpt, nchunk = imp_chunks(g);
  char* p = static_cast<char*>(ws);
  out->e = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)R * g.N);
  out->part_m = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)nchunk * R);
  double* part_l = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)nchunk * R);
  out->lse = reinterpret_cast<double*>(p);
  out->R = R;
  out->nchunk = nchunk;
  ImpArgs a;
  a.q = q;
  a.k = k;
  a.N = g.N;
  a.G = g.G;
  a.d = g.d;
  a.R1 = n_trunks * rpt;
  a.R = R;
  a.qsh = g.qsh;
  a.qst = g.qst;
  a.kvsh = g.kvsh;
  a.kvst = g.kvst;
  a.scale = g.scale64;
  a.trunk_c = (g.N + n_trunks - 1) / n_trunks;
  a.rpt = rpt;
  a.first_row = min(a.trunk_c, g.N) - rpt;
  const dim3 grid((R + IMP_RT - 1) / IMP_RT, (nchunk + IMP_KR - 1) / IMP_KR, g.Hkv);
  if (g.d == 128) {
    imp_scores_kernel<128><<<grid, IMP_THREADS, 0, st>>>(a, out->e, out->part_m, part_l);
  } else {
    imp_scores_kernel<64><<<grid, IMP_THREADS, 0, st>>>(a, out->e, out->part_m, part_l);
  }
  imp_lse_kernel<<<dim3((R + LSE_ROWS - 1) / LSE_ROWS, g.Hkv), 256, 0, st>>>(out->part_m, part_l, nchunk, R,
                                                                             out->lse);
  return hipGetLastError();
}

hipError_t launch_segment_sort(const Geometry& g, const double* score, int32_t* perm, hipStream_t st) {
  const int nseg = (g.N + g.S - 1) / g.S;
  segment_sort_kernel<<<dim3(nseg, g.Hkv), SORT_THREADS, 0, st>>>(score, perm, g.N, g.S);
  return hipGetLastError();
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
// Stage 2b: pooled block logits (section 4, Block Selection).  z[h][I][J] = c * Qbar[h][I] . Kbar_J
// for J <= I, Kbar_J the permuted pooled key when J's segment precedes I's, else the natural one.
// One workgroup per (tile of TI consecutive query blocks inside one segment, group of up to 16
// query heads of one KV head): its 16 pooled queries (TI rows x HC heads) form the A operand of
// v_mfma_f64_16x16x4_f64, held in registers; each wave walks 16-key-block tiles of Kbar as the B
// operand, so every pooled key row read serves 16 logits.
// =====================================================================================

constexpr int ZL_THREADS = 256;

struct ZArgs {
  const double* qbar;   // [Hq][NB][d]
  const double* knat;   // [Hkv][NB][d]
  const double* kperm;  // [Hkv][NB][d] or NULL
  int NB, G, d, B, S;
  int HC, TI;           // heads per workgroup, query blocks per workgroup (HC * TI <= 16)
  int nhc;              // head groups per KV head
  double scale;
  double* z;            // [Hq][NB(NB+1)/2]
};

template <int D>
__global__ __launch_bounds__(ZL_THREADS) void block_logits_kernel(ZArgs a) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = blockIdx.y / a.nhc, hc = blockIdx.y % a.nhc;
  const int I0 = blockIdx.x * a.TI;
  const int nq = a.HC * a.TI;
  // A operand row q = l16: head g*G + hc*HC + q / TI, query block I0 + q % TI
  const int qh = g * a.G + hc * a.HC + l16 / a.TI;
  const int qI = I0 + l16 % a.TI;
  const bool qok = l16 < nq && qI < a.NB && hc * a.HC + l16 / a.TI < a.G;
  const double* qrow = a.qbar + ((size_t)qh * a.NB + qI) * D;
  const int Imax = min(I0 + a.TI, a.NB) - 1;
  const int sI = a.S > 0 ? (I0 * a.B) / a.S : 0;
  // contraction slot of lane group lg at MFMA step ks: k = lg * ksteps + ks, so every lane reads a
  // contiguous run of its row (16-byte loads)
  constexpr int ksteps = D / 4;
  double av[ksteps];  // A operand for every k-step
#pragma unroll
  for (int ks = 0; ks < ksteps; ks += 2) {
    f64x2 x = {0.0, 0.0};
    if (qok) x = *reinterpret_cast<const f64x2*>(qrow + lg * ksteps + ks);
    av[ks] = x[0];
    av[ks + 1] = x[1];
  }
  const size_t ntri = (size_t)a.NB * (a.NB + 1) / 2;
  for (int J0 = 16 * w; J0 <= Imax; J0 += 16 * (ZL_THREADS / 64)) {
    const int J = J0 + l16;
    const bool jok = J <= Imax;
    const bool permuted = a.kperm != nullptr && a.S > 0 && (J * a.B) / a.S < sI;
    // (columns past Imax read row 0, a valid row, and are never stored)
    const double* krow = (permuted ? a.kperm : a.knat) + ((size_t)g * a.NB + (jok ? J : 0)) * D;
    double bv[ksteps];  // all loads issued before the first MFMA waits on one
#pragma unroll
    for (int ks = 0; ks < ksteps; ks += 2) {
      const f64x2 x = *reinterpret_cast<const f64x2*>(krow + lg * ksteps + ks);
      bv[ks] = x[0];
      bv[ks + 1] = x[1];
    }
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int ks = 0; ks < ksteps; ++ks) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[ks], bv[ks], acc, 0, 0, 0);
    // D: column J (lane l16), rows q = lg + 4 r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = lg + 4 * r;
      const int h = g * a.G + hc * a.HC + q / a.TI;
      const int I = I0 + q % a.TI;
      if (q < nq && hc * a.HC + q / a.TI < a.G && I < a.NB && J <= I)
        a.z[(size_t)h * ntri + (size_t)tri_offset(I) + J] = a.scale * acc[r];
    }
  }
}

// =====================================================================================
// Stage 2c: block selection (section 4 with SampleAttention's cumulative-mass rule).  One wave per
// (query head h, query block I): p = softmax(z) over J <= I in fp64; the kept set is the shortest
// prefix of the order (p descending, J ascending) whose mass reaches tau.  Instead of sorting, the
// wave finds the p value t* at which that prefix ends by bisection on the bit pattern of p (for
// p >= 0 it orders like the value): t* is the largest value with mass(p >= t*) >= tau.  Every J with
// p > t* is kept, and of the J with p == t* the smallest ones, as many as the mass still needs.
// Then the forced blocks are added and the kept set is written in ascending J.
// =====================================================================================

constexpr int SEL_WAVES = 4;

// Wave-wide fp64 sum / max through DPP row shifts and row broadcasts (no LDS round trips): an
// inclusive scan inside each 16-lane row, then the row totals are carried across rows; lane 63 ends
// with the result, which is read back as a scalar so every lane takes the same decision.
__device__ __forceinline__ double dpp_f64(double x, int ctrl_kind) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
  switch (ctrl_kind) {  // dpp_ctrl, row_mask, bank_mask, bound_ctrl (reads past a row give 0)
    case 1: lo = __builtin_amdgcn_update_dpp(0, lo, 0x111, 0xf, 0xf, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x111, 0xf, 0xf, true); break;
    case 2: lo = __builtin_amdgcn_update_dpp(0, lo, 0x112, 0xf, 0xf, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x112, 0xf, 0xf, true); break;
    case 4: lo = __builtin_amdgcn_update_dpp(0, lo, 0x114, 0xf, 0xf, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x114, 0xf, 0xf, true); break;
    case 8: lo = __builtin_amdgcn_update_dpp(0, lo, 0x118, 0xf, 0xf, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x118, 0xf, 0xf, true); break;
    case 15: lo = __builtin_amdgcn_update_dpp(0, lo, 0x142, 0xa, 0xf, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x142, 0xa, 0xf, false); break;
    default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x143, 0xc, 0xf, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x143, 0xc, 0xf, false); break;
  }
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

__device__ __forceinline__ double wave_total_f64(double x) {
  x += dpp_f64(x, 1);
  x += dpp_f64(x, 2);
  x += dpp_f64(x, 4);
  x += dpp_f64(x, 8);
  x += dpp_f64(x, 15);
  x += dpp_f64(x, 31);
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)b, 63), hi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

struct SelArgs {
  const double* z;  // [Hq][NB(NB+1)/2]
  int NB, Hq;
  double tau;
  uint32_t flags;
  int32_t* count;
  int32_t* idx;
  double* prob;
};

template <int SEL_PL>  // values per lane: 64 * SEL_PL >= NB
__global__ __launch_bounds__(SEL_WAVES * 64) void block_select_kernel(SelArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * SEL_WAVES + w;
  if (row >= a.Hq * a.NB) return;
  const int h = row / a.NB, I = a.NB - 1 - row % a.NB;  // long rows first
  const int nJ = I + 1;
  const int npl = (nJ + 63) / 64;
  const size_t tri = (size_t)h * ((size_t)a.NB * (a.NB + 1) / 2) + (size_t)tri_offset(I);
  double v[SEL_PL];
  double m = -INFINITY;
#pragma unroll
  for (int i = 0; i < SEL_PL; ++i) {
    const int J = lane + 64 * i;
    v[i] = (i < npl && J < nJ) ? a.z[tri + J] : -INFINITY;
    m = fmax(m, v[i]);
  }
  m = wave_max_f64(m);
  double se = 0.0;
#pragma unroll
  for (int i = 0; i < SEL_PL; ++i) {
    if (i < npl) {
      v[i] = (v[i] > -INFINITY) ? exp(v[i] - m) : 0.0;
      se += v[i];
    }
  }
  se = wave_sum_f64(se);
#pragma unroll
  for (int i = 0; i < SEL_PL; ++i) {
    if (i < npl) {
      v[i] = v[i] / se;
      const int J = lane + 64 * i;
      if (a.prob && J < nJ) a.prob[tri + J] = v[i];
    }
  }
  // mass of the values whose bit pattern is >= t (wave-uniform: butterfly sums agree on every lane)
  auto mass_ge = [&](uint64_t thr) {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < SEL_PL; ++i)
      if (i < npl && (uint64_t)__double_as_longlong(v[i]) >= thr) s += v[i];
    return wave_total_f64(s);
  };
  uint64_t tstar = 0;     // keep every J (tau >= 1, or the mass never reaches tau)
  bool all = true;
  int ntie_keep = 0;      // J with p == t* that are kept, smallest J first
  if (a.tau < 1.0 && mass_ge(0) >= a.tau) {
    all = false;
    for (int bit = 62; bit >= 0; --bit) {
      const uint64_t cand = tstar | (1ull << bit);
      if (mass_ge(cand) >= a.tau) tstar = cand;
    }
    // mass strictly above t*, and how many of the tied values it still needs (at most all of them,
    // whatever the rounding of the running sum)
    double above = 0.0;
    int ntied = 0;
#pragma unroll
    for (int i = 0; i < SEL_PL; ++i) {
      if (i < npl) {
        const uint64_t key = (uint64_t)__double_as_longlong(v[i]);
        if (key > tstar) above += v[i];
        if (key == tstar && lane + 64 * i < nJ) ++ntied;
      }
    }
    above = wave_total_f64(above);
    ntied = (int)wave_total_f64((double)ntied);
    const double pt = __longlong_as_double((long long)tstar);
    double c = above;
    do {
      c += pt;
      ++ntie_keep;
    } while (c < a.tau && ntie_keep < ntied);
  }
  // kept flags, then ascending compaction
  int base = 0, tie_seen = 0;
  for (int i = 0; i < npl; ++i) {
    const int J = lane + 64 * i;
    const uint64_t key = (uint64_t)__double_as_longlong(v[i]);
    bool keep = false;
    if (J < nJ) {
      if (all || key > tstar) keep = true;
      if ((a.flags & 1u) && J == I) keep = true;
      if ((a.flags & 2u) && J == 0) keep = true;
    }
    const bool tie = !all && J < nJ && key == tstar;
    const unsigned long long tb = __ballot(tie);
    if (tie && tie_seen + __popcll(tb & ((1ull << lane) - 1ull)) < ntie_keep) keep = true;
    tie_seen += __popcll(tb);
    const unsigned long long kb = __ballot(keep);
    if (keep) a.idx[tri + base + __popcll(kb & ((1ull << lane) - 1ull))] = J;
    base += __popcll(kb);
  }
  if (lane == 0) a.count[(size_t)h * a.NB + I] = base;
}

size_t mask_workspace_bytes(const Geometry& g) {
  const size_t NB = g.NB;
  return align256(sizeof(double) * g.Hq * NB * g.d) + 2 * align256(sizeof(double) * g.Hkv * NB * g.d) +
         align256(sizeof(double) * g.Hq * (NB * (NB + 1) / 2));
}

// =====================================================================================
// Ranked block order of the marginal-gain early stop (S2O, Early-Stopping Rule: blocks are visited
// in descending estimated importance; Kernel Implementation: the dense window of the query's own
// segment first).  Row (h, I) lists every J <= I: the blocks of I's segment ascending, then the
// earlier-segment blocks by pooled logit z descending, ties by J ascending.  One workgroup per row:
// a bitonic sort in LDS on (order-preserving 64-bit key of -z, J).
// =====================================================================================
constexpr int RANK_THREADS = 256;
constexpr int RANK_MAX = 2048;

__device__ __forceinline__ uint64_t desc_key(double x) {  // ascending in this key = descending in x
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t o = (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
  return ~o;
}

__global__ __launch_bounds__(RANK_THREADS) void block_rank_kernel(const double* z, int NB, int bps, int32_t* count,
                                                                  int32_t* idx) {
  __shared__ uint64_t key[RANK_MAX];
  __shared__ uint16_t jj[RANK_MAX];
  const int t = threadIdx.x;
  const int row = blockIdx.x, h = row / NB, I = row % NB;
  const int J0 = (I / bps) * bps;  // first block of I's segment; J < J0 are the earlier segments
  const size_t ntri = (size_t)NB * (NB + 1) / 2;
  const double* zr = z + (size_t)h * ntri + (size_t)tri_offset(I);
  int n = 1;
  while (n < J0) n <<= 1;
  for (int x = t; x < n; x += RANK_THREADS) {
    const bool live = x < J0;
    key[x] = live ? desc_key(zr[x]) : ~0ull;
    jj[x] = live ? (uint16_t)x : (uint16_t)0xffffu;
  }
  __syncthreads();
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = t; x < n / 2; x += RANK_THREADS) {
        const int lo = 2 * x - (x & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t ka = key[lo], kb = key[hi];
        const uint16_t ja = jj[lo], jb = jj[hi];
        const bool a_after_b = (ka > kb) || (ka == kb && ja > jb);
        if (a_after_b == up) {
          key[lo] = kb;
          key[hi] = ka;
          jj[lo] = jb;
          jj[hi] = ja;
        }
      }
      __syncthreads();
    }
  }
  int32_t* out = idx + (size_t)h * ntri + (size_t)tri_offset(I);
  const int nin = I + 1 - J0;
  for (int x = t; x < nin; x += RANK_THREADS) out[x] = J0 + x;
  for (int x = t; x < J0; x += RANK_THREADS) out[nin + x] = jj[x];
  if (t == 0) count[row] = I + 1;
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
  p += align256(sizeof(double) * g.Hkv * (size_t)g.NB * g.d);
  double* z = reinterpret_cast<double*>(p);
  pool_kernel<<<dim3(g.NB, g.Hq), POOL_THREADS, 0, st>>>(q, g.qsh, g.qst, g.N, g.B, g.d, nullptr, qbar, g.NB);
  pool_kernel<<<dim3(g.NB, g.Hkv), POOL_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.B, g.d, nullptr, knat, g.NB);
  if (perm)
    pool_kernel<<<dim3(g.NB, g.Hkv), POOL_THREADS, 0, st>>>(k, g.kvsh, g.kvst, g.N, g.B, g.d, perm, kperm, g.NB);
  ZArgs za;
  za.qbar = qbar;
  za.knat = knat;
  za.kperm = perm ? kperm : nullptr;
  za.NB = g.NB;
  za.G = g.G;
  za.d = g.d;
  za.B = g.B;
  za.S = g.S;
  za.HC = g.G < 16 ? g.G : 16;
  za.nhc = (g.G + za.HC - 1) / za.HC;
  // query blocks per workgroup: as many as fit 16 rows, never crossing a segment boundary
  const int bps = g.S > 0 ? g.S / g.B : 0;
  int ti = 16 / za.HC;
  while (ti > 1 && bps > 0 && bps % ti != 0) ti >>= 1;
  za.TI = ti < 1 ? 1 : ti;
  za.scale = g.scale64;
  za.z = z;
  const dim3 zgrid((g.NB + za.TI - 1) / za.TI, g.Hkv * za.nhc);
  if (g.d == 128) {
    block_logits_kernel<128><<<zgrid, ZL_THREADS, 0, st>>>(za);
  } else {
    block_logits_kernel<64><<<zgrid, ZL_THREADS, 0, st>>>(za);
  }
  if (flags & kMaskRanked) {
    block_rank_kernel<<<g.Hq * g.NB, RANK_THREADS, 0, st>>>(z, g.NB, g.S / g.B, count, idx);
    return hipGetLastError();
  }
  SelArgs a;
  a.z = z;
  a.NB = g.NB;
  a.Hq = g.Hq;
  a.tau = tau;
  a.flags = flags;
  a.count = count;
  a.idx = idx;
  a.prob = prob;
  const int rows = g.Hq * g.NB;
  const int grid = (rows + SEL_WAVES - 1) / SEL_WAVES;
  if (g.NB <= 64) {
    block_select_kernel<1><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  } else if (g.NB <= 128) {
    block_select_kernel<2><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  } else if (g.NB <= 256) {
    block_select_kernel<4><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  } else if (g.NB <= 512) {
    block_select_kernel<8><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  } else if (g.NB <= 1024) {
    block_select_kernel<16><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  } else {
    block_select_kernel<32><<<grid, SEL_WAVES * 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace pbsa
