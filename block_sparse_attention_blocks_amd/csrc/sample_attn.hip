// SampleAttention's block mask (Technical Deep Dive): stage 1 trunk sampling, stage 2 score-based
// filtering with decoupled filtering of key columns and slashes to a CIA mass target.
//   launch_sampled_softmax   exact causal softmax rows of the sampled queries (importance kernels)
//   sa_weight_kernel         exp(chunk max - row lse), the factor that turns the stored chunk
//                            exponentials into probabilities
//   sa_col_kernel            col[h][j]     = mean over the head's sampled rows of p_ij
//   sa_slash_kernel          slash[h][dlt] = mean over the head's sampled rows of p_{i, i-dlt}
//   sa_cut_kernel            per head and family: the shortest heaviest set reaching the target
//   sa_block_kernel          per head: kept columns per key block, prefix counts of kept slashes
//   sa_mask_kernel           per (h, I): tiles with a kept column, crossed by a kept slash, or forced
#include "estimate.h"

namespace pbsa {
namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int SA_THREADS = 256;
constexpr int CUT_THREADS = 1024;
constexpr int SA_CK = 64;  // key chunk of the stored exponentials

struct SaWs {
  double* w;         // [Hkv][nchunk][R]
  double* col;       // [Hq][N] (when the caller passes none)
  double* slash;     // [Hq][N]
  uint8_t* keep;     // [2][Hq][N]: kept columns, then kept slashes
  uint8_t* colblk;   // [Hq][NB]
  int32_t* spre;     // [Hq][N + 1] prefix counts of kept slashes
  char* softmax_ws;  // the sampled-rows workspace
};

SaWs carve(const Geometry& g, int n_trunks, int rpt, void* ws) {
  const int R = g.G * n_trunks * rpt, nchunk = (g.N + SA_CK - 1) / SA_CK;
  char* c = static_cast<char*>(ws);
  SaWs w;
  w.w = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hkv * (size_t)nchunk * R);
  w.col = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hq * (size_t)g.N);
  w.slash = reinterpret_cast<double*>(c);
  c += align256(sizeof(double) * g.Hq * (size_t)g.N);
  w.keep = reinterpret_cast<uint8_t*>(c);
  c += align256(2 * (size_t)g.Hq * g.N);
  w.colblk = reinterpret_cast<uint8_t*>(c);
  c += align256((size_t)g.Hq * g.NB);
  w.spre = reinterpret_cast<int32_t*>(c);
  c += align256(sizeof(int32_t) * g.Hq * ((size_t)g.N + 1));
  w.softmax_ws = c;
  return w;
}

__global__ __launch_bounds__(SA_THREADS) void sa_weight_kernel(const double* part_m, const double* lse, int nchunk,
                                                               int R, int64_t n, double* w) {
  const int64_t x = (int64_t)blockIdx.x * SA_THREADS + threadIdx.x;
  if (x >= n) return;
  const int64_t per_head = (int64_t)nchunk * R;
  const int g = (int)(x / per_head), r = (int)(x % R);
  const double m = part_m[x];
  w[x] = m > -INFINITY ? exp(m - lse[(size_t)g * R + r]) : 0.0;
}

// Position of sampled row u (0 .. n_trunks*rpt-1): the last rpt positions of trunk u / rpt.
__device__ __forceinline__ int trunk_pos(int u, int rpt, int C, int N) {
  return min((u / rpt + 1) * C, N) - rpt + u % rpt;
}

struct MassArgs {
  const float* e;  // exponentials stored in fp32 (each within 2^-24 relative)
  const double* w;
  int N, G, R, R1, nchunk, rpt, C;
};

// col[h][j]: the head's R1 rows summed in row order (one fma per row), then / R1.
__global__ __launch_bounds__(SA_THREADS) void sa_col_kernel(MassArgs a, double* col) {
  const int j = blockIdx.x * SA_THREADS + threadIdx.x, h = blockIdx.y;
  if (j >= a.N) return;
  const int g = h / a.G, r0 = (h % a.G) * a.R1;
  const float* e = a.e + ((size_t)g * a.R + r0) * a.N + j;
  const double* w = a.w + ((size_t)g * a.nchunk + j / SA_CK) * a.R + r0;
  double s = 0.0;
  for (int u = 0; u < a.R1; ++u) s = fma((double)e[(size_t)u * a.N], w[u], s);
  col[(size_t)h * a.N + j] = s / (double)a.R1;
}

// slash[h][dlt]: p_{i, i - dlt} of the head's rows with i >= dlt, in row order, then / R1.
__global__ __launch_bounds__(SA_THREADS) void sa_slash_kernel(MassArgs a, double* slash) {
  const int dlt = blockIdx.x * SA_THREADS + threadIdx.x, h = blockIdx.y;
  if (dlt >= a.N) return;
  const int g = h / a.G, r0 = (h % a.G) * a.R1;
  double s = 0.0;
  for (int u = 0; u < a.R1; ++u) {
    const int i = trunk_pos(u, a.rpt, a.C, a.N);
    if (i < dlt) continue;
    const int j = i - dlt;
    const size_t r = (size_t)g * a.R + r0 + u;
    s = fma((double)a.e[r * a.N + j], a.w[((size_t)g * a.nchunk + j / SA_CK) * a.R + r0 + u], s);
  }
  slash[(size_t)h * a.N + dlt] = s / (double)a.R1;
}

__device__ __forceinline__ int block_exclusive_count(int x, int* wcnt, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  __syncthreads();
  if (lane == 63) wcnt[wave] = inc;
  __syncthreads();
  int base = inc - x, tot = 0;
  for (int v = 0; v < CUT_THREADS / 64; ++v) {
    if (v < wave) base += wcnt[v];
    tot += wcnt[v];
  }
  *total = tot;
  return base;
}

// The mass cut of one head and family (blockIdx.y: 0 columns, 1 slashes): the kept set is the
// shortest prefix of the order (mass descending, index ascending) whose sum reaches tau.  With
// S(t) = sum of the masses >= t (a fixed-order workgroup sum), the cut value t* = max{t : S(t) >=
// tau} is searched over the bit patterns of non-negative doubles (which order like the values),
// CUT_WAYS-ary: each pass evaluates S at CUT_WAYS evenly spaced patterns inside the current bracket and
// keeps the sub-bracket where S crosses tau.  Masses > t* are kept, and of those equal to t* the
// first k in index order, k the fewest with S(> t*) + k t* >= tau.  Every index is kept when
// tau >= 1 or when the total stays below tau.  The sums read the masses striped over the threads;
// the final pass, which needs index order among equal masses, gives thread t the range
// [t*L, t*L + L).
constexpr int CUT_WAYS = 4;
constexpr int CUT_BATCH = 8;  // loads in flight per thread in a pass
__global__ __launch_bounds__(CUT_THREADS) void sa_cut_kernel(const double* col, const double* slash, int N, int Hq,
                                                             double tau, uint8_t* keep) {
  __shared__ double wsum[CUT_WAYS][CUT_THREADS / 64];
  __shared__ int wcnt[CUT_THREADS / 64];
  __shared__ double wmax[CUT_THREADS / 64];
  __shared__ int wnum[CUT_THREADS / 64];
  const int h = blockIdx.x, fam = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const double* m = (fam == 0 ? col : slash) + (size_t)h * N;
  uint8_t* kp = keep + ((size_t)fam * Hq + h) * N;
  const int L = (N + CUT_THREADS - 1) / CUT_THREADS;
  const int b = min(t * L, N), e = min(b + L, N);
  // One pass: S at the patterns c_w = lo + (w + 1) step, w < CUT_WAYS (a pattern >= hi stands for
  // +inf, where S = 0).  Returns the last w with S(c_w) >= tau, or -1; the same on every thread.
  // Also counts the values whose pattern lies in [lo, hi) (*nwin) and returns the largest (*vwin).
  auto search_pass = [&](uint64_t lo, uint64_t step, uint64_t hi, int* nwin, double* vwin) -> int {
    double thr[CUT_WAYS], part[CUT_WAYS];
    // non-negative values order as their patterns; lo = ~0 (the all-test) matches no value
    const double wlo = lo < 0x7ff0000000000000ull ? __longlong_as_double((long long)lo) : INFINITY;
    const double whi = hi < 0x7ff0000000000000ull ? __longlong_as_double((long long)hi) : INFINITY;
    int cw = 0;
    double mw = -1.0;
#pragma unroll
    for (int w = 0; w < CUT_WAYS; ++w) {
      const uint64_t c = lo + (uint64_t)(w + 1) * step;
      thr[w] = c < hi ? __longlong_as_double((long long)c) : INFINITY;
      part[w] = 0.0;
    }
    // striped (coalesced) and in a fixed order; CUT_BATCH loads are issued before any is used
    for (int x0 = t; x0 < N; x0 += CUT_BATCH * CUT_THREADS) {
      double v[CUT_BATCH];
#pragma unroll
      for (int u = 0; u < CUT_BATCH; ++u) v[u] = x0 + u * CUT_THREADS < N ? m[x0 + u * CUT_THREADS] : -1.0;
#pragma unroll
      for (int u = 0; u < CUT_BATCH; ++u) {
#pragma unroll
        for (int w = 0; w < CUT_WAYS; ++w) part[w] += v[u] >= thr[w] ? v[u] : 0.0;
        const bool in = v[u] >= wlo && v[u] < whi;
        cw += in ? 1 : 0;
        mw = in ? fmax(mw, v[u]) : mw;
      }
    }
#pragma unroll
    for (int w = 0; w < CUT_WAYS; ++w)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) part[w] += __shfl_xor(part[w], o, 64);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      cw += __shfl_xor(cw, o, 64);
      mw = fmax(mw, __shfl_xor(mw, o, 64));
    }
    __syncthreads();  // the previous pass has read wsum
    if (lane == 0) {
#pragma unroll
      for (int w = 0; w < CUT_WAYS; ++w) wsum[w][wave] = part[w];
      wnum[wave] = cw;
      wmax[wave] = mw;
    }
    __syncthreads();
    {
      int n = 0;
      double mx = -1.0;
      for (int v = 0; v < CUT_THREADS / 64; ++v) {
        n += wnum[v];
        mx = fmax(mx, wmax[v]);
      }
      *nwin = n;
      *vwin = mx;
    }
    int best = -1;
#pragma unroll
    for (int w = 0; w < CUT_WAYS; ++w) {
      double sw = 0.0;
      for (int v = 0; v < CUT_THREADS / 64; ++v) sw += wsum[w][v];
      if (sw >= tau) best = w;
    }
    return best;
  };
  // every index when tau >= 1 or when the total S(+0) stays below tau (the bracket lo = -1 (wrapped),
  // step 1, hi = 1 evaluates c_0 = +0 alone)
  int nwin = 0;
  double vwin = 0.0;
  const bool all = tau >= 1.0 || search_pass(~0ull, 1, 1, &nwin, &vwin) < 0;
  if (all) {
    for (int x = b; x < e; ++x) kp[x] = 1;
    return;
  }
  uint64_t lo = 0, hi = 0x7ff0000000000000ull;  // S(+0) >= tau > S(+inf) = 0
  // S(lo) >= tau > S(hi) throughout, so t* lies in [lo, hi): once a single value is left there, it
  // is t* and the search stops (the later passes could only confirm it)
  while (hi - lo > 1) {
    const uint64_t step = (hi - lo + CUT_WAYS) / (CUT_WAYS + 1);  // >= 1
    const int best = search_pass(lo, step, hi, &nwin, &vwin);
    if (nwin == 1) {
      lo = (uint64_t)__double_as_longlong(vwin);
      hi = lo + 1;
      break;
    }
    const uint64_t nlo = best < 0 ? lo : lo + (uint64_t)(best + 1) * step;
    const uint64_t cn = lo + (uint64_t)(best + 2) * step;  // next candidate above the best
    const uint64_t nhi = (best + 1 < CUT_WAYS && cn < hi) ? cn : hi;
    lo = nlo;
    hi = nhi;
  }
  const double ts = __longlong_as_double((long long)lo);
  // S(> t*) = S(hi)
  double above;
  {
    double part = 0.0;
    const double th = __longlong_as_double((long long)hi);
    for (int x0 = t; x0 < N; x0 += CUT_BATCH * CUT_THREADS) {
      double v[CUT_BATCH];
#pragma unroll
      for (int u = 0; u < CUT_BATCH; ++u) v[u] = x0 + u * CUT_THREADS < N ? m[x0 + u * CUT_THREADS] : -1.0;
#pragma unroll
      for (int u = 0; u < CUT_BATCH; ++u) part += v[u] >= th ? v[u] : 0.0;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    __syncthreads();
    if (lane == 0) wsum[0][wave] = part;
    __syncthreads();
    above = 0.0;
    for (int v = 0; v < CUT_THREADS / 64; ++v) above += wsum[0][v];
  }
  int eq = 0;
  for (int x = b; x < e; ++x) eq += m[x] == ts;
  int total;  // values equal to t*
  int seen = block_exclusive_count(eq, wcnt, &total);
  int need = 0;  // equal values to take: the fewest k with above + k t* >= tau, at most all of them
  {
    double acc = above;
    while (acc < tau && need < total) {
      acc += ts;
      ++need;
    }
  }
  for (int x = b; x < e; ++x) {
    const double v = m[x];
    uint8_t k = v > ts;
    if (v == ts) {
      k = seen < need;
      ++seen;
    }
    kp[x] = k;
  }
}

// Per head: kept-column flags per key block, and prefix counts of kept slashes (spre[d] = kept
// slashes below offset d; N + 1 entries).
__global__ __launch_bounds__(CUT_THREADS) void sa_block_kernel(const uint8_t* keep, int N, int Hq, int B, int NB,
                                                               uint8_t* colblk, int32_t* spre) {
  __shared__ int wcnt[CUT_THREADS / 64];
  const int h = blockIdx.x, t = threadIdx.x;
  const uint8_t* kc = keep + (size_t)h * N;
  const uint8_t* ks = keep + ((size_t)Hq + h) * N;
  for (int J = t; J < NB; J += CUT_THREADS) {
    uint8_t any = 0;
    for (int j = J * B; j < min((J + 1) * B, N); ++j) any |= kc[j];
    colblk[(size_t)h * NB + J] = any;
  }
  const int L = (N + CUT_THREADS - 1) / CUT_THREADS;
  const int b = min(t * L, N), e = min(b + L, N);
  int cnt = 0;
  for (int x = b; x < e; ++x) cnt += ks[x];
  int total;
  int run = block_exclusive_count(cnt, wcnt, &total);
  int32_t* sp = spre + (size_t)h * (N + 1);
  for (int x = b; x < e; ++x) {
    sp[x] = run;
    run += ks[x];
  }
  if (t == 0) sp[N] = total;
}

// One wave per (h, I): tile (I, J), J <= I, is kept when forced, when block J holds a kept column,
// or when a kept slash offset lies in [I*B - (last key of J), (last query of I) - J*B].  The kept J
// are written in ascending order by ballot compaction.
__global__ __launch_bounds__(SA_THREADS) void sa_mask_kernel(const uint8_t* colblk, const int32_t* spre, int N, int Hq,
                                                             int B, int NB, uint32_t flags, int32_t* count,
                                                             int32_t* idx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (SA_THREADS / 64) + (threadIdx.x >> 6);
  if (row >= Hq * NB) return;
  const int h = row / NB, I = row % NB;
  const int qlast = min((I + 1) * B, N) - 1;
  const int32_t* sp = spre + (size_t)h * (N + 1);
  int32_t* out = idx + (size_t)h * ((size_t)NB * (NB + 1) / 2) + tri_offset(I);
  int n = 0;
  for (int J0 = 0; J0 <= I; J0 += 64) {
    const int J = J0 + lane;
    bool keep = false;
    if (J <= I) {
      const int klast = min((J + 1) * B, N) - 1;
      const int lo = max(0, I * B - klast), hi = qlast - J * B;
      keep = ((flags & 1u) && J == I) || ((flags & 2u) && J == 0) || colblk[(size_t)h * NB + J] ||
             (sp[hi + 1] - sp[lo] > 0);
    }
    const unsigned long long bal = __ballot(keep);
    if (keep) out[n + __popcll(bal & ((1ull << lane) - 1ull))] = J;
    n += __popcll(bal);
  }
  if (lane == 0) count[(size_t)h * NB + I] = n;
}

}  // namespace

size_t sample_mask_workspace_bytes(const Geometry& g, int n_trunks, int rpt) {
  const int R = g.G * n_trunks * rpt, nchunk = (g.N + SA_CK - 1) / SA_CK;
  return align256(sizeof(double) * g.Hkv * (size_t)nchunk * R) + 2 * align256(sizeof(double) * g.Hq * (size_t)g.N) +
         align256(2 * (size_t)g.Hq * g.N) + align256((size_t)g.Hq * g.NB) +
         align256(sizeof(int32_t) * g.Hq * ((size_t)g.N + 1)) + sampled_softmax_workspace_bytes(g, n_trunks, rpt);
}

hipError_t launch_sample_mask(const Geometry& g, const uint16_t* q, const uint16_t* k, double cia_tau, int n_trunks,
                              int rpt, uint32_t flags, int32_t* count, int32_t* idx, double* col, double* slash,
                              void* ws, hipStream_t st) {
  const SaWs w = carve(g, n_trunks, rpt, ws);
  SampledRows sr;
  hipError_t e = launch_sampled_softmax(g, q, k, n_trunks, rpt, w.softmax_ws, &sr, st);
  if (e != hipSuccess) return e;
  const int64_t nw = (int64_t)g.Hkv * sr.nchunk * sr.R;
  sa_weight_kernel<<<(unsigned)((nw + SA_THREADS - 1) / SA_THREADS), SA_THREADS, 0, st>>>(sr.part_m, sr.lse,
                                                                                          sr.nchunk, sr.R, nw, w.w);
  MassArgs a;
  a.e = sr.e;
  a.w = w.w;
  a.N = g.N;
  a.G = g.G;
  a.R = sr.R;
  a.R1 = n_trunks * rpt;
  a.nchunk = sr.nchunk;
  a.rpt = rpt;
  a.C = (g.N + n_trunks - 1) / n_trunks;
  double* cm = col ? col : w.col;
  double* sm = slash ? slash : w.slash;
  const dim3 mgrid((g.N + SA_THREADS - 1) / SA_THREADS, g.Hq);
  sa_col_kernel<<<mgrid, SA_THREADS, 0, st>>>(a, cm);
  sa_slash_kernel<<<mgrid, SA_THREADS, 0, st>>>(a, sm);
  sa_cut_kernel<<<dim3(g.Hq, 2), CUT_THREADS, 0, st>>>(cm, sm, g.N, g.Hq, cia_tau, w.keep);
  sa_block_kernel<<<g.Hq, CUT_THREADS, 0, st>>>(w.keep, g.N, g.Hq, g.B, g.NB, w.colblk, w.spre);
  const int rows = g.Hq * g.NB, per = SA_THREADS / 64;
  sa_mask_kernel<<<(rows + per - 1) / per, SA_THREADS, 0, st>>>(w.colblk, w.spre, g.N, g.Hq, g.B, g.NB, flags, count,
                                                               idx);
  return hipGetLastError();
}

}  // namespace pbsa
