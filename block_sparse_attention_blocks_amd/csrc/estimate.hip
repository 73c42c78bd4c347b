// Stage 1 (key importance, segment sort) and stage 2 (pooling, block selection) on gfx950.
//
// Ranks and cumulative-mass cuts decided here must agree with an fp64 evaluation of the same
// definitions bit for bit except at genuine near-ties, so nothing is summed in fp32:
//   * the importance logits q.k are exact integer sums on the int8 matrix cores: each bf16 row is
//     written as a 42-bit fixed-point integer at its own largest exponent (exact for every element
//     within 2^34 of the row's largest) and split into six 7-bit digits; the digit products whose
//     weight is at least 2^-42 of the leading one are summed in int32 and combined in fp64, so a
//     logit is off by at most 6 d 2^-40 max|q| max|k| (the dropped products and truncated
//     elements), far below fp32 rounding;
//   * block means of bf16 rows are exact sums divided by a power of two, taken in fp64, and
//     everything after the logits (exponentials, sums, softmax) is fp64.
// The one fp32 value is storage: the importance pass keeps its chunk-normalised exponentials
// (numbers in (0, 1]) rounded to fp32 between its two halves, which moves each importance by at
// most 2^-24 relative (every term is positive) and halves the pass's largest memory stream.
#include "estimate.h"

#include <math.h>

namespace pbsa {

// =====================================================================================
// Stage 1a: key importance (Sparser Block-Sparse Attention via Token Permutation, section 3,
// "Proxy Scoring").  The proxy rows of KV head g are (h, i) with h in g's query-head group and
// i in [N - R1, N), R1 = min(B, N); there are R = G * R1 of them.  Row r maps to
// h = g*G + r / R1, i = N - R1 + r % R1.  imp_j = (1/R) sum_r exp(s_rj - lse_r), s_rj = c q_r.k_j
// over causal j <= i.  Four launches:
//   imp_kdigits: per key row, its fixed-point digits (below) and exponent, once per key
//   imp_scores : per (64-key chunk c, g), the logits of all R rows from digit products on the
//                int8 matrix cores (v_mfma_i32_16x16x64_i8); per row the chunk max m_cr and
//                l_cr = sum exp(s - m_cr) (fp64), and e_rj = exp(s_rj - m_cr) stored to the
//                workspace rounded to fp32
//   imp_lse    : per (row, g), lse_r = M + log sum_c l_cr exp(m_cr - M)
//   imp_colsum : per key, imp_j = (1/R) sum_r e_rj exp(m_c(j)r - lse_r) in row order
// so every logit is computed once and exponentiated once.
//
// Fixed-point digits.  A bf16 value is x = M 2^(e' - 134): M its significand with the implicit bit
// (0..255), e' = max(e, 1) for the exponent field e.  With E the largest e' of x's row (for keys:
// of the 64-key chunk),
// V = trunc(M 2^(e' - E + 34)) is an integer below 2^42 (exact whenever E - e' <= 34) and
// x = (+-V) 2^(E - 168) up to that truncation.  In two's complement, +-V = sum_a D_a 2^(35 - 7a)
// (a = 0..5) with D_0 = (+-V) >> 35 in [-128, 127] and D_a (a >= 1) the 7-bit fields below it, in
// [0, 127]; every digit fits an int8.  For a query row and a key row,
//   q.k = 2^(Eq + Ek - 336) sum_{a,b} (sum_t Dq_a,t Dk_b,t) 2^(70 - 7(a + b)),
// and the level sums A_L = sum_{a+b=L} sum_t Dq_a Dk_b are exact in int32 (|A_L| <= (L+1) d 2^14).
// Levels L <= 5 are kept (21 digit products per 64-wide contraction step); levels 6..10 weigh at
// most 2^-42 of level 0 each.  A_L 2^7 + A_{L+1} still fits an int32 for the pairs (0,1), (2,3),
// (4,5), so a logit is  ((C01 2^14 + C23) 2^14 + C45) 2^(Eq + Ek - 301)  with two fp64 FMAs.
// =====================================================================================

constexpr int IMP_CK = 64;        // keys per chunk (4 MFMA column tiles of 16)
constexpr int IMP_RT = 128;       // proxy rows per workgroup (8 waves x 16 rows)
constexpr int IMP_THREADS = 512;
constexpr int IMP_KR = 16;        // chunks per workgroup, at most (fewer when the grid would be small)
constexpr int COL_KEYS = 256;     // keys per workgroup of imp_colsum
constexpr int COL_ROWS = 256;     // rows staged per pass of imp_colsum

constexpr int IMP_NDIG = 6;       // fixed-point digits per bf16 value

typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Digits of the key rows, chunk-major: [Hkv][nchunk][IMP_NDIG][IMP_CK][d] bytes, then the chunk
// exponents E [Hkv][nchunk] (int32).  Keys past N are zero rows (digits 0).
static inline size_t kdig_bytes(const Geometry& g, size_t nchunk) {
  return (size_t)g.Hkv * nchunk * IMP_NDIG * IMP_CK * g.d;
}
static inline size_t kexp_bytes(const Geometry& g, size_t nchunk) { return sizeof(int) * g.Hkv * nchunk; }

struct ImpWs {
  float* e;        // [Hkv][R][N] chunk-normalised exponentials, rounded to fp32
  double* part_m;  // [Hkv][nchunk][R]
  double* part_l;  // [Hkv][nchunk][R]
  double* lse;     // [Hkv][R]
  double* imp;     // [Hkv][N] (used when the caller passes no importance output)
  int8_t* kdig;    // key digits (layout above)
  int* kexp;       // key chunk exponents
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
  w.e = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * g.Hkv * R * (size_t)g.N);
  w.part_m = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * C * R);
  w.part_l = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * C * R);
  w.lse = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * R);
  w.imp = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)g.N);
  w.kdig = reinterpret_cast<int8_t*>(p);
  p += align256(kdig_bytes(g, C));
  w.kexp = reinterpret_cast<int*>(p);
  return w;
}

size_t importance_workspace_bytes(const Geometry& g) {
  const size_t R = imp_rows(g), C = imp_chunks(g);
  return align256(sizeof(float) * g.Hkv * R * (size_t)g.N) + 2 * align256(sizeof(double) * g.Hkv * C * R) +
         align256(sizeof(double) * g.Hkv * R) + align256(sizeof(double) * g.Hkv * (size_t)g.N) +
         align256(kdig_bytes(g, C)) + align256(kexp_bytes(g, C));
}

struct ImpArgs {
  const uint16_t* q;
  const uint16_t* k;
  int N, G, d, R1, R, Hkv;
  int64_t qsh, qst, kvsh, kvst;
  double scale;
  int trunk_c;    // 0: proxy rows are the last R1 positions; > 0: trunk-sampled rows (chunk length)
  int rpt;        // trunk sampling: rows per trunk
  int first_row;  // smallest proxy position (every key j <= first_row is visible to every proxy row)
  int kr;         // key chunks per workgroup
};

// Chunks per workgroup: IMP_KR, or fewer so that short sequences still spread over at least ~512
// workgroups (a chunk's results do not depend on which workgroup computes it).
static inline int imp_chunks_per_wg(int row_blocks, int nchunk, int hkv) {
  const long long wg_at_one = (long long)row_blocks * nchunk * hkv;
  const long long kr = wg_at_one / 512;
  return (int)(kr < 1 ? 1 : kr > IMP_KR ? IMP_KR : kr);
}

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

// DPP row rotation of a double (16-lane rows): all-reduce helpers for the 16 lanes of one row.  A
// rotation reads a lane of the same row for every lane, so no fill value is needed (mov_dpp).
template <int N>
__device__ __forceinline__ double row_ror_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0x120 + N, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0x120 + N, 0xf, 0xf, false);
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


// exp(dT F) for the logits of the importance pass: dT = T - Tmax <= 0 in the integer units of the
// logit (-inf allowed when MASKED), F > 0 the unit.  With t = dT G (G = F 256 / ln2, clamped at
// -280000) and n = rint(t), the remainder r = (dT - n K) F, K = ln2 / (256 F), has |r| <= ln2/512
// up to rounding (n K F = n ln2/256 to 2^-53 relative, |n| <= 280000: below 1e-13 absolute), and
// exp = 2^(n >> 8) tab[n & 255] p(r) with tab[j] = 2^(j/256) and p the Taylor polynomial of e^r to
// degree 3 (truncation below 1.5e-13 relative).  MASKED: below t = -275200 (dT F < -745.2, which
// covers dT = -inf) the result is 0.  Without MASKED (every dT finite) that test is left out: there
// the ldexp alone gives 0 or a subnormal below 2^-1022, and the values are stored as fp32, whose
// range ends at 2^-149 anyway.
template <bool MASKED>
__device__ __forceinline__ double exp_chunk(double dT, double F, double G, double K, const double* tab) {
  const double t = fmax(dT * G, -280000.0);
  const double n = rint(t);
  const double r = fma(-n, K, dT) * F;
  double p = fma(r, 1.0 / 6.0, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const int ni = (int)n;
  const double y = ldexp(tab[ni & 255] * p, ni >> 8);
  return (MASKED && t < -275200.0) ? 0.0 : y;
}

// Largest exponent field (at least 1) of the bf16 values packed two to a word.
__device__ __forceinline__ int bf16_pair_emax(uint32_t w) {
  return max(max((int)((w >> 7) & 0xffu), (int)((w >> 23) & 0xffu)), 1);
}

// The fixed-point integer +-V of bf16 bits h in a row whose largest exponent is emax (the digit
// representation above): two's complement, |V| < 2^42.
__device__ __forceinline__ uint64_t bf16_fixed(uint32_t h, int emax) {
  const int e = (int)((h >> 7) & 0xffu);
  const uint32_t m = (h & 0x7fu) | (e ? 0x80u : 0u);
  const int sh = 34 - (emax - max(e, 1));
  const uint64_t v = sh >= 0 ? ((uint64_t)m << sh) : (uint64_t)(m >> min(-sh, 31));
  return (h & 0x8000u) ? (uint64_t)(-(int64_t)v) : v;
}

// Digit a (0 = leading, signed) of a fixed-point integer, as the byte the int8 operand holds.
template <int A>
__device__ __forceinline__ uint32_t fixed_digit(uint64_t v) {
  return A == 0 ? (uint32_t)(v >> 35) & 0xffu : (uint32_t)(v >> (35 - 7 * A)) & 0x7fu;
}

// Digits of four fixed-point integers as one word (byte i from v[i]).
template <int A>
__device__ __forceinline__ uint32_t pack_digits(const uint64_t* v) {
  return fixed_digit<A>(v[0]) | (fixed_digit<A>(v[1]) << 8) | (fixed_digit<A>(v[2]) << 16) |
         (fixed_digit<A>(v[3]) << 24);
}

// Key digits, once per key: one workgroup per (64-key chunk, KV head); a thread takes 8 values
// (16 bytes) of a row.  All keys of a chunk share one exponent E (the largest over the chunk), so
// a logit's unit is the same along a row of the chunk.
template <int D>
__global__ __launch_bounds__(256) void imp_kdigits_kernel(const uint16_t* k, int N, int64_t kvsh, int64_t kvst,
                                                          int8_t* kdig, int* kexp) {
  constexpr int cpr = D / 8;
  constexpr int NLD = IMP_CK * cpr / 256;
  __shared__ int wmax[4];
  const int c = blockIdx.x, g = blockIdx.y, t = threadIdx.x, nchunk = gridDim.x;
  const uint16_t* kbase = k + (int64_t)g * kvsh;
  int8_t* out = kdig + ((size_t)g * nchunk + c) * IMP_NDIG * IMP_CK * D;
  u32x4 w[NLD];
  int em = 1;
#pragma unroll
  for (int x = 0; x < NLD; ++x) {
    const int idx = t + x * 256, row = idx / cpr, ch = idx % cpr, j = c * IMP_CK + row;
    w[x] = u32x4{0u, 0u, 0u, 0u};
    if (j < N) w[x] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * kvst + ch * 8);
    em = max(em, max(max(bf16_pair_emax(w[x][0]), bf16_pair_emax(w[x][1])),
                     max(bf16_pair_emax(w[x][2]), bf16_pair_emax(w[x][3]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) em = max(em, __shfl_xor(em, o));
  if ((t & 63) == 0) wmax[t >> 6] = em;
  __syncthreads();
  em = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
#pragma unroll
  for (int x = 0; x < NLD; ++x) {
    const int idx = t + x * 256, row = idx / cpr, ch = idx % cpr;
    uint64_t v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_fixed(w[x][e] & 0xffffu, em);
      v[2 * e + 1] = bf16_fixed(w[x][e] >> 16, em);
    }
    int8_t* o = out + row * D + ch * 8;
    *reinterpret_cast<uint2*>(o + 0 * IMP_CK * D) = make_uint2(pack_digits<0>(v), pack_digits<0>(v + 4));
    *reinterpret_cast<uint2*>(o + 1 * IMP_CK * D) = make_uint2(pack_digits<1>(v), pack_digits<1>(v + 4));
    *reinterpret_cast<uint2*>(o + 2 * IMP_CK * D) = make_uint2(pack_digits<2>(v), pack_digits<2>(v + 4));
    *reinterpret_cast<uint2*>(o + 3 * IMP_CK * D) = make_uint2(pack_digits<3>(v), pack_digits<3>(v + 4));
    *reinterpret_cast<uint2*>(o + 4 * IMP_CK * D) = make_uint2(pack_digits<4>(v), pack_digits<4>(v + 4));
    *reinterpret_cast<uint2*>(o + 5 * IMP_CK * D) = make_uint2(pack_digits<5>(v), pack_digits<5>(v + 4));
  }
  if (t == 0) kexp[(size_t)g * nchunk + c] = em;
}

// v_mfma_i32_16x16x64_i8 (lane l): A holds row l%16 and B column l%16, each 16 int8 of the
// contraction from lane group l/16 (the same 16 indices on both sides); D holds column l%16, rows
// 4 (l/16) + i in its four int32 i = 0..3.  Each wave keeps the digits of its 16 proxy rows in
// registers (A), lane group lg holding elements 64 h + 16 lg .. + 15 of each 64-wide step h; the key
// digits of a chunk are copied to LDS, one row of each digit plane per key padded to D + 16 bytes
// (the 16 lanes of a B read then cover all 64 banks once), while the next chunk's digits are loaded
// into registers.  Workgroups are numbered so that the row blocks of one chunk range are dispatched
// to the same XCD (consecutive workgroup ids go to consecutive XCDs) and read its key digits
// through one L2.  ET is the stored type of the exponentials (fp32 for both users of the kernel).
template <int D, typename ET>
__global__ __launch_bounds__(IMP_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void imp_scores_kernel(
    ImpArgs a, const int8_t* kdig, const int* kexp,
                                                                 ET* E, double* part_m, double* part_l) {
  constexpr int NH = D / 64;                       // 64-wide contraction steps
  constexpr int PITCH = D + 16;                    // bytes per key row of a staged digit plane
  constexpr int U16 = D / 16;                      // 16-byte pieces per key row of a plane
  constexpr int NST = IMP_NDIG * IMP_CK * U16 / IMP_THREADS;  // pieces per thread per chunk
  __shared__ __align__(16) int8_t Ks[IMP_NDIG * IMP_CK * PITCH];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int nchunk = (a.N + IMP_CK - 1) / IMP_CK;

  // work item: XCD x = blockIdx.x % 8 takes items x * per + blockIdx.x / 8 (row block fastest)
  const int nrb = (a.R + IMP_RT - 1) / IMP_RT, ncg = (nchunk + a.kr - 1) / a.kr;
  const int items = nrb * ncg * a.Hkv, per = (items + 7) / 8;
  const int item = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (item >= items) return;
  const int r0 = (item % nrb) * IMP_RT, g = item / (nrb * ncg);
  const int c0 = ((item / nrb) % ncg) * a.kr, c1 = min(c0 + a.kr, nchunk);

  // A operand: digits of proxy row r0 + 16 w + l16, elements 64 h + 16 lg + i
  const int ra = r0 + 16 * w + l16;
  i32x4 av[IMP_NDIG][NH];
  int emq;
  {
    const uint16_t* src = nullptr;
    if (ra < a.R) {
      int h, i;
      imp_row(a, g, ra, &h, &i);
      src = a.q + (int64_t)h * a.qsh + (int64_t)i * a.qst;
    }
    u32x4 raw[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        raw[h][c] = src ? *reinterpret_cast<const u32x4*>(src + 64 * h + 16 * lg + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    emq = 1;
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) emq = max(emq, bf16_pair_emax(raw[h][c][e]));
    emq = max(emq, __shfl_xor(emq, 16));
    emq = max(emq, __shfl_xor(emq, 32));
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {  // elements 4 q4 .. 4 q4 + 3 of the lane's 16
        const u32x4& r = raw[h][q4 >> 1];
        uint64_t v[4];
        v[0] = bf16_fixed(r[2 * (q4 & 1)] & 0xffffu, emq);
        v[1] = bf16_fixed(r[2 * (q4 & 1)] >> 16, emq);
        v[2] = bf16_fixed(r[2 * (q4 & 1) + 1] & 0xffffu, emq);
        v[3] = bf16_fixed(r[2 * (q4 & 1) + 1] >> 16, emq);
        av[0][h][q4] = (int)pack_digits<0>(v);
        av[1][h][q4] = (int)pack_digits<1>(v);
        av[2][h][q4] = (int)pack_digits<2>(v);
        av[3][h][q4] = (int)pack_digits<3>(v);
        av[4][h][q4] = (int)pack_digits<4>(v);
        av[5][h][q4] = (int)pack_digits<5>(v);
      }
  }
  // this lane's D rows (proxy rows r0 + 16 w + 4 lg + rr): query positions and exponents; the unit
  // of a logit is c 2^(Eq + Ek - 301)
  int qi[4], eq[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = r0 + 16 * w + 4 * lg + rr;
    int h, i;
    imp_row(a, g, r, &h, &i);
    qi[rr] = r < a.R ? i : -1;
    eq[rr] = __shfl(emq, 4 * lg + rr) - 301;
  }
  const double cG = a.scale * (256.0 / 0.69314718055994530942), cK = 0.69314718055994530942 / (256.0 * a.scale);
  __shared__ double tab[256];  // 2^(j/256)
  static_assert(IMP_THREADS >= 256, "one table entry per thread");
  if (t < 256) tab[t] = exp2((double)t * (1.0 / 256.0));
  const int first_proxy = a.first_row;  // every key j <= first_proxy is visible to every proxy row

  const int8_t* kd = kdig + (size_t)g * nchunk * IMP_NDIG * IMP_CK * D;
  const int* ke = kexp + (size_t)g * nchunk;
  auto prefetch = [&](int c, u32x4* pf) {
    const u32x4* src = reinterpret_cast<const u32x4*>(kd + (size_t)c * IMP_NDIG * IMP_CK * D);
#pragma unroll
    for (int x = 0; x < NST; ++x) pf[x] = src[t + x * IMP_THREADS];
  };
  // piece u = t + x * IMP_THREADS of the chunk: plane u / (IMP_CK U16), key (u / U16) % IMP_CK,
  // bytes 16 (u % U16) of the row
  auto stage = [&](const u32x4* pf) {
#pragma unroll
    for (int x = 0; x < NST; ++x) {
      const int u = t + x * IMP_THREADS;
      const int pl = u / (IMP_CK * U16), key = (u / U16) % IMP_CK, pc = u % U16;
      *reinterpret_cast<u32x4*>(Ks + (pl * IMP_CK + key) * PITCH + 16 * pc) = pf[x];
    }
  };
  const int8_t* bbase = Ks + l16 * PITCH + 16 * lg;  // B of plane b, column tile tt, step h

  u32x4 pf[NST];
  prefetch(c0, pf);
  for (int c = c0; c < c1; ++c) {
    stage(pf);
    const int ek = ke[c];
    __syncthreads();
    if (c + 1 < c1) prefetch(c + 1, pf);
    double x[4][4];  // logit of row 4 lg + rr, key 16 tt + l16, in units of c 2^(Eq + Ek - 301)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      i32x4 lv[IMP_NDIG];
#pragma unroll
      for (int L = 0; L < IMP_NDIG; ++L) lv[L] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int b = 0; b < IMP_NDIG; ++b) {
          const i32x4 bv = *reinterpret_cast<const i32x4*>(bbase + (b * IMP_CK + 16 * tt) * PITCH + 64 * h);
#pragma unroll
          for (int aa = 0; aa + b < IMP_NDIG; ++aa)
            lv[aa + b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[aa][h], bv, lv[aa + b], 0, 0, 0);
        }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c01 = lv[0][rr] * 128 + lv[1][rr];
        const int c23 = lv[2][rr] * 128 + lv[3][rr];
        const int c45 = lv[4][rr] * 128 + lv[5][rr];
        x[tt][rr] = fma(fma((double)c01, 16384.0, (double)c23), 16384.0, (double)c45);
      }
    }
    // per proxy row: chunk max, sum of exponentials, and the exponentials themselves
    const int j0 = c * IMP_CK;
    const bool open = j0 + IMP_CK - 1 <= first_proxy && j0 + IMP_CK <= a.N;  // no key of the chunk is masked
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const double F = ldexp(a.scale, eq[rr] + ek), G = ldexp(cG, eq[rr] + ek), K = ldexp(cK, -eq[rr] - ek);
      double sv[4];
      double m;
      if (open) {
        const double tm = row_max_f64(fmax(fmax(x[0][rr], x[1][rr]), fmax(x[2][rr], x[3][rr])));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sv[tt] = exp_chunk<false>(x[tt][rr] - tm, F, G, K, tab);
        m = tm * F;
      } else {
        const int i = qi[rr];
        double tm = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int j = j0 + 16 * tt + l16;
          const bool ok = (i >= 0) && (j < a.N) && (j <= i);
          sv[tt] = ok ? x[tt][rr] : -INFINITY;
          tm = fmax(tm, sv[tt]);
        }
        tm = row_max_f64(tm);
        const double tmm = tm > -INFINITY ? tm : 0.0;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sv[tt] = exp_chunk<true>(sv[tt] - tmm, F, G, K, tab);
        m = tm * F;  // -inf for a row with no key in the chunk
      }
      double l = (sv[0] + sv[1]) + (sv[2] + sv[3]);
      l = row_sum_f64(l);
      const int r = r0 + 16 * w + 4 * lg + rr;
      if (r < a.R) {
        ET* er = E + ((size_t)g * a.R + r) * a.N;
        if (j0 + IMP_CK <= a.N) {  // the chunk lies inside the sequence: one address, no key checks
          ET* ej = er + j0 + l16;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) ej[16 * tt] = (ET)sv[tt];
        } else {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int j = j0 + 16 * tt + l16;
            if (j < a.N) er[j] = (ET)sv[tt];
          }
        }
        if (l16 == 0) {
          const size_t o = ((size_t)g * nchunk + c) * a.R + r;
          part_m[o] = m;
          part_l[o] = l;
        }
      }
    }
    __syncthreads();  // every wave is done with this chunk's digits before they are replaced
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

// imp_j = (1/R) sum_r e_rj * exp(m_c(j)r - lse_r), rows summed in order in fp64.
__global__ __launch_bounds__(COL_KEYS) void imp_colsum_kernel(const float* E, const double* part_m,
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
      const float* col = E + ((size_t)g * R + rb) * N + j;
      const int nr = min(COL_ROWS, R - rb);
      const double* wc = wsh[t / IMP_CK];
      for (int rr = 0; rr < nr; ++rr) sum = fma((double)col[(size_t)rr * N], wc[rr], sum);
    }
  }
  if (j < N) imp[(size_t)g * N + j] = sum / (double)R;
}

// Key digits, then the logits and chunk exponentials of the R proxy rows (a fully set up).
static void launch_scores(const Geometry& g, const ImpArgs& a, int8_t* kdig, int* kexp, float* e, double* part_m,
                          double* part_l, hipStream_t st) {
  const int nchunk = imp_chunks(g);
  const int items = ((a.R + IMP_RT - 1) / IMP_RT) * ((nchunk + a.kr - 1) / a.kr) * g.Hkv;
  const int nwg = (items + 7) / 8 * 8;
  if (g.d == 128) {
    imp_kdigits_kernel<128><<<dim3(nchunk, g.Hkv), 256, 0, st>>>(a.k, g.N, g.kvsh, g.kvst, kdig, kexp);
    imp_scores_kernel<128, float><<<nwg, IMP_THREADS, 0, st>>>(a, kdig, kexp, e, part_m, part_l);
  } else {
    imp_kdigits_kernel<64><<<dim3(nchunk, g.Hkv), 256, 0, st>>>(a.k, g.N, g.kvsh, g.kvst, kdig, kexp);
    imp_scores_kernel<64, float><<<nwg, IMP_THREADS, 0, st>>>(a, kdig, kexp, e, part_m, part_l);
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
  a.trunk_c = 0;
  a.rpt = 0;
  a.first_row = g.N - a.R1;
  const int nchunk = imp_chunks(g);
  a.Hkv = g.Hkv;
  a.kr = imp_chunks_per_wg((a.R + IMP_RT - 1) / IMP_RT, nchunk, g.Hkv);
  launch_scores(g, a, w.kdig, w.kexp, w.e, w.part_m, w.part_l, st);
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
  return align256(sizeof(float) * g.Hkv * R * (size_t)g.N) + 2 * align256(sizeof(double) * g.Hkv * C * R) +
         align256(sizeof(double) * g.Hkv * R) + align256(kdig_bytes(g, C)) + align256(kexp_bytes(g, C));
}

hipError_t launch_sampled_softmax(const Geometry& g, const uint16_t* q, const uint16_t* k, int n_trunks, int rpt,
                                  void* ws, SampledRows* out, hipStream_t st) {
  const int R = g.G * n_trunks * rpt, nchunk = imp_chunks(g);
  char* p = static_cast<char*>(ws);
  out->e = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * g.Hkv * (size_t)R * g.N);
  out->part_m = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)nchunk * R);
  double* part_l = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)nchunk * R);
  out->lse = reinterpret_cast<double*>(p);
  p += align256(sizeof(double) * g.Hkv * (size_t)R);
  int8_t* kdig = reinterpret_cast<int8_t*>(p);
  p += align256(kdig_bytes(g, nchunk));
  int* kexp = reinterpret_cast<int*>(p);
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
  a.Hkv = g.Hkv;
  a.kr = imp_chunks_per_wg((R + IMP_RT - 1) / IMP_RT, nchunk, g.Hkv);
  launch_scores(g, a, kdig, kexp, out->e, out->part_m, part_l, st);
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

__device__ __forceinline__ void pool_body(const uint16_t* src, int64_t sh, int64_t st_, int N, int B, int d,
                                          const int32_t* rowmap, double* dst, int NB, int h) {
  __shared__ double part[32][128];
  const int J = blockIdx.x, t = threadIdx.x;
  const int lanes = d / 8;                 // threads per row
  const int rp = POOL_THREADS / lanes;     // rows in flight
  const int c = t % lanes, rs = t / lanes;
  const int r0 = J * B;
  const int cnt = min(B, N - r0);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = src + (int64_t)h * sh;
  // four rows per trip: their loads are all issued before the first is added, and the rows are
  // added in ascending order as before
  constexpr int U = 4;
  for (int rb = rs; rb < cnt; rb += U * rp) {
    int pos[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * rp;
      pos[u] = r < cnt ? (rowmap ? rowmap[(size_t)h * N + r0 + r] : r0 + r) : -1;
    }
    u32x4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = pos[u] >= 0 && pos[u] < N;  // a corrupt index list contributes nothing
      raw[u] = ok ? *reinterpret_cast<const u32x4*>(base + (int64_t)pos[u] * st_ + c * 8) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (pos[u] < 0 || pos[u] >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_bits_to_f32(raw[u][e] & 0xffffu);
        acc[2 * e + 1] += (double)bf16_bits_to_f32(raw[u][e] >> 16);
      }
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

// The three poolings of the mask stage in one launch (fewer launches on short sequences): grid rows
// [0, Hq) pool Q, the next Hkv the natural K, the last Hkv (when perm is given) the permuted K.
struct PoolJobs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t qsh, qst, ksh, kst;
  const int32_t* perm;
  double *qbar, *knat, *kperm;
  int Hq, Hkv;
};
__global__ __launch_bounds__(POOL_THREADS) void pool_kernel(PoolJobs p, int N, int B, int d, int NB) {
  const int y = blockIdx.y;
  if (y < p.Hq)
    pool_body(p.q, p.qsh, p.qst, N, B, d, nullptr, p.qbar, NB, y);
  else if (y < p.Hq + p.Hkv)
    pool_body(p.k, p.ksh, p.kst, N, B, d, nullptr, p.knat, NB, y - p.Hq);
  else
    pool_body(p.k, p.ksh, p.kst, N, B, d, p.perm, p.kperm, NB, y - p.Hq - p.Hkv);
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
    // Invariant: mass_ge(tstar) >= tau > mass_ge(tstar + 2^(bit+1)), so t* lies in that window.
    // Once the window holds a single value of the row, that value is t*: the remaining probes
    // could only confirm it, so the search stops there (checked from the mantissa bits on).
    for (int bit = 62; bit >= 0; --bit) {
      if (bit < 52) {
        const uint64_t hi = tstar + (2ull << bit);  // window [tstar, hi); bit <= 51, no overflow
        int cnt = 0;
        int src = -1, slot = 0;
#pragma unroll
        for (int i = 0; i < SEL_PL; ++i) {
          if (i < npl) {
            const uint64_t key = (uint64_t)__double_as_longlong(v[i]);
            const unsigned long long bw = __ballot(lane + 64 * i < nJ && key >= tstar && key < hi);
            if (bw && src < 0) {
              src = __ffsll((long long)bw) - 1;
              slot = i;
            }
            cnt += __popcll(bw);
          }
        }
        if (cnt == 1) {
          double only = 0.0;
#pragma unroll
          for (int i = 0; i < SEL_PL; ++i)
            if (i == slot) only = __shfl(v[i], src, 64);
          tstar = (uint64_t)__double_as_longlong(only);
          break;
        }
      }
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
  {
    PoolJobs pj = {q, k, g.qsh, g.qst, g.kvsh, g.kvst, perm, qbar, knat, kperm, g.Hq, g.Hkv};
    pool_kernel<<<dim3(g.NB, g.Hq + (perm ? 2 : 1) * g.Hkv), POOL_THREADS, 0, st>>>(pj, g.N, g.B, g.d, g.NB);
  }
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
