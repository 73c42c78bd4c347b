// Stage 3: causal block-sparse attention prefill with index-driven K/V gather, on gfx950.
//
// One workgroup computes one (query head h, query block I): BLK query rows, one wave per 32 rows.
// It walks the row's kept key blocks J in ascending order.  For each J the workgroup
//   1. resolves the BLK physical key rows of J (through perm when J's segment precedes I's:
//      S2O section 1, the index list steers the load and nothing is moved),
//   2. gathers the K tile (and V tile) from HBM into LDS with 16-byte loads per lane,
//   3. computes S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_bf16), so every lane owns
//      one query column and the online softmax (S2O section 3: m, l, acc) needs no cross-lane
//      work except one swap between the two half-waves,
//   4. optionally gates the tile on its exact max score (Block Sparse Flash Attention, Approach):
//      below the threshold the V load and PV are skipped,
//   5. accumulates O^T += V^T P^T on the matrix cores from a transposed V tile in LDS.
//
// MFMA 32x32x16 bf16 register layouts used below (lane = 0..63, l32 = lane % 32, h2 = lane / 32):
//   A (32 x 16): lane holds row l32, k = 8*h2 + e (e = 0..7)
//   B (16 x 32): lane holds column l32, k = 8*h2 + e
//   C (32 x 32): lane holds column l32, rows 8*(r/4) + 4*h2 + r%4 in register r = 0..15
// Only the pairing of A and B along k matters for a contraction, so V^T is stored with the key
// order inside every 16-key group permuted to match the keys that the P^T operand inherits from
// the layout of S^T.
#include "common.h"

#include <math.h>

namespace pbsa {

template <int D, int BLK>
struct AttnCfg {
  static constexpr int WAVES = BLK / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  static constexpr int KSTEPS = D / 16;                // k-steps of S^T = K Q^T
  static constexpr int KB = BLK / 32;                  // 32-key sub-blocks of a tile
  static constexpr int DB = D / 32;                    // 32-row d sub-blocks of O^T
  static constexpr int KLOADS = BLK * KCH / THREADS;   // K chunks per thread
  static constexpr int VBLOCKS = (BLK / 8) * (D / 8);  // 8 x 8 blocks of the V transpose
};

// LDS swizzles: XOR the 16-byte chunk index so that MFMA operand reads (32 consecutive rows, one
// chunk) and tile writes hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int BLK>
__device__ __forceinline__ int v_swz(int d) {
  return BLK == 128 ? (((d >> 3) + 2 * (d & 7)) & 15) : ((d >> 1) & 7);
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;
  const int32_t* count;
  const int32_t* idx;
  const float* theta;
  float* out;
  float* lse;
  uint32_t* kept;
  int32_t* err;
  float* tmax;
  int N, Hq, G, S, NB;
  int64_t qsh, kvsh, osh, ost;          // head strides (elements), out token stride
  uint32_t q_row_bytes, kv_row_bytes;    // token strides in bytes
  uint32_t q_bytes, kv_bytes;            // bytes of one head's slab (buffer bound)
  float scale;  // c
  float sl2;    // c * log2(e)
};

enum { MODE_ATTN = 0, MODE_ATTN_GATED = 1, MODE_TILE_MAX = 2 };

__device__ __forceinline__ uint32_t half16(const u32x4& x, int dd) {
  return (x[dd >> 1] >> ((dd & 1) * 16)) & 0xffffu;
}

template <int D, int BLK>
__device__ __forceinline__ void load_k_tile(uint16_t* Ks, rsrc_t kr, uint32_t row_bytes, const int* rowid) {
  using C = AttnCfg<D, BLK>;
  const int t = threadIdx.x;
  u32x4 val[C::KLOADS];
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int ci = t + i * C::THREADS;
    const int row = ci / C::KCH, c = ci % C::KCH;
    const int r = rowid[row];
    val[i] = buf_load16(kr, r >= 0 ? (uint32_t)r * row_bytes + c * 16 : kOutOfRange);
  }
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int ci = t + i * C::THREADS;
    const int row = ci / C::KCH, c = ci % C::KCH;
    *reinterpret_cast<u32x4*>(Ks + row * D + ((c ^ k_swz<D>(row)) * 8)) = val[i];
  }
}

// V tile [BLK keys][D] -> LDS V^T [D][BLK] with the per-16-key position map
// key k -> (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1), via an 8 x 8 register transpose per thread.
template <int D, int BLK>
__device__ __forceinline__ void load_v_tile(uint16_t* Vt, rsrc_t vr, uint32_t row_bytes, const int* rowid) {
  using C = AttnCfg<D, BLK>;
  const int t = threadIdx.x;
  if (C::VBLOCKS < C::THREADS && t >= C::VBLOCKS) return;
  const int dg = t % (D / 8), kg = t / (D / 8);
  u32x4 rv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = rowid[kg * 8 + i];
    rv[i] = buf_load16(vr, r >= 0 ? (uint32_t)r * row_bytes + dg * 16 : kOutOfRange);
  }
  const int c0 = (kg >> 1) * 2, sub = (kg & 1) * 4;
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) {
    const int d = dg * 8 + dd;
    const int sw = v_swz<BLK>(d);
    u32x2 lo, hi;
    lo[0] = half16(rv[0], dd) | (half16(rv[1], dd) << 16);
    lo[1] = half16(rv[2], dd) | (half16(rv[3], dd) << 16);
    hi[0] = half16(rv[4], dd) | (half16(rv[5], dd) << 16);
    hi[1] = half16(rv[6], dd) | (half16(rv[7], dd) << 16);
    *reinterpret_cast<u32x2*>(Vt + d * BLK + ((c0 ^ sw) * 8) + sub) = lo;
    *reinterpret_cast<u32x2*>(Vt + d * BLK + (((c0 + 1) ^ sw) * 8) + sub) = hi;
  }
}

template <int D, int BLK, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(AttnCfg<D, BLK>::THREADS, AttnCfg<D, BLK>::THREADS),
                          amdgpu_waves_per_eu(1)))
void attn_kernel(AttnArgs a) {
  using C = AttnCfg<D, BLK>;
  __shared__ __align__(16) uint16_t Ks[BLK * D];
  __shared__ __align__(16) uint16_t Vt[(MODE == MODE_TILE_MAX) ? 8 : D * BLK];
  __shared__ int rowid[BLK];
  __shared__ float red[C::WAVES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int w = blockIdx.x;
  const int I = a.NB - 1 - w / a.Hq;  // longest rows first
  const int h = w % a.Hq;
  const int g = h / a.G;
  const int I0 = I * BLK;
  const int qloc = wave * 32 + l32;
  const int qpos = I0 + qloc;
  const bool qvalid = qpos < a.N;
  const size_t ntri = (size_t)a.NB * (a.NB + 1) / 2;

  const rsrc_t qr = make_rsrc(a.q + (int64_t)h * a.qsh, a.q_bytes);
  const rsrc_t kr = make_rsrc(a.k + (int64_t)g * a.kvsh, a.kv_bytes);
  const rsrc_t vr = make_rsrc(a.v + (int64_t)g * a.kvsh, a.kv_bytes);

  // Q fragment of this lane: B operand (column = query qloc) for every k-step of S^T = K Q^T.
  bf16x8 qf[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    const uint32_t off = qvalid ? (uint32_t)qpos * a.q_row_bytes + kk * 32 + h2 * 16 : kOutOfRange;
    qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(qr, off));
  }

  int cnt = I + 1;
  const int32_t* list = nullptr;
  if (MODE != MODE_TILE_MAX && a.count != nullptr) {
    cnt = a.count[(size_t)h * a.NB + I];
    list = a.idx + (size_t)h * ntri + tri_offset(I);
    if (cnt < 0 || cnt > I + 1) {
      if (t == 0 && a.err) atomicOr(a.err, 4);
      cnt = cnt < 0 ? 0 : I + 1;
    }
  }
  const int sI = a.S > 0 ? I0 / a.S : 0;

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int it = 0; it < cnt; ++it) {
    const int J = list ? list[it] : it;
    if (J < 0 || J > I) {
      if (t == 0 && a.err) atomicOr(a.err, 1);
      continue;
    }
    const bool diag = (J == I);
    const bool permuted = a.perm != nullptr && a.S > 0 && (J * BLK) / a.S < sI;
    __syncthreads();  // every wave is done with the previous tile's LDS
    if (t < BLK) {
      const int p = J * BLK + t;
      int r = -1;
      if (p < a.N) {
        r = permuted ? a.perm[(size_t)g * a.N + p] : p;
        if (r < 0 || r >= a.N) {
          if (a.err) atomicOr(a.err, 2);
          r = -1;
        }
      }
      rowid[t] = r;
    }
    __syncthreads();
    load_k_tile<D, BLK>(Ks, kr, a.kv_row_bytes, rowid);
    if (MODE == MODE_ATTN) load_v_tile<D, BLK>(Vt, vr, a.kv_row_bytes, rowid);
    __syncthreads();

    f32x16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int row = kb * 32 + l32;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + row * D + (((kk * 2 + h2) ^ k_swz<D>(row)) * 8));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // bound how far LDS operand reads are hoisted
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (diag && key > qloc) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));

    if (MODE == MODE_TILE_MAX || (MODE == MODE_ATTN_GATED && !diag)) {
      float tm = wave_max_f32(qvalid ? mx : -INFINITY);
      if (lane == 0) red[wave] = tm;
      __syncthreads();
      tm = red[0];
#pragma unroll
      for (int x = 1; x < C::WAVES; ++x) tm = fmaxf(tm, red[x]);
      if (MODE == MODE_TILE_MAX) {
        if (t == 0) a.tmax[(size_t)h * ntri + tri_offset(I) + J] = tm * a.scale;
        continue;
      }
      if (tm * a.scale < a.theta[(size_t)h * a.NB + I]) continue;  // gate: no V load, no PV
    }
    if (MODE == MODE_ATTN_GATED) {
      load_v_tile<D, BLK>(Vt, vr, a.kv_row_bytes, rowid);
      __syncthreads();
    }
    if (MODE != MODE_TILE_MAX) {
      if (a.kept && t == 0) {
        const size_t bit = tri_offset(I) + J;
        const size_t words = (ntri + 31) / 32;
        atomicOr(&a.kept[(size_t)h * words + bit / 32], 1u << (bit % 32));
      }
      const float m_new = fmaxf(m_run, mx * a.sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      m_run = m_new;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, -m_use));
          l_run += p;
          pb[r >> 3][r & 7] = (__bf16)p;
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int d = db * 32 + l32;
            const int c = kb * 4 + hf * 2 + h2;
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + d * BLK + ((c ^ v_swz<BLK>(d)) * 8));
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[hf], o[db], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  if (MODE == MODE_TILE_MAX) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    float* orow = a.out + (int64_t)h * a.osh + (int64_t)qpos * a.ost;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = o[db][rq * 4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * rq + 4 * h2) = val;
      }
    if (a.lse && h2 == 0)
      a.lse[(size_t)h * a.N + qpos] = l_tot > 0.f ? m_run * 0.69314718055994531f + logf(l_tot) : -INFINITY;
  }
}

template <int D, int BLK, int MODE>
static hipError_t launch_mode(const AttnArgs& a, int nwg, hipStream_t st) {
  attn_kernel<D, BLK, MODE><<<nwg, AttnCfg<D, BLK>::THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t dispatch(const Geometry& g, const AttnArgs& a, hipStream_t st) {
  const int nwg = g.Hq * g.NB;
  if (g.d == 128 && g.B == 128) return launch_mode<128, 128, MODE>(a, nwg, st);
  if (g.d == 128 && g.B == 64) return launch_mode<128, 64, MODE>(a, nwg, st);
  if (g.d == 64 && g.B == 128) return launch_mode<64, 128, MODE>(a, nwg, st);
  return launch_mode<64, 64, MODE>(a, nwg, st);
}

static AttnArgs make_args(const Geometry& g) {
  AttnArgs a = {};
  a.N = g.N;
  a.Hq = g.Hq;
  a.G = g.G;
  a.S = g.S;
  a.NB = g.NB;
  a.qsh = g.qsh;
  a.kvsh = g.kvsh;
  a.q_row_bytes = (uint32_t)(g.qst * 2);
  a.kv_row_bytes = (uint32_t)(g.kvst * 2);
  a.q_bytes = (uint32_t)((int64_t)g.N * g.qst * 2);
  a.kv_bytes = (uint32_t)((int64_t)g.N * g.kvst * 2);
  a.osh = g.osh;
  a.ost = g.ost;
  a.scale = g.scale;
  a.sl2 = g.scale * 1.4426950408889634f;
  return a;
}

hipError_t launch_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* perm, const int32_t* count, const int32_t* idx,
                            const float* theta, float* out, float* lse, uint32_t* kept, int32_t* err,
                            hipStream_t st) {
  AttnArgs a = make_args(g);
  a.q = q;
  a.k = k;
  a.v = v;
  a.perm = perm;
  a.count = count;
  a.idx = idx;
  a.theta = theta;
  a.out = out;
  a.lse = lse;
  a.kept = kept;
  a.err = err;
  if (theta) return dispatch<MODE_ATTN_GATED>(g, a, st);
  return dispatch<MODE_ATTN>(g, a, st);
}

hipError_t launch_tile_max(const Geometry& g, const uint16_t* q, const uint16_t* k, float* tmax, hipStream_t st) {
  AttnArgs a = make_args(g);
  a.q = q;
  a.k = k;
  a.v = k;
  a.tmax = tmax;
  a.S = 0;
  return dispatch<MODE_TILE_MAX>(g, a, st);
}

}  // namespace pbsa
