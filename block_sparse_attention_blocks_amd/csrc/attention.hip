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
  static constexpr int KT = 64;                        // keys per pipelined LDS stage
  static constexpr int STAGES = BLK / KT;              // stages per key block
};

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
  float gain_tau;             // marginal-gain early stop threshold (S2O kernels)
  unsigned long long* queue;  // work deques of the pipelined kernels (workspace)
  int nq;                     // number of deques: one per KV group, at most one per XCD
  int Hkv;
  int two_pass;               // S2O kernels: two-pass lists over the per-segment prefix order kvr
  const int32_t* kvr;         // per-segment prefix key order (NULL when no segment has a prefix)
  int64_t kvr_L;              // entries of kvr per KV head
  const int32_t* qperm;       // two-pass lists: query order inside segments [Hkv][N], or NULL
};

enum { MODE_ATTN = 0, MODE_ATTN_GATED = 1, MODE_TILE_MAX = 2, MODE_DENSE = 3 };

// ---------------------------------------------------------------------------------------------
// Pipelined kernel.  K and V tiles are gathered straight from HBM into LDS by the buffer unit
// (buffer_load_dwordx4 ... lds: lane i of a wave fills bytes [16 i, 16 i + 16) of a 1 KiB LDS
// window, from any global address it chooses), so the gather needs no registers and no VALU.
// Both tiles keep the natural [key][d] layout with a per-row XOR swizzle of the 16-byte chunks,
// chosen through the per-lane source addresses.  K feeds S^T = K Q^T with 16-byte reads; V feeds
// O^T = V^T P^T through ds_read_b64_tr_b16, which transposes 16-bit data across each 16-lane
// group: lane i receives element e = M[4e + i/4][i%4] of the 4-element rows M[j] addressed by
// lanes j.  Pointing lane j at V[k0 + j/4][d0 + 4 (j%4) ...] hands lane i the four keys
// k0..k0+3 of column d0 + i.
// ---------------------------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int D>
__device__ __forceinline__ int kt_swz(int row) {  // K tile: 16 consecutive rows hit 16 chunks
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vt_swz(int key) {  // V tile: 4 consecutive keys hit disjoint banks
  return D == 128 ? ((key & 3) << 2) : ((key & 3) << 1);
}

// Byte offset of key row r in a head's slab, or kOutOfRange (the buffer load then returns zeros).
__device__ __forceinline__ uint32_t row_offset(int r, uint32_t row_bytes) {
  return r >= 0 ? (uint32_t)r * row_bytes : kOutOfRange;
}

// A key row looked up for a later gather is kept raw (a natural position, a perm entry, or kPastEnd
// for a row past the sequence) until it is stored, so the perm load is not waited for where it is
// issued.  checked_row_offset turns it into a byte offset; a perm entry out of range sets bit 2 of
// err and reads zeros.
constexpr int kPastEnd = -2147483647 - 1;
__device__ __forceinline__ uint32_t checked_row_offset(int raw, int N, uint32_t row_bytes, int32_t* err) {
  if (raw == kPastEnd) return kOutOfRange;
  if (raw < 0 || raw >= N) {
    if (err) atomicOr(err, 2);
    return kOutOfRange;
  }
  return (uint32_t)raw * row_bytes;
}

// One pending row lookup: every lane issues the perm load (a buffer load that returns zero when the
// row is natural or unused), with no branch around it, so nothing consumes the loaded value before
// row_lookup_offset at the point where the row id is stored.
struct RowLook {
  int code;  // natural position (>= 0), kViaPerm (the row is the perm entry pv), or kPastEnd
  int pv;    // perm entry
};
constexpr int kViaPerm = -1;
__device__ __forceinline__ RowLook row_lookup(rsrc_t permr, int p, int N, bool want, bool permuted) {
  RowLook r;
  const bool live = want && p < N;
  const bool via = live && permuted;
  r.code = via ? kViaPerm : live ? p : kPastEnd;
  r.pv = (int)__builtin_amdgcn_raw_buffer_load_b32(permr, via ? (uint32_t)p * 4u : kOutOfRange, 0, 0);
  return r;
}
// plim bounds a row taken from the index map (N for perm; the segment's prefix length for the
// per-segment prefix order, so that a history row always precedes the query block's segment).
__device__ __forceinline__ uint32_t row_lookup_offset(const RowLook& r, int N, int plim, uint32_t row_bytes,
                                                      int32_t* err) {
  return checked_row_offset(r.code == kViaPerm ? r.pv : r.code, r.code == kViaPerm ? plim : N, row_bytes, err);
}

// One gathered tile: the rows at byte offsets row_off(j) of the head's slab into LDS [ROWS][D]
// with the chunk swizzle.  An offset of kOutOfRange leaves a zero row.
template <int D, int BLK, bool IS_V, typename RowFn, int ROWS = AttnCfg<D, BLK>::KT,
          int WAVES = AttnCfg<D, BLK>::WAVES>
__device__ __forceinline__ void dma_tile(uint16_t* dst, rsrc_t r, RowFn row_off) {
  constexpr int RPI = 512 / D;  // rows per 1 KiB wave instruction
  constexpr int LPR = D / 8;    // lanes per row
  constexpr int NI = ROWS / (RPI * WAVES);
  static_assert(NI * RPI * WAVES == ROWS, "tile rows must split evenly over the waves");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row0 = (wave * NI + i) * RPI;
    const int rw = row0 + lane / LPR;
    const uint32_t c = (lane % LPR) ^ (IS_V ? vt_swz<D>(rw) : kt_swz<D>(rw));
    const uint32_t off = row_off(rw) + c * 16;  // kOutOfRange + c*16 stays out of range
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + row0 * D), 16, off, 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Online-softmax state of one lane's query column (S2O section 3: m, l, acc).  m is kept in log2
// units and only moved when a block of scores exceeds it by more than kLazy: the probabilities
// are then at most 2^kLazy, well inside fp32 and bf16 range, and most steps skip the rescale.
constexpr float kLazy = 8.0f;

template <int D, int BLK>
struct SoftmaxState {
  f32x16 o[AttnCfg<D, BLK>::DB];
  float m;     // reference max, log2 units
  float l;     // sum of the bf16-rounded probabilities relative to m (this lane's half of the keys)
  float thr;   // (m + kLazy) in raw score units: a block whose raw max exceeds it moves m
  float muse;  // m, or 0 while m is -inf (no finite score yet), as the exponent offset
  float lb;    // l when the current key block started, rescaled with l (marginal-gain stop)
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < AttnCfg<D, BLK>::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    m = -INFINITY;
    l = 0.f;
    thr = -INFINITY;
    muse = 0.f;
    lb = 0.f;
  }
};

// Lazy rescale on a block's raw (unscaled) row max: when it exceeds the threshold of any lane of
// the wave, those lanes move m to the block max (log2 units) and scale l and acc by 2^(m_old - m).
template <int D, int BLK>
__device__ __forceinline__ void lazy_rescale(SoftmaxState<D, BLK>& st, float raw_max, float sl2) {
  const bool need = raw_max > st.thr;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float m_new = need ? raw_max * sl2 : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
    st.lb *= alpha;
#pragma unroll
    for (int db = 0; db < AttnCfg<D, BLK>::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= alpha;
    st.m = m_new;
    st.thr = (m_new + kLazy) / sl2;
    st.muse = (m_new == -INFINITY) ? 0.f : m_new;
  }
}

// K operands of score block kb: A operand (row = key kb*32 + l32) for every k-step of S^T = K Q^T.
template <int D, int BLK>
__device__ __forceinline__ void load_k_ops(bf16x8* kop, const uint16_t* Ks, int kb) {
  using C = AttnCfg<D, BLK>;
  const int lane = threadIdx.x & 63;
  const int krow = kb * 32 + (lane & 31), h2 = lane >> 5;
  const uint16_t* kp = Ks + krow * D;
  const int ksw = kt_swz<D>(krow);
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk)
    kop[kk] = *reinterpret_cast<const bf16x8*>(kp + (((kk * 2 + h2) ^ ksw) * 8));
}

// Causal mask of a score block on the diagonal tile: rel = query row - first key of the block -
// 4*h2, so register r holds key offset 8*(r/4) + r%4 relative to it.  The empty volatile asm keeps
// the enclosing `if (diag)` a real (uniform) branch: if-converted, the compares and selects would
// run on every block.
__device__ __forceinline__ void causal_mask(f32x16& s, int rel) {
  asm volatile("" : "+v"(rel));
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (8 * (r >> 2) + (r & 3) > rel) s[r] = -INFINITY;
  asm volatile("" : "+v"(s));  // the selects stay inside the caller's diagonal branch
}

// S^T block (32 keys x this wave's 32 queries) from preloaded K operands, with the causal mask on
// the diagonal tile.
template <int D, int BLK>
__device__ __forceinline__ f32x16 block_scores_ops(const bf16x8* kop, const bf16x8* qf, bool diag, int rel) {
  using C = AttnCfg<D, BLK>;
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[kk], s, 0, 0, 0);
  if (diag) causal_mask(s, rel);
  return s;
}

template <int D, int BLK>
__device__ __forceinline__ f32x16 block_scores(const uint16_t* Ks, const bf16x8* qf, int kb, bool diag, int rel) {
  bf16x8 kop[AttnCfg<D, BLK>::KSTEPS];
  load_k_ops<D, BLK>(kop, Ks, kb);
  return block_scores_ops<D, BLK>(kop, qf, diag, rel);
}

// V^T operands of block kb through the transposing LDS read: for half hf and d block db, keys
// kb*32 + 16 hf + 4 h2 + {0..3} then + 8 -- the keys this lane's P operand holds.
template <int D, int BLK>
__device__ __forceinline__ void load_v_ops(bf16x8* vop, const uint16_t* Vs, int kb) {
  using C = AttnCfg<D, BLK>;
  const int lane = threadIdx.x & 63;
  const int h2 = lane >> 5, i16 = lane & 15, dsub = (lane >> 4) & 1;
  typedef short s16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int key0 = kb * 32 + 16 * hf + 4 * h2 + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int dcol = db * 32 + dsub * 16 + 4 * (i16 & 3);
      const uint16_t* p0 = Vs + key0 * D + (((dcol >> 3) ^ vt_swz<D>(key0)) * 8) + (dcol & 7);
      const uint16_t* p1 = Vs + (key0 + 8) * D + (((dcol >> 3) ^ vt_swz<D>(key0 + 8)) * 8) + (dcol & 7);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
      const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      vop[hf * C::DB + db] = __builtin_bit_cast(bf16x8, both);
    }
  }
}

// Values of lanes l and l ^ 32 (the two halves of one query column) side by side.
__device__ __forceinline__ void half_swap(float x, float* a, float* b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  *a = __uint_as_float(r[0]);
  *b = __uint_as_float(r[1]);
}

// Row max of a score block over this lane's query (both half-waves), unscaled.
__device__ __forceinline__ float block_row_max(const f32x16& s) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  float a, b;
  half_swap(mx, &a, &b);
  return fmaxf(a, b);
}

// Online softmax of one 32-key score block and O^T += V^T P^T with preloaded V^T operands.
template <int D, int BLK>
__device__ __forceinline__ void block_softmax_pv_ops(SoftmaxState<D, BLK>& st, const f32x16& s, const bf16x8* vop,
                                                     float sl2) {
  using C = AttnCfg<D, BLK>;
  lazy_rescale<D, BLK>(st, block_row_max(s), sl2);
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pb[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) pb[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[r], sl2, -st.muse));
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 pair = {pb[hf][2 * e], pb[hf][2 * e + 1]};
      st.l = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, st.l, false);
    }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[hf * C::DB + db], pb[hf], st.o[db], 0, 0, 0);
}

template <int D, int BLK>
__device__ __forceinline__ void block_softmax_pv(SoftmaxState<D, BLK>& st, const f32x16& s, const uint16_t* Vs,
                                                 int kb, float sl2) {
  bf16x8 vop[2 * AttnCfg<D, BLK>::DB];
  load_v_ops<D, BLK>(vop, Vs, kb);
  block_softmax_pv_ops<D, BLK>(st, s, vop, sl2);
}

// One KT-key stage from LDS: for each 32-key block, the V operands of this block and the K
// operands of the next are read while the scores and softmax of this block are computed.  kop0
// holds the K operands of block 0, read by the caller as soon as the stage buffer was ready.
template <int D, int BLK>
__device__ __forceinline__ void stage_compute(SoftmaxState<D, BLK>& st, const uint16_t* Kc, const uint16_t* Vc,
                                              const bf16x8* qf, const bf16x8* kop0, bool diag, int rel0,
                                              float sl2) {
  using C = AttnCfg<D, BLK>;
  constexpr int NKB = C::KT / 32;
  bf16x8 kop[C::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) kop[kk] = kop0[kk];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    bf16x8 vop[2 * C::DB];
    load_v_ops<D, BLK>(vop, Vc, kb);
    const f32x16 sc = block_scores_ops<D, BLK>(kop, qf, diag, rel0 - kb * 32);
    if (kb + 1 < NKB) load_k_ops<D, BLK>(kop, Kc, kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    block_softmax_pv_ops<D, BLK>(st, sc, vop, sl2);
  }
}

template <int D, int BLK>
__device__ __forceinline__ void write_output(const AttnArgs& a, const SoftmaxState<D, BLK>& st, int h, int qpos,
                                             bool qvalid, int h2) {
  using C = AttnCfg<D, BLK>;
  float la, lb;
  half_swap(st.l, &la, &lb);
  const float l_tot = la + lb;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!qvalid) return;
  float* orow = a.out + (int64_t)h * a.osh + (int64_t)qpos * a.ost;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      f32x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = st.o[db][rq * 4 + e] * inv;
      *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * rq + 4 * h2) = val;
    }
  if (a.lse && h2 == 0)
    a.lse[(size_t)h * a.N + qpos] = l_tot > 0.f ? st.m * 0.69314718055994531f + logf(l_tot) : -INFINITY;
}

// Pipelined kernel configuration: HPW query heads of one KV group per workgroup (WAVES_PER_HEAD
// waves of 32 query rows each), KT-key LDS stages, NBUF stage buffers.
template <int D, int BLK, int HPW>
struct PipeCfg {
  static constexpr int WAVES_PER_HEAD = BLK / 32;
  static constexpr int WAVES = HPW * WAVES_PER_HEAD;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KT = AttnCfg<D, BLK>::KT;
  static constexpr int STAGES = BLK / KT;
  static constexpr int NBUF = HPW == 1 ? 2 : 3;  // one workgroup per CU has room for three
  static constexpr int RING = NBUF;              // row-id slots: stage y uses slot y % NBUF
  static constexpr int NDMA = 2 * KT / ((512 / D) * WAVES);  // gather instructions per wave per stage
  static constexpr int MAXNB = 2048;
};

// Workgroup -> (query block I, first query head h).  Rows with more key blocks (larger I) go first.
// The dispatcher deals workgroups to the 8 XCDs round-robin (w % 8) and each XCD has its own L2;
// when the head units divide by 8, XCD x gets a contiguous range of query heads, so the heads of a
// KV group run side by side on one XCD and reuse the gathered K/V tiles in its L2.
__device__ __forceinline__ void work_item(int NB, int units, int hpw, int w, int* I, int* h) {
  int u;
  if ((units & 7) == 0) {
    const int up = units >> 3, r = w >> 3;
    *I = NB - 1 - r / up;
    u = (w & 7) * up + r % up;
  } else {
    *I = NB - 1 - w / units;
    u = w % units;
  }
  *h = u * hpw;
}

__device__ __forceinline__ void work_item(const AttnArgs& a, int w, int* I, int* h) {
  work_item(a.NB, a.Hq, 1, w, I, h);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier of the pipelined loops: this wave's LDS operations complete, then s_barrier.
// __syncthreads() would also drain every outstanding global load, including the stage gathers
// issued for later stages; here each wave first waits (wait_vmcnt) only for the gathers of the
// stage about to be read, so the later ones stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Union of the kept key-block lists of query heads h0 .. h0+HPW-1 for query block I, in ascending
// J, into mlist as J | (bit 16 + x set when head h0 + x kept J).  Returns the list length.  Mask
// entries out of range are skipped and flagged in a.err.
template <int HPW, int THREADS>
__device__ __forceinline__ int union_list(const AttnArgs& a, int h0, int I, size_t ntri, uint8_t* selb, uint32_t* mlist,
                                          int* mcount) {
  constexpr int MAXNB = PipeCfg<128, 128, 1>::MAXNB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int J = t; J <= I; J += THREADS)
#pragma unroll
    for (int x = 0; x < HPW; ++x) selb[x * MAXNB + J] = 0;
  __syncthreads();
#pragma unroll
  for (int x = 0; x < HPW; ++x) {
    int cnt = a.count[(size_t)(h0 + x) * a.NB + I];
    if (cnt < 0 || cnt > I + 1) {
      if (t == 0 && a.err) atomicOr(a.err, 4);
      cnt = cnt < 0 ? 0 : I + 1;
    }
    const int32_t* list = a.idx + (size_t)(h0 + x) * ntri + tri_offset(I);
    for (int k = t; k < cnt; k += THREADS) {
      const int J = list[k];
      if (J >= 0 && J <= I) {
        selb[x * MAXNB + J] = 1;
      } else if (a.err) {
        atomicOr(a.err, 1);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    int base = 0;
    for (int J0 = 0; J0 <= I; J0 += 64) {
      const int J = J0 + lane;
      uint32_t bits = 0;
      if (J <= I) {
#pragma unroll
        for (int x = 0; x < HPW; ++x) bits |= (uint32_t)selb[x * MAXNB + J] << (16 + x);
      }
      const unsigned long long bal = __ballot(bits != 0);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (bits) mlist[pos] = (uint32_t)J | bits;
      base += __popcll(bal);
    }
    if (lane == 0) *mcount = base;
  }
  __syncthreads();
  return *mcount;
}

// The ranked key-block list of one head (marginal-gain early stop), kept in its order, into mlist
// as J | head bit.  An entry out of range is flagged in a.err and kept without the head bit, so its
// stage is gathered but not computed.  Returns the list length.
template <int THREADS>
__device__ __forceinline__ int ranked_list(const AttnArgs& a, int h, int I, size_t ntri, uint32_t* mlist,
                                           int* mcount) {
  const int t = threadIdx.x;
  if (t == 0) {
    int cnt = a.count[(size_t)h * a.NB + I];
    if (cnt < 0 || cnt > I + 1) {
      if (a.err) atomicOr(a.err, 4);
      cnt = cnt < 0 ? 0 : I + 1;
    }
    *mcount = cnt;
  }
  __syncthreads();
  const int cnt = *mcount;
  const int32_t* list = a.idx + (size_t)h * ntri + tri_offset(I);
  for (int k = t; k < cnt; k += THREADS) {
    const int J = list[k];
    const bool ok = J >= 0 && J <= I;
    if (!ok && a.err) atomicOr(a.err, 1);
    mlist[k] = ok ? ((uint32_t)J | (1u << 16)) : 0u;
  }
  __syncthreads();
  return cnt;
}

// The two-pass list of S2O (Kernel Implementation) for a query block of the segment that starts at
// block J0: pass 1, the own segment's blocks J0 .. Jend ascending (Jend = I in natural query order,
// the segment's last block when queries are permuted); pass 2, blocks 0 .. J0-1 of the segment's
// prefix key order (block J = ranked keys J*B .. J*B+B-1).  Returns the list length, Jend + 1.
template <int THREADS>
__device__ __forceinline__ int two_pass_list(int Jend, int J0, uint32_t* mlist) {
  const int nin = Jend + 1 - J0;
  for (int x = threadIdx.x; x <= Jend; x += THREADS)
    mlist[x] = (uint32_t)(x < nin ? J0 + x : x - nin) | (1u << 16);
  __syncthreads();
  return Jend + 1;
}

// ---------------------------------------------------------------------------------------------
// Work distribution of the pipelined kernels.  A work item is one query block I for one unit of
// HPW query heads.  Deque q holds, in order of descending I, the items of the KV groups g with
// g % nq == q (nq = min(8, Hkv)), so the items of one KV group share a deque and, through it, one
// XCD's L2.  A persistent workgroup reads the XCD it runs on from the hardware, takes items from
// the front of that XCD's deque (longest rows first), and once it is empty takes the shortest
// remaining items from the back of the other deques: the XCDs finish together even when the KV
// groups keep very different numbers of blocks.
//
// Each deque is one 64-bit word, front index in the low half and back index in the high half,
// changed only by atomic adds: +1 claims the front item f if f < b in the returned word, -2^32
// claims the back item b-1 if b-1 >= f.  Every add sees one consistent (f, b), the two ends only
// move towards each other, so no item is claimed twice and a workgroup that finds every deque
// empty can stop.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int deque_items(const AttnArgs& a, int q, int units_per_group) {
  const int groups = (a.Hkv - q + a.nq - 1) / a.nq;
  return a.NB * groups * units_per_group;
}

__global__ __launch_bounds__(64) void deque_init_kernel(AttnArgs a, int units_per_group) {
  const int q = threadIdx.x;
  if (q < a.nq) a.queue[q] = (unsigned long long)deque_items(a, q, units_per_group) << 32;
}

// item code (q << 24 | index) or -1 when every deque is empty
__device__ __forceinline__ int claim_item(const AttnArgs& a, int home) {
  unsigned long long old = atomicAdd(&a.queue[home], 1ull);
  int f = (int)(uint32_t)old, b = (int)(uint32_t)(old >> 32);
  if (f < b) return (home << 24) | f;
  for (int k = 1; k < a.nq; ++k) {
    const int q = home + k < a.nq ? home + k : home + k - a.nq;
    old = atomicAdd(&a.queue[q], 0xFFFFFFFF00000000ull);
    f = (int)(uint32_t)old;
    b = (int)(uint32_t)(old >> 32);
    if (b >= 1 && b - 1 >= f) return (q << 24) | (b - 1);
  }
  return -1;
}

// item code -> (query block I, first query head h0)
__device__ __forceinline__ void item_work(const AttnArgs& a, int code, int hpw, int units_per_group, int* I,
                                          int* h0) {
  const int q = code >> 24, i = code & 0xffffff;
  const int groups = (a.Hkv - q + a.nq - 1) / a.nq;
  const int per_I = groups * units_per_group;
  *I = a.NB - 1 - i / per_I;
  const int j = i % per_I;
  const int g = q + a.nq * (j / units_per_group);
  *h0 = (g * units_per_group + j % units_per_group) * hpw;
}

__device__ __forceinline__ int xcd_id() { return (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 0xfu); }

// Software-pipelined block-sparse (DENSE = false) or dense causal (DENSE = true) attention for
// HPW query heads h0 .. h0+HPW-1 of one KV group and one query block I.  The workgroup walks the
// union of the heads' kept key blocks in ascending order; each KT-key stage of a block is gathered
// once into LDS and used by the waves of every head that kept the block (the query heads of a
// group usually keep nearly the same blocks).  While stage s is computed, stages s+1 .. s+NBUF-1
// are in flight, and the physical row ids of stage s+NBUF are fetched from perm.
//
// S2O = true (one head per workgroup): the list is the head's ranked list, taken in its order, and
// after every earlier-segment block the workgroup stops the row when each query's share of that
// block in its softmax denominator is below a.gain_tau (S2O, Early-Stopping Rule).
template <int D, int BLK, bool DENSE, int HPW, bool S2O = false>
__global__ __attribute__((amdgpu_flat_work_group_size(PipeCfg<D, BLK, HPW>::THREADS, PipeCfg<D, BLK, HPW>::THREADS),
                          amdgpu_waves_per_eu(2)))
void attn_pipe_kernel(AttnArgs a) {
  static_assert(!S2O || (HPW == 1 && !DENSE), "the marginal-gain stop runs one head per workgroup");
  using C = PipeCfg<D, BLK, HPW>;
  constexpr int KT = C::KT;
  constexpr int NBUF = C::NBUF;
  // stage buffers as distinct LDS objects, so reads of one are not ordered behind the gathers still
  // filling the others
  __shared__ __align__(16) uint16_t K0[KT * D];
  __shared__ __align__(16) uint16_t K1[KT * D];
  __shared__ __align__(16) uint16_t K2[NBUF > 2 ? KT * D : 8];
  __shared__ __align__(16) uint16_t K3[NBUF > 3 ? KT * D : 8];
  __shared__ __align__(16) uint16_t V0[KT * D];
  __shared__ __align__(16) uint16_t V1[KT * D];
  __shared__ __align__(16) uint16_t V2[NBUF > 2 ? KT * D : 8];
  __shared__ __align__(16) uint16_t V3[NBUF > 3 ? KT * D : 8];
  __shared__ uint32_t rowid[DENSE ? 1 : C::RING][KT];  // byte offsets of the gathered rows
  __shared__ uint32_t mlist[DENSE ? 1 : C::MAXNB];  // J | kept-by-head bits << 16
  __shared__ uint8_t selb[DENSE ? 1 : HPW * C::MAXNB];
  __shared__ int mcount;
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stage buffers");
  auto Kb = [&](int b) __attribute__((always_inline)) -> uint16_t* {
    return b == 0 ? K0 : b == 1 ? K1 : b == 2 ? K2 : K3;
  };
  auto Vb = [&](int b) __attribute__((always_inline)) -> uint16_t* {
    return b == 0 ? V0 : b == 1 ? V1 : b == 2 ? V2 : V3;
  };

  __shared__ int item_sh;
  __shared__ int stop_flag[2][S2O ? C::WAVES : 1];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int hh = wave / C::WAVES_PER_HEAD;   // this wave's head within the workgroup
  const int wq = wave % C::WAVES_PER_HEAD;   // this wave's 32-row slice of the query block
  const int upg = a.G / HPW;                 // head units per KV group
  const int home = xcd_id() % a.nq;

  // stage buffers start finite (zero); rows a gather leaves unwritten keep finite older data, and
  // keys past N only occur in the last diagonal block, where the causal mask removes them
  {
    constexpr int NZ = KT * D * 2 / 16;
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    for (int i = t; i < NZ; i += C::THREADS)
#pragma unroll
      for (int b = 0; b < NBUF; ++b) {
        reinterpret_cast<u32x4*>(Kb(b))[i] = z;
        reinterpret_cast<u32x4*>(Vb(b))[i] = z;
      }
  }

  for (;;) {
  if (t == 0) item_sh = claim_item(a, home);
  __syncthreads();
  const int code = item_sh;
  if (code < 0) break;
  int I, h0;
  item_work(a, code, HPW, upg, &I, &h0);
  const int h = h0 + hh;
  const int g = h0 / a.G;
  const int I0 = I * BLK;
  const int qloc = wq * 32 + l32;
  const int qpos = I0 + qloc;  // slot of this lane's query in the (possibly permuted) order
  const int sI = a.S > 0 ? I0 / a.S : 0;
  const bool two_pass = S2O && a.two_pass;  // history through the segment's prefix order
  const bool qperm_on = two_pass && a.qperm != nullptr;
  const int J0 = sI * a.S / BLK;             // first block of the query block's segment
  bool qvalid = qpos < a.N;
  int qnat = qpos;  // natural position of the query (its causal limit and output row)
  if (qperm_on && qvalid) {
    const int v = a.qperm[(size_t)g * a.N + qpos];
    if (v < sI * a.S || v >= min((sI + 1) * a.S, a.N)) {  // not a position of this segment
      if (a.err) atomicOr(a.err, 8);
      qvalid = false;
    } else {
      qnat = v;
    }
  }
  const size_t ntri = (size_t)a.NB * (a.NB + 1) / 2;
  const rsrc_t qr = make_rsrc(a.q + (int64_t)h * a.qsh, a.q_bytes);
  const rsrc_t kr = make_rsrc(a.k + (int64_t)g * a.kvsh, a.kv_bytes);
  const rsrc_t vr = make_rsrc(a.v + (int64_t)g * a.kvsh, a.kv_bytes);

  bf16x8 qf[AttnCfg<D, BLK>::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < AttnCfg<D, BLK>::KSTEPS; ++kk) {
    const uint32_t off = qvalid ? (uint32_t)qnat * a.q_row_bytes + kk * 32 + h2 * 16 : kOutOfRange;
    qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(qr, off));
  }

  // merged key-block list: ascending J kept by any of the workgroup's heads
  const int Jend = qperm_on ? min((min((sI + 1) * a.S, a.N) + BLK - 1) / BLK, a.NB) - 1 : I;
  const int nblk = DENSE     ? I + 1
                   : two_pass ? two_pass_list<C::THREADS>(Jend, J0, mlist)
                   : S2O      ? ranked_list<C::THREADS>(a, h0, I, ntri, mlist, &mcount)
                              : union_list<HPW, C::THREADS>(a, h0, I, ntri, selb, mlist, &mcount);
  const int nst = nblk * C::STAGES;
  const uint32_t all_heads = ((1u << HPW) - 1u) << 16;
  auto entry_of = [&](int s) -> uint32_t {  // wave-uniform
    const int u = s / C::STAGES;
    return DENSE ? ((uint32_t)u | all_heads) : (uint32_t)__builtin_amdgcn_readfirstlane(mlist[u]);
  };
  // index map of the history rows: perm of the KV head, or segment sI's prefix order
  const int plim = two_pass ? sI * a.S : a.N;
  const int32_t* pbase = two_pass ? (sI > 0 ? a.kvr + (size_t)g * a.kvr_L + (size_t)a.S * sI * (sI - 1) / 2 : nullptr)
                         : a.perm ? a.perm + (size_t)g * a.N
                                  : nullptr;
  const rsrc_t permr = make_rsrc(pbase, pbase ? (uint32_t)plim * 4u : 0u);
  const bool mapped = a.perm != nullptr || two_pass;
  // lookup of row j of stage s (want = false: an unused lookup that reads nothing)
  auto lookup = [&](int s, int j, bool want) -> RowLook {
    const int J = (int)(entry_of(s) & 0xffffu);
    const int p = J * BLK + (s % C::STAGES) * KT + j;
    return row_lookup(permr, p, a.N, want, !DENSE && mapped && a.S > 0 && (J * BLK) / a.S < sI);
  };
  auto row_off = [&](const RowLook& r) { return row_lookup_offset(r, a.N, plim, a.kv_row_bytes, a.err); };
  // next row lookup, of stage x (issued one step before its row ids are stored)
  auto lookup_ahead = [&](int x) -> RowLook { return lookup(x < nst ? x : 0, t & (KT - 1), x < nst && t < KT); };
  // gather stage s into buffer b = s % NBUF (b is passed separately so that it folds to a constant)
  auto gather = [&](int s, int b) __attribute__((always_inline)) {
    uint16_t* Kd = Kb(b);
    uint16_t* Vd = Vb(b);
    if (DENSE) {
      auto rf = [&](int j) { return row_off(lookup(s, j, true)); };
      dma_tile<D, BLK, false, decltype(rf), KT, C::WAVES>(Kd, kr, rf);
      dma_tile<D, BLK, true, decltype(rf), KT, C::WAVES>(Vd, vr, rf);
    } else {
      const uint32_t* ids = rowid[b];
      auto rf = [&](int j) { return ids[j]; };
      dma_tile<D, BLK, false, decltype(rf), KT, C::WAVES>(Kd, kr, rf);
      dma_tile<D, BLK, true, decltype(rf), KT, C::WAVES>(Vd, vr, rf);
    }
  };

  SoftmaxState<D, BLK> st;
  st.init();

  RowLook pr_prev = RowLook{kPastEnd, 0};  // lookup of stage s + NBUF, issued in step s - 1
  if (nst > 0) {
    if (!DENSE && t < KT)
      for (int x = 0; x < NBUF && x < nst; ++x) rowid[x][t] = row_off(lookup(x, t, true));
    if (!DENSE) pr_prev = lookup_ahead(NBUF);
    __syncthreads();  // zero fill and row ids visible
#pragma unroll
    for (int x = 0; x < NBUF - 1; ++x)
      if (x < nst) gather(x, x);
    wait_vmcnt<0>();
    __syncthreads();
  }

  // One pipeline step: compute stage s while stages s+1 .. s+NBUF-2 are in flight and stage
  // s+NBUF-1 is gathered into the buffer of stage s-1.  The row ids of stage s+NBUF are stored from
  // the lookup issued one step earlier, and the lookup of stage s+NBUF+1 is issued.
  constexpr int LOOK = DENSE ? 0 : 1;  // lookup loads per wave per step
  auto step = [&](int s, int b) __attribute__((always_inline)) -> bool {  // b = s % NBUF
    const uint16_t* Kc = Kb(b);
    const uint16_t* Vc = Vb(b);
    // the first K operands of this stage are read right after the barrier that made the stage
    // ready, so their LDS latency passes while the lookups and gathers below are issued (a stage
    // this head skips reads them for nothing)
    bf16x8 kop0[AttnCfg<D, BLK>::KSTEPS];
    load_k_ops<D, BLK>(kop0, Kc, 0);
    RowLook pr_next;
    if (!DENSE) pr_next = lookup_ahead(s + NBUF + 1);
    __builtin_amdgcn_sched_barrier(0);  // the lookup is issued before the gathers (vmcnt order)
    const bool issue = s + NBUF - 1 < nst;
    if (issue) gather(s + NBUF - 1, (b + NBUF - 1) % NBUF);
    const uint32_t e = s < nst ? entry_of(s) : 0u;
    if ((e >> (16 + hh)) & 1u) {
      const int J = (int)(e & 0xffffu);
      const int koff = (s % C::STAGES) * KT;  // first key of this stage inside block J
      if (a.kept && lane == 0 && wq == 0 && (s % C::STAGES) == 0) {
        // row (h, I) of the kept bitmap: packed triangle, or NB bits per row with permuted queries
        const size_t bit = qperm_on ? (size_t)I * a.NB + J : tri_offset(I) + J;
        const size_t words = qperm_on ? ((size_t)a.NB * a.NB + 31) / 32 : (ntri + 31) / 32;
        atomicOr(&a.kept[(size_t)h * words + bit / 32], 1u << (bit % 32));
      }
      if (S2O && (s % C::STAGES) == 0) st.lb = st.l;  // a new key block starts
      // causal mask: on the diagonal tile, or on every own-segment tile when queries are permuted
      // (key j is visible to the query at natural position qnat iff j <= qnat)
      stage_compute<D, BLK>(st, Kc, Vc, qf, kop0, qperm_on ? J >= J0 : J == I,
                            (qperm_on ? qnat - J * BLK : qloc) - koff - 4 * h2, a.sl2);
      if (S2O && (s % C::STAGES) == C::STAGES - 1) {
        // this block's share of each query's denominator (both half-waves of the query summed)
        float la, lbh, da, db;
        half_swap(st.l, &la, &lbh);
        half_swap(st.l - st.lb, &da, &db);
        const bool small = !qvalid || (da + db < a.gain_tau * (la + lbh));
        const bool wave_small = __builtin_amdgcn_ballot_w64(small) == ~0ull;  // taken by the whole wave
        if (lane == 0) stop_flag[(s / C::STAGES) & 1][wave] = wave_small;
      }
    }
    if (!DENSE && s + NBUF < nst && t < KT) rowid[b][t] = row_off(pr_prev);  // slot of stage s+NBUF
    if (!DENSE) pr_prev = pr_next;
    // stage s + 1 must have landed; the loads of the NBUF - 2 newer steps may stay in flight
    if (issue) {
      wait_vmcnt<(NBUF - 2) * (C::NDMA + LOOK)>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (S2O && s < nst && (s % C::STAGES) == C::STAGES - 1) {
      // after an earlier-segment block: stop when every wave found its share below the threshold
      const uint32_t e2 = entry_of(s);
      const int J = (int)(e2 & 0xffffu);
      if (((e2 >> 16) & 1u) && a.S > 0 && (J * BLK) / a.S < sI) {
        bool all = true;
#pragma unroll
        for (int x = 0; x < C::WAVES; ++x) all = all && stop_flag[(s / C::STAGES) & 1][x];
        return all;
      }
    }
    return false;
  };
  // every trip runs all NBUF steps (the ones past the end only wait and synchronise), so the
  // pending lookup passes from step to step without a copy that would wait for it
  if constexpr (S2O) {
    bool stopped = false;
    for (int s = 0; s < nst && !stopped; s += NBUF) {
#pragma unroll
      for (int x = 0; x < NBUF; ++x) {
        if (step(s + x, x)) {
          stopped = true;
          break;
        }
      }
    }
    if (stopped) wait_vmcnt<0>();  // gathers already issued for later stages land before reuse
  } else {
    for (int s = 0; s < nst; s += NBUF) {
#pragma unroll
      for (int x = 0; x < NBUF; ++x) step(s + x, x);
    }
  }
  write_output<D, BLK>(a, st, h, qnat, qvalid, h2);
  __syncthreads();  // every wave is done with this item's LDS before the next claim
  }
}

// Score block kb of a tile (S^T, 32 keys x 32 queries) with K operands read from LDS a quarter of
// the k-steps at a time (fewer live registers than load_k_ops), causal mask on the diagonal.
template <int D, int BLK>
constexpr int tile_kq() { return AttnCfg<D, BLK>::KSTEPS >= 4 ? AttnCfg<D, BLK>::KSTEPS / 4 : 1; }

// The first operand batch of score block 0 of a tile (read early by the caller).
template <int D, int BLK>
__device__ __forceinline__ void tile_first_ops(const uint16_t* Ks, bf16x8* kop) {
  const int lane = threadIdx.x & 63;
  const int krow = lane & 31, h2 = lane >> 5;
  const uint16_t* kp = Ks + krow * D;
  const int ksw = kt_swz<D>(krow);
#pragma unroll
  for (int kk = 0; kk < tile_kq<D, BLK>(); ++kk) kop[kk] = *reinterpret_cast<const bf16x8*>(kp + (((kk * 2 + h2) ^ ksw) * 8));
}

template <int D, int BLK>
__device__ __forceinline__ f32x16 tile_scores(const uint16_t* Ks, const bf16x8* qf, int kb, bool diag, int rel,
                                              const bf16x8* first = nullptr) {
  using C = AttnCfg<D, BLK>;
  constexpr int KQ = tile_kq<D, BLK>();  // k-steps per operand batch
  const int lane = threadIdx.x & 63;
  const int krow = kb * 32 + (lane & 31), h2 = lane >> 5;
  const uint16_t* kp = Ks + krow * D;
  const int ksw = kt_swz<D>(krow);
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int k0 = 0; k0 < C::KSTEPS; k0 += KQ) {
    bf16x8 kop[KQ];
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk)
      kop[kk] = (first && k0 == 0) ? first[kk] : *reinterpret_cast<const bf16x8*>(kp + ((((k0 + kk) * 2 + h2) ^ ksw) * 8));
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qf[k0 + kk], s, 0, 0, 0);
  }
  if (diag) causal_mask(s, rel);
  return s;
}

// Row max over a whole key tile (KB score blocks) of this lane's query, both half-waves, unscaled.
template <int KB>
__device__ __forceinline__ float tile_row_max(const f32x16* s) {
  float mx = s[0][0];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  float x, y;
  half_swap(mx, &x, &y);
  return fmaxf(x, y);
}

// Online-softmax update with a whole kept tile: one lazy rescale on the tile's row max, then the
// bf16 probabilities of all its keys (pb[2 kb + hf] holds registers 8 hf .. 8 hf + 7 of score
// block kb) and their sum.  The PV product with pb is issued separately (tile_pv).
template <int D, int BLK>
__device__ __forceinline__ void tile_softmax(SoftmaxState<D, BLK>& st, const f32x16* s, float row_max, bf16x8* pb,
                                             float sl2) {
  using C = AttnCfg<D, BLK>;
  lazy_rescale<D, BLK>(st, row_max, sl2);
  const float m_use = st.muse;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) pb[2 * kb + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -m_use));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2 pair = {pb[2 * kb + hf][2 * e], pb[2 * kb + hf][2 * e + 1]};
        st.l = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, st.l, false);
      }
  }
}

// O^T += V^T P^T for a whole tile from the transposed V tile in LDS.
template <int D, int BLK>
__device__ __forceinline__ void tile_pv(SoftmaxState<D, BLK>& st, const bf16x8* pb, const uint16_t* Vs) {
  using C = AttnCfg<D, BLK>;
  const int lane = threadIdx.x & 63;
  const int h2 = lane >> 5, i16 = lane & 15, dsub = (lane >> 4) & 1;
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  // one 16-key half of a score block at a time keeps the V operands to 4 DB registers
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int key0 = kb * 32 + 16 * hf + 4 * h2 + (i16 >> 2);
      bf16x8 vop[C::DB];
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const int dcol = db * 32 + dsub * 16 + 4 * (i16 & 3);
        const uint16_t* p0 = Vs + key0 * D + (((dcol >> 3) ^ vt_swz<D>(key0)) * 8) + (dcol & 7);
        const uint16_t* p1 = Vs + (key0 + 8) * D + (((dcol >> 3) ^ vt_swz<D>(key0 + 8)) * 8) + (dcol & 7);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
        const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        vop[db] = __builtin_bit_cast(bf16x8, both);
      }
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[db], pb[2 * kb + hf], st.o[db], 0, 0, 0);
    }
}

// Software-pipelined early-stop attention (Block Sparse Flash Attention, Approach) for HPW query
// heads of one KV group and one query block I.  The workgroup walks the key blocks u = 0, 1, ... of
// the row (every J <= I when DENSE, else the union of the heads' kept lists).  Iteration u:
//   - gather the K tile of block u+1 (one block ahead) and resolve the row ids of block u+2;
//   - S_u = K_u Q^T for every head that has block u, and each wave's max over its valid entries;
//   - wait for the gathers in flight, barrier;
//   - O += V_{u-1}^T P_{u-1} for the heads that kept block u-1 (its V gather was hidden behind S_u);
//   - per head, the exact tile max of S_u against theta[h][I] (the diagonal is always kept); a
//     kept tile updates (m, l) and yields P_u; the V tile of block u is gathered only if some head
//     kept it.
// A tile that no head keeps costs its K gather and QK^T only; a skipped tile leaves (m, l, acc)
// untouched.  Buffers: K and V double-buffered, row ids in a ring of four, partial maxima double-
// buffered, so one barrier per key block suffices.
template <int D, int BLK, bool DENSE, int HPW>
__global__ __attribute__((amdgpu_flat_work_group_size(PipeCfg<D, BLK, HPW>::THREADS, PipeCfg<D, BLK, HPW>::THREADS),
                          amdgpu_waves_per_eu(2)))
void attn_gate_pipe_kernel(AttnArgs a) {
  using C = PipeCfg<D, BLK, HPW>;
  using AC = AttnCfg<D, BLK>;
  constexpr int WPH = C::WAVES_PER_HEAD;
  constexpr int KB = AC::KB;
  __shared__ __align__(16) uint16_t K0[BLK * D];
  __shared__ __align__(16) uint16_t K1[BLK * D];
  __shared__ __align__(16) uint16_t V0[BLK * D];
  __shared__ __align__(16) uint16_t V1[BLK * D];
  __shared__ uint32_t rowid[4][BLK];  // byte offsets of the gathered rows, ring of four blocks
  __shared__ uint32_t mlist[DENSE ? 1 : C::MAXNB];  // J | kept-by-head bits << 16
  __shared__ uint8_t selb[DENSE ? 1 : HPW * C::MAXNB];
  __shared__ int mcount;
  __shared__ float red[2][C::WAVES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  const int hh = wave / WPH;  // this wave's head within the workgroup
  const int wq = wave % WPH;  // this wave's 32-row slice of the query block
  int I, h0;
  work_item(a.NB, a.Hq / HPW, HPW, blockIdx.x, &I, &h0);
  const int h = h0 + hh;
  const int g = h0 / a.G;
  const int I0 = I * BLK;
  const int qloc = wq * 32 + l32;
  const int qpos = I0 + qloc;
  const bool qvalid = qpos < a.N;
  const size_t ntri = (size_t)a.NB * (a.NB + 1) / 2;
  const rsrc_t qr = make_rsrc(a.q + (int64_t)h * a.qsh, a.q_bytes);
  const rsrc_t kr = make_rsrc(a.k + (int64_t)g * a.kvsh, a.kv_bytes);
  const rsrc_t vr = make_rsrc(a.v + (int64_t)g * a.kvsh, a.kv_bytes);

  {  // rows past N are never written by the gather: start from finite (zero) tiles
    constexpr int NZ = BLK * D * 2 / 16;
    for (int i = t; i < NZ; i += C::THREADS) {
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(K0)[i] = z;
      reinterpret_cast<u32x4*>(K1)[i] = z;
      reinterpret_cast<u32x4*>(V0)[i] = z;
      reinterpret_cast<u32x4*>(V1)[i] = z;
    }
  }
  bf16x8 qf[AC::KSTEPS];
#pragma unroll
  for (int kk = 0; kk < AC::KSTEPS; ++kk) {
    const uint32_t off = qvalid ? (uint32_t)qpos * a.q_row_bytes + kk * 32 + h2 * 16 : kOutOfRange;
    qf[kk] = __builtin_bit_cast(bf16x8, buf_load16(qr, off));
  }
  float th[HPW];
#pragma unroll
  for (int x = 0; x < HPW; ++x) th[x] = a.theta[(size_t)(h0 + x) * a.NB + I];

  const int nblk = DENSE ? I + 1 : union_list<HPW, C::THREADS>(a, h0, I, ntri, selb, mlist, &mcount);
  const int sI = a.S > 0 ? I0 / a.S : 0;
  const uint32_t all_heads = ((1u << HPW) - 1u) << 16;
  auto entry_of = [&](int u) -> uint32_t {  // wave-uniform
    return DENSE ? ((uint32_t)u | all_heads) : (uint32_t)__builtin_amdgcn_readfirstlane(mlist[u]);
  };
  const rsrc_t permr = make_rsrc(a.perm ? a.perm + (size_t)g * a.N : nullptr, a.perm ? (uint32_t)a.N * 4u : 0u);
  // lookup of row j of block u (want = false: an unused lookup that reads nothing)
  auto lookup = [&](int u, int j, bool want) -> RowLook {
    const int J = (int)(entry_of(u) & 0xffffu);
    const int p = J * BLK + j;
    return row_lookup(permr, p, a.N, want, a.perm != nullptr && a.S > 0 && (J * BLK) / a.S < sI);
  };
  auto row_off = [&](const RowLook& r) { return row_lookup_offset(r, a.N, a.N, a.kv_row_bytes, a.err); };
  auto gather_k = [&](int u, uint16_t* dst) {
    const uint32_t* ids = rowid[u & 3];
    auto rf = [&](int j) { return ids[j]; };
    dma_tile<D, BLK, false, decltype(rf), BLK, C::WAVES>(dst, kr, rf);
  };
  auto gather_v = [&](int u, uint16_t* dst) {
    const uint32_t* ids = rowid[u & 3];
    auto rf = [&](int j) { return ids[j]; };
    dma_tile<D, BLK, true, decltype(rf), BLK, C::WAVES>(dst, vr, rf);
  };

  SoftmaxState<D, BLK> st;
  st.init();
  bf16x8 pb[2 * KB];  // probabilities of the last kept tile, consumed one iteration later
  bool keep_prev = false;

  if (nblk > 0) {
    if (t < BLK)
      for (int u = 0; u < 2 && u < nblk; ++u) rowid[u][t] = row_off(lookup(u, t, true));
    __syncthreads();  // zero fill and row ids visible
    gather_k(0, K0);
    wait_vmcnt<0>();
    __syncthreads();
  }

  auto step = [&](int u, const uint16_t* Kc, uint16_t* Kn, const uint16_t* Vp, uint16_t* Vc) {
    bf16x8 first[tile_kq<D, BLK>()];  // read before the lookups and the gather are issued
    tile_first_ops<D, BLK>(Kc, first);
    const RowLook pr = lookup(u + 2 < nblk ? u + 2 : 0, t & (BLK - 1), u + 2 < nblk && t < BLK);
    __builtin_amdgcn_sched_barrier(0);  // the lookup is issued before the gather (vmcnt order)
    if (u + 1 < nblk) gather_k(u + 1, Kn);
    const uint32_t e = entry_of(u);
    const int J = (int)(e & 0xffffu);
    const bool diag = J == I;
    f32x16 sc[KB];
    float row_max = -INFINITY;
    if ((e >> (16 + hh)) & 1u) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        sc[kb] = tile_scores<D, BLK>(Kc, qf, kb, diag, qloc - kb * 32 - 4 * h2, kb == 0 ? first : nullptr);
      row_max = tile_row_max<KB>(sc);
    }
    const float wm = wave_max_f32(qvalid ? row_max : -INFINITY);
    if (lane == 0) red[u & 1][wave] = wm;
    if (u + 2 < nblk && t < BLK) rowid[(u + 2) & 3][t] = row_off(pr);
    wait_vmcnt<0>();  // V of block u-1 and K of block u+1 have landed (this wave's share)
    __syncthreads();
    if (keep_prev) tile_pv<D, BLK>(st, pb, Vp);
    bool any = false, keep = false;
#pragma unroll
    for (int x = 0; x < HPW; ++x) {
      float tm = red[u & 1][x * WPH];
#pragma unroll
      for (int y = 1; y < WPH; ++y) tm = fmaxf(tm, red[u & 1][x * WPH + y]);
      const bool kx = ((e >> (16 + x)) & 1u) && (diag || !(tm * a.scale < th[x]));
      any = any || kx;
      if (x == hh) keep = kx;
    }
    if (keep) tile_softmax<D, BLK>(st, sc, row_max, pb, a.sl2);
    if (any) gather_v(u, Vc);
    if (keep && a.kept && lane == 0 && wq == 0) {
      const size_t bit = tri_offset(I) + J;
      atomicOr(&a.kept[(size_t)h * ((ntri + 31) / 32) + bit / 32], 1u << (bit % 32));
    }
    keep_prev = keep;
  };
  for (int u = 0; u < nblk; u += 2) {
    step(u, K0, K1, V1, V0);
    if (u + 1 < nblk) step(u + 1, K1, K0, V0, V1);
  }
  if (nblk > 0) {
    wait_vmcnt<0>();
    __syncthreads();
    if (keep_prev) tile_pv<D, BLK>(st, pb, ((nblk - 1) & 1) ? V1 : V0);
  }
  write_output<D, BLK>(a, st, h, qpos, qvalid, h2);
}

// Early-stop kernel (Block Sparse Flash Attention, Approach) and calibration tile maxima.  Per key
// block: gather K, compute the whole tile's scores, reduce their exact max across the workgroup,
// and only when the tile is kept gather V and run the same online-softmax / PV steps as the
// pipelined kernel; a threshold of -inf keeps every tile.  MODE_TILE_MAX only writes
// the scaled tile maxima.
template <int D, int BLK, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(AttnCfg<D, BLK>::THREADS, AttnCfg<D, BLK>::THREADS),
                          amdgpu_waves_per_eu(1)))
void attn_gated_kernel(AttnArgs a) {
  using C = AttnCfg<D, BLK>;
  __shared__ __align__(16) uint16_t Ks[BLK * D];
  __shared__ __align__(16) uint16_t Vs[(MODE == MODE_TILE_MAX) ? 8 : BLK * D];
  __shared__ uint32_t rowid[BLK];
  __shared__ float red[C::WAVES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, h2 = lane >> 5;
  int I, h;
  work_item(a, blockIdx.x, &I, &h);
  const int g = h / a.G;
  const int I0 = I * BLK;
  const int qloc = wave * 32 + l32;
  const int qpos = I0 + qloc;
  const bool qvalid = qpos < a.N;
  const size_t ntri = (size_t)a.NB * (a.NB + 1) / 2;
  const rsrc_t qr = make_rsrc(a.q + (int64_t)h * a.qsh, a.q_bytes);
  const rsrc_t kr = make_rsrc(a.k + (int64_t)g * a.kvsh, a.kv_bytes);
  const rsrc_t vr = make_rsrc(a.v + (int64_t)g * a.kvsh, a.kv_bytes);
  {
    u32x4* z = reinterpret_cast<u32x4*>(Ks);
    for (int i = t; i < BLK * D * 2 / 16; i += C::THREADS) z[i] = u32x4{0u, 0u, 0u, 0u};
    if (MODE != MODE_TILE_MAX) {
      u32x4* zv = reinterpret_cast<u32x4*>(Vs);
      for (int i = t; i < BLK * D * 2 / 16; i += C::THREADS) zv[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
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
  SoftmaxState<D, BLK> st;
  st.init();

  for (int it = 0; it < cnt; ++it) {
    const int J = list ? list[it] : it;
    if (J < 0 || J > I) {
      if (t == 0 && a.err) atomicOr(a.err, 1);
      continue;
    }
    const bool diag = (J == I);
    const bool permuted = a.perm != nullptr && a.S > 0 && (J * BLK) / a.S < sI;
    __syncthreads();  // previous tile's LDS reads are done
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
      rowid[t] = row_offset(r, a.kv_row_bytes);
    }
    __syncthreads();
    auto rf = [&](int j) { return rowid[j]; };
    dma_tile<D, BLK, false, decltype(rf), BLK>(Ks, kr, rf);
    wait_dma();
    __syncthreads();
    f32x16 sc[C::KB];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      sc[kb] = block_scores<D, BLK>(Ks, qf, kb, diag, qloc - kb * 32 - 4 * h2);
      mx = fmaxf(mx, block_row_max(sc[kb]));
    }
    if (MODE == MODE_TILE_MAX || !diag) {
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
    if (MODE != MODE_TILE_MAX) {
      dma_tile<D, BLK, true, decltype(rf), BLK>(Vs, vr, rf);
      if (a.kept && t == 0) {
        const size_t bit = tri_offset(I) + J;
        atomicOr(&a.kept[(size_t)h * ((ntri + 31) / 32) + bit / 32], 1u << (bit % 32));
      }
      wait_dma();
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) block_softmax_pv<D, BLK>(st, sc[kb], Vs, kb, a.sl2);
    }
  }
  if (MODE != MODE_TILE_MAX) write_output<D, BLK>(a, st, h, qpos, qvalid, h2);
}

// Persistent launch of the pipelined kernel: the deques are reset on the stream, then as many
// workgroups start as fit on the device at once (never more than there are items).
template <int D, int BLK, bool DENSE, int HPW, bool S2O = false>
static hipError_t launch_persistent(const AttnArgs& a, int items, hipStream_t st) {
  constexpr int THREADS = PipeCfg<D, BLK, HPW>::THREADS;
  static int resident[64] = {0};  // workgroups resident on the whole device, per device ordinal
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (resident[dev] == 0) {
    int cus = 0, per_cu = 0;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_pipe_kernel<D, BLK, DENSE, HPW, S2O>,
                                                          THREADS, 0)) != hipSuccess)
      return e;
    resident[dev] = cus * (per_cu > 0 ? per_cu : 1);
  }
  if ((long long)a.NB * (a.Hq / HPW) >= (1ll << 24)) return hipErrorInvalidValue;  // item index field
  deque_init_kernel<<<1, 64, 0, st>>>(a, a.G / HPW);
  const int grid = items < resident[dev] ? items : resident[dev];
  attn_pipe_kernel<D, BLK, DENSE, HPW, S2O><<<grid, THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int BLK, int MODE>
static hipError_t launch_mode(const AttnArgs& a, int nwg, hipStream_t st) {
  if constexpr (MODE == MODE_ATTN || MODE == MODE_DENSE) {
    constexpr bool DENSE = MODE == MODE_DENSE;
    if ((a.G & 1) == 0) {
      return launch_persistent<D, BLK, DENSE, 2>(a, nwg / 2, st);
    } else {
      return launch_persistent<D, BLK, DENSE, 1>(a, nwg, st);
    }
  } else if (MODE == MODE_ATTN_GATED && (a.G & 1) == 0) {
    if (a.count == nullptr) {
      attn_gate_pipe_kernel<D, BLK, true, 2><<<nwg / 2, PipeCfg<D, BLK, 2>::THREADS, 0, st>>>(a);
    } else {
      attn_gate_pipe_kernel<D, BLK, false, 2><<<nwg / 2, PipeCfg<D, BLK, 2>::THREADS, 0, st>>>(a);
    }
  } else {
    attn_gated_kernel<D, BLK, MODE><<<nwg, AttnCfg<D, BLK>::THREADS, 0, st>>>(a);
  }
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
  a.Hkv = g.Hkv;
  a.nq = g.Hkv < kMaxDeques ? g.Hkv : kMaxDeques;
  a.scale = g.scale;
  a.sl2 = g.scale * 1.4426950408889634f;
  return a;
}

hipError_t launch_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* perm, const int32_t* count, const int32_t* idx,
                            const float* theta, float* out, float* lse, uint32_t* kept, int32_t* err,
                            void* ws, hipStream_t st) {
  AttnArgs a = make_args(g);
  a.queue = static_cast<unsigned long long*>(ws);
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
  if (count == nullptr) return dispatch<MODE_DENSE>(g, a, st);
  return dispatch<MODE_ATTN>(g, a, st);
}

// Early-stop thresholds from calibration tile maxima (Block Sparse Flash Attention, Approach:
// thresholds fixed offline so that about `keep` tiles per query block survive): theta[h][I] is the
// keep-th largest of tmax[h][I(I+1)/2 + J] over J <= I, or -inf when the row has at most keep
// tiles.  One wave per row.  Each value maps to a 32-bit key that orders like the float (sign bit
// flipped for non-negative values, all bits flipped for negative ones); the wave then builds the
// largest key t with count(key >= t) >= keep bit by bit from the top, which is exactly the key of
// the keep-th largest value, so the result is one of the row's own values.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__global__ __launch_bounds__(256) void calibrate_kernel(const float* tmax, int Hq, int NB, int keep, float* theta) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= Hq * NB) return;
  const int h = row / NB, I = row % NB;
  const int n = I + 1;
  if (n <= keep) {
    if (lane == 0) theta[row] = -INFINITY;
    return;
  }
  const size_t ntri = (size_t)NB * (NB + 1) / 2;
  const float* r = tmax + (size_t)h * ntri + (size_t)I * (I + 1) / 2;
  uint32_t t = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    int cnt = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool ge = j < n && order_key(r[j]) >= cand;
      cnt += __popcll(__ballot(ge));
    }
    if (cnt >= keep) t = cand;
  }
  if (lane == 0) theta[row] = order_key_inv(t);
}

hipError_t launch_calibrate(int Hq, int NB, const float* tmax, int keep, float* theta, hipStream_t st) {
  const int rows = Hq * NB;
  calibrate_kernel<<<(rows + 3) / 4, 256, 0, st>>>(tmax, Hq, NB, keep, theta);
  return hipGetLastError();
}

// One head per workgroup with the marginal-gain stop, over ranked lists (a.count / a.idx) or over
// the two-pass lists of the per-segment prefix order (a.kvr).
static hipError_t launch_s2o_kernel(const Geometry& g, const AttnArgs& a, hipStream_t st) {
  const int items = g.Hq * g.NB;
  if (g.d == 128 && g.B == 128) return launch_persistent<128, 128, false, 1, true>(a, items, st);
  if (g.d == 128 && g.B == 64) return launch_persistent<128, 64, false, 1, true>(a, items, st);
  if (g.d == 64 && g.B == 128) return launch_persistent<64, 128, false, 1, true>(a, items, st);
  return launch_persistent<64, 64, false, 1, true>(a, items, st);
}

hipError_t launch_s2o_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* perm, const int32_t* count, const int32_t* idx, float gain_tau,
                                float* out, float* lse, uint32_t* kept, int32_t* err, void* ws, hipStream_t st) {
  AttnArgs a = make_args(g);
  a.queue = static_cast<unsigned long long*>(ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.perm = perm;
  a.count = count;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.kept = kept;
  a.err = err;
  a.gain_tau = gain_tau;
  return launch_s2o_kernel(g, a, st);
}

hipError_t launch_s2o_prefix_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const int32_t* kv_rank, int64_t rank_len, const int32_t* qperm,
                                       float gain_tau, float* out, float* lse, uint32_t* kept, int32_t* err,
                                       void* ws, hipStream_t st) {
  AttnArgs a = make_args(g);
  a.queue = static_cast<unsigned long long*>(ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.two_pass = 1;
  a.kvr = kv_rank;
  a.kvr_L = rank_len;
  a.qperm = qperm;
  a.out = out;
  a.lse = lse;
  a.kept = kept;
  a.err = err;
  a.gain_tau = gain_tau;
  return launch_s2o_kernel(g, a, st);
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
