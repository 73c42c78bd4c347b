// Device helpers shared by the stage-3 attention kernels (attention.hip, attention_dual.hip):
// argument block, LDS tile layouts and gathers, online-softmax pieces on the bf16 MFMA, block
// lists and the per-XCD work deques.
//
// MFMA 32x32x16 bf16 register layouts used throughout (lane = 0..63, l32 = lane % 32, h2 = lane / 32):
//   A (32 x 16): lane holds row l32, k = 8*h2 + e (e = 0..7)
//   B (16 x 32): lane holds column l32, k = 8*h2 + e
//   C (32 x 32): lane holds column l32, rows 8*(r/4) + 4*h2 + r%4 in register r = 0..15
// Only the pairing of A and B along k matters for a contraction, so V^T is stored with the key
// order inside every 16-key group permuted to match the keys that the P^T operand inherits from
// the layout of S^T.
#pragma once

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
  static constexpr int KT = 64;                        // keys per pipelined LDS stage (default)
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
  int claim_back;             // take items from the back of the home deque (and the front of the others)
  int Hkv;
  int two_pass;               // S2O kernels: two-pass lists over the per-segment prefix order kvr
  const int32_t* kvr;         // per-segment prefix key order (NULL when no segment has a prefix)
  int64_t kvr_L;              // entries of kvr per KV head
  const int32_t* qperm;       // two-pass lists: query order inside segments [Hkv][N], or NULL
  int out_bf16;               // out holds bf16 values (same element strides) instead of fp32
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

// LDS DMA written as inline assembly, for the pipelined kernel.  Issued through the builtin, these
// loads are tracked by the compiler's wait-count pass, which made later VALU writes wait for the
// gather just issued (a vmcnt wait in the middle of the current stage's softmax), so the gather
// of stage s+2 had to land within stage s.  The pass does not see loads issued from inline
// assembly: the kernel waits for them itself (wait_vmcnt before every barrier that hands a stage
// buffer to the readers).  M0 holds the LDS destination; the one wait state between writing M0
// and the DMA is the s_nop.  No VGPR is written, so nothing in flight can clobber a register.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

__device__ __forceinline__ void lds_dma_b128(rsrc_t r, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds" ::"v"(off), "s"(lds), "s"(r)
               : "memory");
}
__device__ __forceinline__ void lds_dma_b32(rsrc_t r, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds" ::"v"(off), "s"(lds), "s"(r)
               : "memory");
}

// One gathered tile: the rows at byte offsets row_off(j) of the head's slab into LDS [ROWS][D]
// with the chunk swizzle.  An offset of kOutOfRange leaves a zero row.
// lane: this lane's index, passed in when the caller wants the per-lane swizzle offsets computed
// at each gather rather than hoisted out of its loop (see opaque_lane); -1 reads threadIdx.x.
template <int D, int BLK, bool IS_V, typename RowFn, int ROWS = AttnCfg<D, BLK>::KT,
          int WAVES = AttnCfg<D, BLK>::WAVES, bool ASM = false>
__device__ __forceinline__ void dma_tile(uint16_t* dst, rsrc_t r, RowFn row_off, int lane_in = -1) {
  constexpr int RPI = 512 / D;  // rows per 1 KiB wave instruction
  constexpr int LPR = D / 8;    // lanes per row
  constexpr int NI = ROWS / (RPI * WAVES);
  static_assert(NI * RPI * WAVES == ROWS, "tile rows must split evenly over the waves");
  const int lane = lane_in >= 0 ? lane_in : (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row0 = (wave * NI + i) * RPI;
    const int rw = row0 + lane / LPR;
    const uint32_t c = (lane % LPR) ^ (IS_V ? vt_swz<D>(rw) : kt_swz<D>(rw));
    const uint32_t off = row_off(rw) + c * 16;  // kOutOfRange + c*16 stays out of range
    if constexpr (ASM) {
      lds_dma_b128(r, lds_addr(dst) + row0 * D * 2, off);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + row0 * D), 16, off, 0, 0, 0);
    }
  }
}

// The rows of a gather that one lane issues: row (wave * NI + i) * RPI + lane / LPR for i < NI, the
// same rows in the K and the V tile of a stage.
template <int D, int ROWS, int WAVES>
struct GatherLane {
  static constexpr int RPI = 512 / D;
  static constexpr int LPR = D / 8;
  static constexpr int NI = ROWS / (RPI * WAVES);
  __device__ static __forceinline__ int row0(int i) {  // first row of the wave's i-th DMA (uniform)
    return (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * NI + i) * RPI;
  }
  __device__ static __forceinline__ int row(int i) { return row0(i) + (int)(threadIdx.x & 63) / LPR; }
};

// dma_tile (inline-assembly form) from row offsets already in registers, ro[i] for the lane's row
// GatherLane::row(i).  The offsets of a stage are read from LDS together before the first DMA: the
// DMA's asm statement orders memory, so an LDS read placed after one DMA waits for its own round
// trip before the next DMA can issue.
template <int D, bool IS_V, int ROWS, int WAVES>
__device__ __forceinline__ void dma_tile_ro(uint16_t* dst, rsrc_t r, const uint32_t* ro) {
  using L = GatherLane<D, ROWS, WAVES>;
  static_assert(L::NI * L::RPI * WAVES == ROWS, "tile rows must split evenly over the waves");
  const int lane = (int)(threadIdx.x & 63);
#pragma unroll
  for (int i = 0; i < L::NI; ++i) {
    const int row0 = L::row0(i);
    const int rw = row0 + lane / L::LPR;
    const uint32_t c = (lane % L::LPR) ^ (IS_V ? vt_swz<D>(rw) : kt_swz<D>(rw));
    lds_dma_b128(r, lds_addr(dst) + row0 * D * 2, ro[i] + c * 16);  // kOutOfRange + c*16 stays out of range
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// A copy of x that the compiler cannot see through.  Values derived from it inside a loop body are
// computed there instead of being hoisted out of the loop and kept in registers for its whole
// length: where registers run short, the hoisted per-lane constants were spilled, and reloading a
// spilled value waits (vmcnt) for every load in flight, gathers included.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

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
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // probabilities converted two at a time (one packed conversion per pair), each pair added to the
  // row sum as it is and placed as one dword of the PV operand
  u32x4_t pw[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(s[2 * j], sl2, -st.muse)),
                     __builtin_amdgcn_exp2f(fmaf(s[2 * j + 1], sl2, -st.muse))};
    const bf16x2 pair = __builtin_convertvector(x, bf16x2);
    st.l = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, st.l, false);
    pw[j >> 2][j & 3] = __builtin_bit_cast(unsigned int, pair);
  }
  bf16x8 pb[2];
  pb[0] = __builtin_bit_cast(bf16x8, pw[0]);
  pb[1] = __builtin_bit_cast(bf16x8, pw[1]);
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
template <int D, int BLK, int KT = AttnCfg<D, BLK>::KT>
__device__ __forceinline__ void stage_compute(SoftmaxState<D, BLK>& st, const uint16_t* Kc, const uint16_t* Vc,
                                              const bf16x8* qf, const bf16x8* kop0, bool diag, int rel0,
                                              float sl2) {
  using C = AttnCfg<D, BLK>;
  constexpr int NKB = KT / 32;
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
  if (a.out_bf16) {  // the same fp32 values, rounded to bf16 (nearest even) as they are stored
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + (int64_t)h * a.osh + (int64_t)qpos * a.ost;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        bf16x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (__bf16)(st.o[db][rq * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * rq + 4 * h2) = val;
      }
  } else {
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
  }
  if (a.lse && h2 == 0)
    a.lse[(size_t)h * a.N + qpos] = l_tot > 0.f ? st.m * 0.69314718055994531f + logf(l_tot) : -INFINITY;
}

// Pipelined kernel configuration: HPW query heads of one KV group per workgroup (WAVES_PER_HEAD
// waves of 32 query rows each), KT-key LDS stages, NBUF stage buffers.
template <int D, int BLK, int HPW, int KT_ = AttnCfg<D, BLK>::KT>
struct PipeCfg {
  static constexpr int WAVES_PER_HEAD = BLK / 32;
  static constexpr int WAVES = HPW * WAVES_PER_HEAD;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KT = KT_;
  static constexpr int STAGES = BLK / KT;
  // one workgroup per CU has room for three 64-key stages (two of 128 keys)
  static constexpr int NBUF = (HPW == 1 || KT == 128) ? 2 : 3;
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
__device__ __forceinline__ int two_pass_list(int Jend, int J0, uint32_t* mlist, int hpw) {
  const int nin = Jend + 1 - J0;
  const uint32_t heads = ((1u << hpw) - 1u) << 16;  // every head of the workgroup walks the list
  for (int x = threadIdx.x; x <= Jend; x += THREADS)
    mlist[x] = (uint32_t)(x < nin ? J0 + x : x - nin) | heads;
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

static __global__ __launch_bounds__(64) void deque_init_kernel(AttnArgs a, int units_per_group) {
  const int q = threadIdx.x;
  if (q < a.nq) a.queue[q] = (unsigned long long)deque_items(a, q, units_per_group) << 32;
}

// item code (q << 24 | index) or -1 when every deque is empty.  With a.claim_back the two ends swap
// roles (the home deque's shortest rows first, the others' longest stolen); the results do not
// depend on which workgroup computes an item or when, which that order lets a caller check.
__device__ __forceinline__ int claim_item(const AttnArgs& a, int home) {
  if (a.claim_back) {
    unsigned long long old = atomicAdd(&a.queue[home], 0xFFFFFFFF00000000ull);
    int f = (int)(uint32_t)old, b = (int)(uint32_t)(old >> 32);
    if (b >= 1 && b - 1 >= f) return (home << 24) | (b - 1);
    for (int k = 1; k < a.nq; ++k) {
      const int q = home + k < a.nq ? home + k : home + k - a.nq;
      old = atomicAdd(&a.queue[q], 1ull);
      f = (int)(uint32_t)old;
      b = (int)(uint32_t)(old >> 32);
      if (f < b) return (q << 24) | f;
    }
    return -1;
  }
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

}  // namespace pbsa
