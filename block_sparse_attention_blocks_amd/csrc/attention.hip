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
// The register layouts and shared pieces are in attn_device.h.
#include "attn_device.h"

namespace pbsa {

// Software-pipelined block-sparse (DENSE = false) or dense causal (DENSE = true) attention for
// HPW query heads h0 .. h0+HPW-1 of one KV group and one query block I.  The workgroup walks the
// union of the heads' kept key blocks in ascending order; each KT-key stage of a block is gathered
// once into LDS and used by the waves of every head that kept the block (the query heads of a
// group usually keep nearly the same blocks).  While stage s is computed, stages s+1 .. s+NBUF-1
// are in flight, and the physical row ids of stage s+NBUF are fetched from perm.
//
// S2O = true: after every earlier-segment block, a head stops its row when each query's share of
// that block in its softmax denominator is below a.gain_tau (S2O, Early-Stopping Rule), and the
// workgroup stops when all its heads have.  With ranked lists (HPW = 1) the list is the head's own
// ranked list, taken in its order.  With the two-pass lists (a.two_pass) every query head of a KV
// group walks the same blocks in the same order -- its own segment, then the KV head's prefix
// order -- so HPW = 2 heads share each gathered tile until they stop; a head that has stopped
// leaves its later tiles to the other.
// Keys per LDS stage: the mask path of head pairs takes whole 128-key blocks (two buffers), which
// pays each stage's fixed part (row ids, gather issue, wait, barrier) once per block; the dense
// and marginal-gain paths keep 64-key stages.
template <int BLK, bool DENSE, int HPW, bool S2O>
constexpr int pipe_kt() { return (!DENSE && !S2O && HPW == 2 && BLK == 128) ? 128 : 64; }

template <int D, int BLK, bool DENSE, int HPW, bool S2O = false>
__global__ __attribute__((amdgpu_flat_work_group_size(PipeCfg<D, BLK, HPW>::THREADS, PipeCfg<D, BLK, HPW>::THREADS),
                          amdgpu_waves_per_eu(2)))
void attn_pipe_kernel(AttnArgs a) {
  static_assert(!S2O || !DENSE, "the marginal-gain stop walks lists");
  using C = PipeCfg<D, BLK, HPW, pipe_kt<BLK, DENSE, HPW, S2O>()>;
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
                   : two_pass ? two_pass_list<C::THREADS>(Jend, J0, mlist, HPW)
                   : S2O      ? (HPW == 1 ? ranked_list<C::THREADS>(a, h0, I, ntri, mlist, &mcount) : 0)
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
      dma_tile<D, BLK, false, decltype(rf), KT, C::WAVES, true>(Kd, kr, rf);
      dma_tile<D, BLK, true, decltype(rf), KT, C::WAVES, true>(Vd, vr, rf);
    } else {
      // the lane's row offsets, read once for both tiles and all before the first DMA
      using L = GatherLane<D, KT, C::WAVES>;
      uint32_t ro[L::NI];
#pragma unroll
      for (int i = 0; i < L::NI; ++i) ro[i] = rowid[b][L::row(i)];
      dma_tile_ro<D, false, KT, C::WAVES>(Kd, kr, ro);
      dma_tile_ro<D, true, KT, C::WAVES>(Vd, vr, ro);
    }
  };

  SoftmaxState<D, BLK> st;
  st.init();
  uint32_t done = 0;  // heads of the workgroup whose row has stopped (marginal-gain stop)

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
    // this stage's list entry is read ahead of the gathers below, whose asm statements would
    // otherwise hold the LDS read back until they are issued
    const uint32_t e = s < nst ? entry_of(s) : 0u;
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
    if (((e & ~(done << 16)) >> (16 + hh)) & 1u) {
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
      stage_compute<D, BLK, KT>(st, Kc, Vc, qf, kop0, qperm_on ? J >= J0 : J == I,
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
      // after an earlier-segment block: a head that processed it stops when every one of its waves
      // found its share below the threshold; the workgroup stops when every head has
      const uint32_t e2 = entry_of(s);
      const int J = (int)(e2 & 0xffffu);
      if (a.S > 0 && (J * BLK) / a.S < sI) {
#pragma unroll
        for (int x = 0; x < HPW; ++x) {
          if ((((e2 & ~(done << 16)) >> (16 + x)) & 1u) == 0) continue;
          bool all = true;
#pragma unroll
          for (int y = 0; y < C::WAVES_PER_HEAD; ++y)
            all = all && stop_flag[(s / C::STAGES) & 1][x * C::WAVES_PER_HEAD + y];
          if (all) done |= 1u << x;
        }
        return done == (1u << HPW) - 1u;
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

// Scores of every score block of a tile, with the K operands streamed through a ring of PF + 1
// registers in block-major, k-step-minor order: the read of operand i + PF is issued before the
// product that takes operand i, so PF reads are in flight under the products instead of one batch
// read and waited for at a time.  first holds operands 0 .. PF - 1 (tile_first_ring, read early by
// the caller).  The products of each block run in k-step order, as in tile_scores.
template <int D, int BLK>
__device__ __forceinline__ bf16x8 tile_k_operand(const uint16_t* Ks, int i) {
  constexpr int KS = AttnCfg<D, BLK>::KSTEPS;
  const int lane = threadIdx.x & 63, h2 = lane >> 5;
  const int kb = i / KS, kk = i % KS;
  const int krow = kb * 32 + (lane & 31);
  return *reinterpret_cast<const bf16x8*>(Ks + krow * D + (((kk * 2 + h2) ^ kt_swz<D>(krow)) * 8));
}
template <int D, int BLK, int PF>
__device__ __forceinline__ void tile_first_ring(const uint16_t* Ks, bf16x8* first) {
#pragma unroll
  for (int i = 0; i < PF; ++i) first[i] = tile_k_operand<D, BLK>(Ks, i);
}
template <int D, int BLK, int PF>
__device__ __forceinline__ void tile_scores_ring(const uint16_t* Ks, const bf16x8* qf, f32x16* sc, bool diag, int rel,
                                                 const bf16x8* first) {
  using C = AttnCfg<D, BLK>;
  constexpr int KS = C::KSTEPS, NT = C::KB * KS;
  bf16x8 ring[PF + 1];
#pragma unroll
  for (int i = 0; i < PF; ++i) ring[i] = first[i];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    if (i + PF < NT) ring[(i + PF) % (PF + 1)] = tile_k_operand<D, BLK>(Ks, i + PF);
    const int kb = i / KS, kk = i % KS;
    if (kk == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
    }
    sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % (PF + 1)], qf[kk], sc[kb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (diag) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) causal_mask(sc[kb], rel - kb * 32);
  }
}
#ifndef PBSA_GATE_PF
#define PBSA_GATE_PF 2
#endif

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
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    // two probabilities per packed conversion; each pair is added to the row sum as it is and placed
    // as one dword of the PV operand
    u32x4_t pw[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const f32x2 x = {__builtin_amdgcn_exp2f(fmaf(s[kb][2 * j], sl2, -m_use)),
                       __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j + 1], sl2, -m_use))};
      const bf16x2 pair = __builtin_convertvector(x, bf16x2);
      st.l = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, st.l, false);
      pw[j >> 2][j & 3] = __builtin_bit_cast(unsigned int, pair);
    }
    pb[2 * kb] = __builtin_bit_cast(bf16x8, pw[0]);
    pb[2 * kb + 1] = __builtin_bit_cast(bf16x8, pw[1]);
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

  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
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
  // Q operands and thresholds complete here, before the loop: the compiler cannot see the gathers'
  // waits (inline assembly), and waits left to it inside the loop would count the gathers in
  // flight as well
#pragma unroll
  for (int kk = 0; kk < AC::KSTEPS; ++kk) asm volatile("" ::"v"(qf[kk]));
#pragma unroll
  for (int x = 0; x < HPW; ++x) asm volatile("" ::"v"(th[x]));

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
  // Gathers as inline-assembly DMAs, which the compiler's wait-count pass does not track: issued
  // through the builtin, a V gather still in flight made the compiler wait for it (vmcnt(0)) before
  // the first LDS read of the next step, so the V load of a kept tile was not hidden behind the next
  // tile's QK^T.  The kernel waits for its gathers itself (wait_vmcnt before each barrier).  A lane's
  // row offsets are read together before its first DMA.
  using GL = GatherLane<D, BLK, C::WAVES>;
  auto gather_k = [&](int u, uint16_t* dst) {
    uint32_t ro[GL::NI];
#pragma unroll
    for (int i = 0; i < GL::NI; ++i) ro[i] = rowid[u & 3][GL::row(i)];
    dma_tile_ro<D, false, BLK, C::WAVES>(dst, kr, ro);
  };
  auto gather_v = [&](int u, uint16_t* dst) {
    uint32_t ro[GL::NI];
#pragma unroll
    for (int i = 0; i < GL::NI; ++i) ro[i] = rowid[u & 3][GL::row(i)];
    dma_tile_ro<D, true, BLK, C::WAVES>(dst, vr, ro);
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
    const RowLook pr = lookup(u + 2 < nblk ? u + 2 : 0, t & (BLK - 1), u + 2 < nblk && t < BLK);
    __builtin_amdgcn_sched_barrier(0);  // the lookup is issued before the gather (vmcnt order)
    if (u + 1 < nblk) gather_k(u + 1, Kn);
    bf16x8 first[PBSA_GATE_PF];
    tile_first_ring<D, BLK, PBSA_GATE_PF>(Kc, first);
    const uint32_t e = entry_of(u);
    const int J = (int)(e & 0xffffu);
    const bool diag = J == I;
    f32x16 sc[KB];
    float row_max = -INFINITY;
    if ((e >> (16 + hh)) & 1u) {
      const int rel = opaque(qloc - 4 * h2);  // causal offset, computed per tile (see opaque)
      tile_scores_ring<D, BLK, PBSA_GATE_PF>(Kc, qf, sc, diag, rel, first);
      row_max = tile_row_max<KB>(sc);
    }
    const float wm = wave_max_f32(qvalid ? row_max : -INFINITY);
    if (lane == 0) red[u & 1][opaque(wave)] = wm;
    if (u + 2 < nblk && t < BLK) rowid[(u + 2) & 3][opaque(t)] = row_off(pr);
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
// The number of resident workgroups is queried on every call (the runtime answers from the kernel's
// metadata without touching the device), so the library keeps no state between calls.
template <int D, int BLK, bool DENSE, int HPW, bool S2O = false>
static hipError_t launch_persistent(const AttnArgs& a, int items, hipStream_t st, int max_wg = 0) {
  constexpr int THREADS = PipeCfg<D, BLK, HPW>::THREADS;
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_pipe_kernel<D, BLK, DENSE, HPW, S2O>, THREADS,
                                                        0)) != hipSuccess)
    return e;
  int resident = cus * (per_cu > 0 ? per_cu : 1);
  if (max_wg > 0 && max_wg < resident) resident = max_wg;
  if ((long long)a.NB * (a.Hq / HPW) >= (1ll << 24)) return hipErrorInvalidValue;  // item index field
  deque_init_kernel<<<1, 64, 0, st>>>(a, a.G / HPW);
  const int grid = items < resident ? items : resident;
  attn_pipe_kernel<D, BLK, DENSE, HPW, S2O><<<grid, THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int BLK, int MODE>
static hipError_t launch_mode(const AttnArgs& a, int nwg, hipStream_t st, int max_wg) {
  if constexpr (MODE == MODE_ATTN || MODE == MODE_DENSE) {
    constexpr bool DENSE = MODE == MODE_DENSE;
    if ((a.G & 1) == 0) {
      return launch_persistent<D, BLK, DENSE, 2>(a, nwg / 2, st, max_wg);
    } else {
      return launch_persistent<D, BLK, DENSE, 1>(a, nwg, st, max_wg);
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
static hipError_t dispatch(const Geometry& g, const AttnArgs& a, hipStream_t st, int max_wg = 0) {
  const int nwg = g.Hq * g.NB;
  if (g.d == 128 && g.B == 128) return launch_mode<128, 128, MODE>(a, nwg, st, max_wg);
  if (g.d == 128 && g.B == 64) return launch_mode<128, 64, MODE>(a, nwg, st, max_wg);
  if (g.d == 64 && g.B == 128) return launch_mode<64, 128, MODE>(a, nwg, st, max_wg);
  return launch_mode<64, 64, MODE>(a, nwg, st, max_wg);
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
                            void* ws, hipStream_t st, const LaunchOpts& opt) {
  AttnArgs a = make_args(g);
  a.queue = static_cast<unsigned long long*>(ws);
  a.claim_back = opt.claim_back ? 1 : 0;
  a.out_bf16 = opt.out_bf16 ? 1 : 0;
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
  if (count == nullptr) return dispatch<MODE_DENSE>(g, a, st, opt.max_wg);
  return dispatch<MODE_ATTN>(g, a, st, opt.max_wg);
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

// The marginal-gain stop: one head per workgroup over ranked lists (a.count / a.idx), whose order
// differs from head to head; over the two-pass lists of the per-segment prefix order (a.kvr), which
// every head of a KV group shares, two heads per workgroup when the group size is even.
template <int HPW>
static hipError_t launch_s2o_hpw(const Geometry& g, const AttnArgs& a, hipStream_t st) {
  const int items = g.Hq * g.NB / HPW;
  if (g.d == 128 && g.B == 128) return launch_persistent<128, 128, false, HPW, true>(a, items, st);
  if (g.d == 128 && g.B == 64) return launch_persistent<128, 64, false, HPW, true>(a, items, st);
  if (g.d == 64 && g.B == 128) return launch_persistent<64, 128, false, HPW, true>(a, items, st);
  return launch_persistent<64, 64, false, HPW, true>(a, items, st);
}

static hipError_t launch_s2o_kernel(const Geometry& g, const AttnArgs& a, hipStream_t st) {
  if (a.two_pass && (g.G & 1) == 0) return launch_s2o_hpw<2>(g, a, st);
  return launch_s2o_hpw<1>(g, a, st);
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

hipError_t launch_tile_max(const Geometry& g, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                           float* tmax, hipStream_t st) {
  AttnArgs a = make_args(g);
  a.q = q;
  a.k = k;
  a.v = k;
  a.perm = perm;
  a.tmax = tmax;
  if (perm == nullptr) a.S = 0;
  return dispatch<MODE_TILE_MAX>(g, a, st);
}

}  // namespace pbsa
