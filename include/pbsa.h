/*
 * pbsa.h -- permuted block-sparse attention prefill on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpbsa.so.  Three calls make up one prefill of one attention layer (batch 1):
 *
 *   1. pbsa_build_segment_permutation  key importance from the last block of queries, then a
 *                                      descending sort inside every segment -> index list perm
 *   2. pbsa_estimate_block_mask        mean-pooled block scores, softmax per query block, and the
 *                                      shortest set of key blocks reaching a cumulative mass
 *   3. pbsa_block_sparse_attn_prefill  causal attention over the selected key blocks, keys
 *                                      gathered through perm, online softmax, optional tile-max
 *                                      early stop
 *
 * plus pbsa_tile_max and pbsa_calibrate_thresholds (offline calibration of the early-stop
 * thresholds) and small helpers.
 *
 * Sources of each operation (page title, section):
 *   - Sparser Block-Sparse Attention via Token Permutation: section 2 (segmented permutation),
 *     section 3 (proxy scoring from the last query block, sorting inside segments), section 4
 *     (block selection by mean pooling on the permuted keys), Problem Statement (block-sparse
 *     attention skips blocks outside a mask).
 *   - S2O: Early Stopping for Sparse Attention via Online Permutation: section 1 (the
 *     permutation is an index array that steers which tokens a tile loads; tensors stay in place)
 *     and section 3 (FlashAttention-style online softmax state m, l, acc).
 *   - SampleAttention (Technical Deep Dive): sparsity chosen by the attention mass that must be
 *     kept per query.
 *   - Block Sparse Flash Attention, Approach: exact QK^T of a tile, V load and PV skipped when the
 *     tile's max score is below a calibrated per-(head, position) threshold.
 *
 * Conventions shared by every call
 *   - Tensors: q [Hq][N][d], k and v [Hkv][N][d], bf16 (passed as uint16_t bit patterns), with
 *     element strides given in pbsa_shape (0 = contiguous [heads][tokens][d]); the d dimension must
 *     be contiguous and token strides multiples of 8 elements, base pointers 16-byte aligned.
 *     out is fp32 with its own strides; lse is fp32 [Hq][N] contiguous.
 *   - Query head h reads KV head h / (Hq / Hkv).  Block J = tokens [J*B, min((J+1)*B, N));
 *     NB = ceil(N / B).  Segment of block J = (J*B) / S.  N need not be a multiple of B or S.
 *   - Ownership: every pointer is device memory owned by the caller (except pbsa_shape, which is
 *     host memory read during the call).  The library allocates nothing.  Scratch memory is the
 *     caller's workspace, sized by pbsa_workspace_size; the only exception is
 *     pbsa_block_sparse_attn_prefill_noalloc, whose 256-byte queue array is a device variable of
 *     the library (one per GPU, with its address kept per device after the first call).
 *   - Streams: stream is a hipStream_t (NULL = the default stream).  Every call only enqueues
 *     work on it and returns; outputs are valid once the stream reaches that point.  Inputs,
 *     outputs and workspace must stay alive until then.  Calls that share a workspace must be
 *     ordered on one stream.
 *   - Errors: the status is returned synchronously.  Arguments are validated before anything is
 *     enqueued, so an error other than PBSA_ERR_HIP leaves every output untouched.  No exception
 *     crosses the ABI.  Calls are reentrant.
 *   - Supported: d in {64, 128}; B in {64, 128}; S a positive multiple of B up to 8192 (or 0 for
 *     "no permutation"); Hq a positive multiple of Hkv; N >= 0 (N = 0 is a no-op); NB <= 2048.
 *     One head of q, k or v spans less than 2^31 bytes (N * token stride * 2), and each of q, k,
 *     v and out, all heads included, less than 2^48 bytes; larger strides return
 *     PBSA_ERR_UNSUPPORTED.
 */
#ifndef PBSA_H
#define PBSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PBSA_OK = 0,
  PBSA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, stride, tau, flag combination */
  PBSA_ERR_UNSUPPORTED = 2,  /* a valid shape the library does not handle (d, B, S, NB limits) */
  PBSA_ERR_WORKSPACE = 3,    /* workspace null or smaller than pbsa_workspace_size */
  PBSA_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} pbsa_status;

typedef struct {
  int32_t seq_len;        /* N, tokens (>= 0) */
  int32_t num_q_heads;    /* Hq */
  int32_t num_kv_heads;   /* Hkv, divides Hq */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t block_size;     /* B: query block = key block, 64 or 128 */
  int32_t segment_size;   /* S: multiple of B (<= 8192); 0 = no permutation */
  float softmax_scale;    /* logit scale c; <= 0 selects 1/sqrt(d) */
  int64_t q_stride_head, q_stride_token;    /* elements; 0,0 = contiguous [Hq][N][d] */
  int64_t kv_stride_head, kv_stride_token;  /* elements, shared by k and v; 0,0 = contiguous */
  int64_t o_stride_head, o_stride_token;    /* elements of out; 0,0 = contiguous */
} pbsa_shape;

/* Workspace selectors for pbsa_workspace_size. */
enum {
  PBSA_OP_PERMUTATION = 0,
  PBSA_OP_MASK = 1,
  PBSA_OP_ATTENTION = 2,
  PBSA_OP_PREFIX_RANK = 3,
  PBSA_OP_QUERY_PERM = 4
};

/* Flags of pbsa_estimate_block_mask. */
enum {
  PBSA_FORCE_DIAG = 1u,   /* always keep the diagonal block J = I */
  PBSA_FORCE_FIRST = 2u,  /* always keep block J = 0 of the row's (permuted) order */
  /* instead of a mass cut: list every J <= I in the order of the marginal-gain early stop (S2O,
   * Early-Stopping Rule and Kernel Implementation): the blocks of I's own segment ascending, then
   * the earlier-segment blocks by pooled logit z descending, ties by J ascending; count = I + 1.
   * The force flags are then not used (mass_tau is still checked to lie in (0, 1]).  Needs
   * segment_size > 0 and block_prob == NULL (no probabilities are written). */
  PBSA_MASK_RANKED = 4u
};

/*
 * Bytes of workspace the given call needs for this shape (0 if none; SIZE_MAX if the shape is
 * invalid).  Monotone non-decreasing in N.  Host-only; never touches the GPU.
 */
size_t pbsa_workspace_size(const pbsa_shape* shape, int op);

/*
 * Stage 1 -- segmented key permutation as an index list.
 *
 * Sparser Block-Sparse Attention via Token Permutation, sections 2 and 3.  For KV head g the proxy
 * rows are the last B query positions [max(0, N-B), N) of each of its Hq/Hkv query heads.  Each row
 * i takes the causal softmax of c * q_i . k_j over j <= i; importance[g][j] is the mean of these
 * probabilities over all proxy rows (masked entries count 0), computed in fp64 except that the
 * per-chunk exponentials are stored as fp32 between the two halves of the pass, so each value is
 * within 2^-24 relative of the exact fp64 mean (plus fp64 rounding).  Inside every
 * segment [s*S, min((s+1)*S, N)) the positions are sorted by importance descending, ties by
 * position ascending: perm[g][s*S + r] = position of the r-th key.  perm is a bijection on each
 * segment; K and V are never moved.
 *
 *   q, k        bf16 inputs (see conventions); v is not needed
 *   perm        out, int32 [Hkv][N]
 *   importance  out, fp64 [Hkv][N], or NULL
 *   workspace   >= pbsa_workspace_size(shape, PBSA_OP_PERMUTATION) bytes, 256-byte aligned
 * Requires segment_size > 0.
 */
pbsa_status pbsa_build_segment_permutation(const pbsa_shape* shape, const uint16_t* q,
                                           const uint16_t* k, int32_t* perm, double* importance,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 2 -- block mask by mean pooling and cumulative mass.
 *
 * Sparser Block-Sparse Attention via Token Permutation, section 4, with the keep rule of
 * SampleAttention's cumulative attention mass.  In fp64: Qbar[h][I] = mean of the query rows of
 * block I; for J <= I, Kbar[J] = mean of the keys block J stands for when read by I -- rows
 * perm[g][J*B ...] when J's segment is strictly before I's segment, natural rows J*B ... otherwise
 * (perm == NULL: natural rows always).  z_J = c * Qbar . Kbar[J]; p = softmax over J <= I.  Order J
 * by (p descending, J ascending) and keep the shortest prefix whose running sum is >= mass_tau
 * (every J <= I if mass_tau >= 1 or the sum stays below it), then add J = I (PBSA_FORCE_DIAG) and
 * J = 0 (PBSA_FORCE_FIRST).
 *
 *   perm         int32 [Hkv][N] from stage 1, or NULL (permutation off)
 *   mass_tau     in (0, 1]
 *   block_count  out, int32 [Hq][NB]: number of kept blocks of row (h, I)
 *   block_idx    out, int32 [Hq][NB(NB+1)/2]: row (h, I) starts at I(I+1)/2 and lists its kept
 *                J in ascending order; entries past block_count are left unspecified
 *   block_prob   out, fp64 [Hq][NB(NB+1)/2] (p of row (h, I) at I(I+1)/2 + J), or NULL
 *   workspace    >= pbsa_workspace_size(shape, PBSA_OP_MASK) bytes, 256-byte aligned
 * Requires segment_size > 0 when perm is not NULL.
 */
pbsa_status pbsa_estimate_block_mask(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                     const int32_t* perm, double mass_tau, uint32_t flags,
                                     int32_t* block_count, int32_t* block_idx, double* block_prob,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 3 -- causal block-sparse attention prefill.
 *
 * Sparser Block-Sparse Attention via Token Permutation, Problem Statement; S2O section 1 (index-
 * driven gather) and section 3 (online softmax).  For query i of block I of head h:
 *   K_hi = { j : j in rows(J, I) for a kept J of row (h, I), j <= i }
 *   out[h][i] = sum_{j in K_hi} softmax_j(c q_i . k_j) v_j,   lse[h][i] = log sum_j exp(c q_i . k_j)
 * rows(J, I) as in stage 2.  A query with no key gets out = 0 and lse = -inf.  bf16 products are
 * accumulated in fp32 on the matrix cores; probabilities are rounded to bf16 for the PV product.
 *
 *   perm              int32 [Hkv][N] or NULL (natural order)
 *   block_count/idx   the mask of stage 2, or both NULL for dense causal attention (every J <= I)
 *   early_stop_theta  fp32 [Hq][NB] or NULL.  Block Sparse Flash Attention, Approach: for a kept
 *                     J != I the kernel computes the tile's exact scores; if their max over valid
 *                     (i, j) pairs, c * max q_i . k_j, is below theta[h][I], the V load and the
 *                     PV product are skipped and the tile leaves (m, l, acc) unchanged.
 *   out               out, fp32, strides o_stride_*
 *   lse               out, fp32 [Hq][N] natural-log LSE, or NULL
 *   kept_bitmap       out, uint32 [Hq][ceil(NB(NB+1)/2 / 32)], or NULL: bit I(I+1)/2 + J set for
 *                     every tile that was computed through PV; must be zeroed by the caller
 *   device_error      out, int32, or NULL: set to a non-zero code if an index in perm or the mask
 *                     is out of range (the offending entries are skipped); caller zeroes it
 *   workspace         >= pbsa_workspace_size(shape, PBSA_OP_ATTENTION) bytes (256 when N > 0),
 *                     256-byte aligned: the work queues of the persistent kernel, reset by this
 *                     call on the stream (calls sharing it must be ordered on one stream)
 */
pbsa_status pbsa_block_sparse_attn_prefill(const pbsa_shape* shape, const uint16_t* q,
                                           const uint16_t* k, const uint16_t* v,
                                           const int32_t* perm, const int32_t* block_count,
                                           const int32_t* block_idx,
                                           const float* early_stop_theta, float* out, float* lse,
                                           uint32_t* kept_bitmap, int32_t* device_error,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* Launch options of pbsa_block_sparse_attn_prefill_ex. */
typedef struct pbsa_launch_options {
  int32_t max_workgroups; /* >= 0: cap on the workgroups of the persistent kernel (0: as many as
                             fit on the device), e.g. to leave compute units to concurrent work */
  uint32_t flags;         /* PBSA_LAUNCH_* bits */
} pbsa_launch_options;

/* Workgroups take work items from the back of their home queue and steal from the front of the
 * others (the default order is the reverse: longest query rows first). */
#define PBSA_LAUNCH_CLAIM_BACK 1u

/*
 * pbsa_block_sparse_attn_prefill with launch options: the same operation, arguments, layouts,
 * results and errors.  The options change only how the persistent kernel of the mask and dense
 * paths spreads query rows over workgroups (the early-stop path launches one workgroup per query
 * block and head unit and ignores them); each row is computed by one workgroup in a fixed order,
 * so out, lse and kept_bitmap are bitwise the same under every option.
 *   options   NULL (defaults) or a pbsa_launch_options; max_workgroups < 0 or an unknown flag bit
 *             returns PBSA_ERR_INVALID_ARG
 */
pbsa_status pbsa_block_sparse_attn_prefill_ex(const pbsa_shape* shape, const uint16_t* q,
                                              const uint16_t* k, const uint16_t* v,
                                              const int32_t* perm, const int32_t* block_count,
                                              const int32_t* block_idx,
                                              const float* early_stop_theta, float* out, float* lse,
                                              uint32_t* kept_bitmap, int32_t* device_error,
                                              void* workspace, size_t workspace_bytes,
                                              const pbsa_launch_options* options, void* stream);

/*
 * pbsa_block_sparse_attn_prefill with a bf16 output: the same operation, arguments, layouts and
 * errors, except that out points to bf16 values (uint16_t bit patterns, [Hq][N][d] by the shape's
 * o strides in elements).  Each output element is the fp32 value pbsa_block_sparse_attn_prefill
 * writes, rounded to the nearest bf16 (ties to even), so callers whose next layer reads bf16 need
 * no separate conversion pass, and the output write is half as large.  lse stays fp32.
 */
pbsa_status pbsa_block_sparse_attn_prefill_bf16out(const pbsa_shape* shape, const uint16_t* q,
                                                   const uint16_t* k, const uint16_t* v,
                                                   const int32_t* perm, const int32_t* block_count,
                                                   const int32_t* block_idx,
                                                   const float* early_stop_theta, uint16_t* out,
                                                   float* lse, uint32_t* kept_bitmap,
                                                   int32_t* device_error, void* workspace,
                                                   size_t workspace_bytes, void* stream);

/*
 * pbsa_block_sparse_attn_prefill without a workspace, for callers that cannot allocate device
 * memory: code recorded under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, layouts, results and errors as pbsa_block_sparse_attn_prefill; the
 * work queues live in a 256-byte device array of the library instead (each GPU it runs on holds
 * its own copy until the process ends; its address is looked up on the first call on a device).
 * The call allocates nothing and calls no allocating routine.  Limit: the queues of one call take
 * 8 bytes per KV head, at most 64; a shape needing more than the array returns PBSA_ERR_WORKSPACE
 * (none does today).  Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call resets what it uses on its stream before its kernel): calls that overlap on
 * one GPU -- on different streams, or from several host threads without ordering -- race.
 */
pbsa_status pbsa_block_sparse_attn_prefill_noalloc(const pbsa_shape* shape, const uint16_t* q,
                                                   const uint16_t* k, const uint16_t* v,
                                                   const int32_t* perm, const int32_t* block_count,
                                                   const int32_t* block_idx,
                                                   const float* early_stop_theta, float* out,
                                                   float* lse, uint32_t* kept_bitmap,
                                                   int32_t* device_error, void* stream);

/*
 * Attention with the marginal-gain early stop (S2O, Early-Stopping Rule; Kernel Implementation).
 * block_count/block_idx must hold the ranked order of pbsa_estimate_block_mask with
 * PBSA_MASK_RANKED (every J <= I: the blocks of I's own segment first, then the earlier-segment
 * blocks by descending pooled logit).  For query block I of head h the list is processed in that
 * order; the blocks of I's own segment are always processed.  After each earlier-segment block b,
 * with l_i the softmax denominator of query i over every key processed so far (b included) and
 * dl_i the part b contributed, the row stops when dl_i < gain_tau * l_i for every query i of the
 * block (b itself stays processed).  out/lse are then softmax attention over the processed blocks,
 * keys gathered through perm as in pbsa_block_sparse_attn_prefill.  The kernel sums bf16-rounded
 * probabilities in fp32, so a decision within about 1% of the threshold can differ from an exact
 * evaluation.
 *   gain_tau     >= 0 and finite (0: never stop, every J <= I is processed)
 *   kept_bitmap  out, or NULL: bit I(I+1)/2 + J set for every processed block (caller zeroes it)
 *   other arguments as for pbsa_block_sparse_attn_prefill; segment_size must be > 0.
 */
pbsa_status pbsa_s2o_attn_prefill(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* perm, const int32_t* block_count,
                                  const int32_t* block_idx, float gain_tau, float* out, float* lse,
                                  uint32_t* kept_bitmap, int32_t* device_error, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Historical KV ranking (S2O, Methodology 1, Historical KV Permutation): the keys before each
 * segment ranked against a representative query of the segment.
 *
 * For KV head g and segment sigma >= 1 (segments of segment_size S, nseg = ceil(N / S)): the
 * representative r = mean of the query rows of segment sigma over the G query heads of g (fp64, from
 * the bf16 values); every key j < sigma*S (the causal prefix) gets the score r . k_j (fp64, then
 * rounded to fp32); the prefix is listed by score descending, equal fp32 scores by position.
 *
 *   kv_rank    out, int32 [Hkv][pbsa_prefix_rank_length(shape)]: segment sigma's order (key
 *              positions, a permutation of 0 .. sigma*S-1) at offset S*sigma*(sigma-1)/2
 *   workspace  >= pbsa_workspace_size(shape, PBSA_OP_PREFIX_RANK) bytes, 256-byte aligned
 * Requires segment_size > 0; PBSA_ERR_UNSUPPORTED for more than 256 segments or more than 2^31
 * entries over all KV heads.  Scores within one fp32 rounding of each other may come out in
 * position order rather than in exact fp64 order.
 */
pbsa_status pbsa_build_prefix_kv_ranking(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         int32_t* kv_rank, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Entries per KV head of the historical ranking, S * nseg * (nseg - 1) / 2, or -1 if the shape is
 * invalid or unsupported for it.  Host-only. */
int64_t pbsa_prefix_rank_length(const pbsa_shape* shape);

/*
 * Query permutation (S2O, Methodology 1, Query Permutation; PBS-Attn 1, query permutation
 * equivariance and the inverse transformation).
 *
 * For KV head g: the guide vector u = mean of the keys of g over the sequence (fp64); the score of
 * position i = (1/G) * sum over the G query heads of g of q_{h,i} . u (fp64); inside each segment
 * (segment_size S) the positions are listed by score descending, ties by position.
 *   qperm      out, int32 [Hkv][N]: entries a .. b-1 of each segment [a, b) are that segment's
 *              positions in this order; shared by the G query heads of g
 *   workspace  >= pbsa_workspace_size(shape, PBSA_OP_QUERY_PERM) bytes, 256-byte aligned
 * Requires segment_size > 0.
 */
pbsa_status pbsa_build_query_permutation(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         int32_t* qperm, void* workspace, size_t workspace_bytes,
                                         void* stream);

/*
 * S2O's two-pass attention with the marginal-gain early stop (Kernel Implementation; Early-Stopping
 * Rule).  For query block I of head h (segment sigma, first block J0 = sigma*S/B): pass 1 takes the
 * own segment's blocks J0 .. I in natural order (causal mask on the diagonal); pass 2 takes blocks
 * J = 0, 1, ..., J0-1 of the prefix order kv_rank (block J = the keys of ranks J*B .. J*B+B-1 of
 * segment sigma, KV head g(h)).  After each pass-2 block the row stops as in pbsa_s2o_attn_prefill
 * (every query's share of that block in its softmax denominator below gain_tau; that block stays
 * processed).  out/lse: softmax attention over the processed keys.
 *   kv_rank      from pbsa_build_prefix_kv_ranking (entries must lie in the segment's prefix: an
 *                entry outside it is skipped and sets bit 2 of device_error)
 *   qperm        from pbsa_build_query_permutation, or NULL (queries in natural order).  With it,
 *                query block I holds the queries at positions qperm[g][I*B ...], pass 1 takes every
 *                block of the own segment under the per-token causal mask (key j visible to the
 *                query at position i iff j <= i), and each output and lse row is written at the
 *                query's own position.  An entry outside its segment sets bit 4 (value 8) of
 *                device_error and that query is skipped (its row is not written).
 *   kept_bitmap  out, or NULL: one bit per processed entry J (J >= J0: natural block J; J < J0:
 *                prefix-order block J) of row (h, I): bit I(I+1)/2 + J, words
 *                ceil(NB(NB+1)/2 / 32) per head; with qperm bit I*NB + J, words ceil(NB*NB / 32)
 *                per head.  The caller zeroes it.
 *   other arguments as for pbsa_s2o_attn_prefill; segment_size must be > 0.
 */
pbsa_status pbsa_s2o_prefix_attn_prefill(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, const int32_t* kv_rank, const int32_t* qperm,
                                         float gain_tau, float* out, float* lse, uint32_t* kept_bitmap,
                                         int32_t* device_error, void* workspace,
                                         size_t workspace_bytes, void* stream);

/*
 * SampleAttention's block mask (SampleAttention, Technical Deep Dive: stage 1 trunk sampling,
 * stage 2 score-based filtering with decoupled filtering, a block-level mask).
 *
 * Stage 1: the sequence is cut into n_trunks chunks of C = ceil(N / n_trunks) positions; the last
 * rows_per_trunk positions of each are the sampled queries of every query head.  Their exact causal
 * softmax rows are computed in fp64 (the per-chunk exponentials stored as fp32, so each mass is
 * within 2^-24 relative of the exact one); col[h][j] is the mean over head h's sampled rows of p_ij and
 * slash[h][dlt] the mean of p_{i, i-dlt} (each sums to 1).  Stage 2: the columns and the slashes are
 * cut separately, each keeping the shortest prefix of (mass descending, index ascending) whose sum
 * reaches cia_tau (every index if cia_tau >= 1 or the sum stays below it).  Tile (I, J), J <= I, is
 * kept when block J holds a kept column, when a kept slash offset is realised by some pair of the
 * tile (i in I, j in J, j <= i, i - j = dlt), with PBSA_FORCE_DIAG for J = I and with
 * PBSA_FORCE_FIRST for J = 0.  Keys stay in natural order (perm = NULL for the attention call).
 *
 *   cia_tau        in (0, 1]
 *   n_trunks, rows_per_trunk  >= 1, and every chunk must hold rows_per_trunk positions
 *   block_count    out, int32 [Hq][NB]
 *   block_idx      out, int32 [Hq][NB(NB+1)/2], ascending J per row at I(I+1)/2
 *   col_mass, slash_mass  out, fp64 [Hq][N] each, or NULL
 *   workspace      >= pbsa_sample_mask_workspace_size(shape, n_trunks, rows_per_trunk) bytes,
 *                  256-byte aligned (it holds the sampled rows' exponentials: Hkv * G * n_trunks *
 *                  rows_per_trunk * N floats)
 */
pbsa_status pbsa_sample_attention_mask(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                       double cia_tau, int32_t n_trunks, int32_t rows_per_trunk,
                                       uint32_t flags, int32_t* block_count, int32_t* block_idx,
                                       double* col_mass, double* slash_mass, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Workspace bytes of pbsa_sample_attention_mask (0 when N = 0; SIZE_MAX for an invalid shape or
 * sampling).  Host-only. */
size_t pbsa_sample_mask_workspace_size(const pbsa_shape* shape, int32_t n_trunks, int32_t rows_per_trunk);

/*
 * Early-stop calibration helper (Block Sparse Flash Attention, Approach: offline thresholds).
 * tile_max[h][I(I+1)/2 + J] = c * max over i in block I, j in the key rows block J stands for when
 * read by I, j <= i, of q_i . k_j, for every J <= I -- the statistic stage 3's gate compares, on the
 * same rows and with the same fp32 accumulation.
 *   perm      nullable, int32 [Hkv][N]: as in pbsa_block_sparse_attn_prefill, a block of a segment
 *             before I's (shape->segment_size > 0) stands for the keys perm[g][J*B .. J*B+B-1]; NULL
 *             (or segment_size 0) gives natural order.  Thresholds for a permuted mask are calibrated
 *             with the calibration inputs' own permutation.
 *   tile_max  out, fp32 [Hq][NB(NB+1)/2]
 * A perm entry out of [0, N) reads a zero key row (no error word here).
 */
pbsa_status pbsa_tile_max(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                          float* tile_max, void* stream);

/*
 * Early-stop thresholds from calibration tile maxima (Block Sparse Flash Attention, Approach:
 * thresholds are set offline so that roughly the top `keep` tiles of each query block survive).
 *   tile_max  fp32 [Hq][NB(NB+1)/2], as written by pbsa_tile_max on calibration inputs
 *   keep      >= 1
 *   theta     out, fp32 [Hq][NB]: theta[h][I] = the keep-th largest of tile_max[h][I(I+1)/2 + J]
 *             over J <= I (one of those values, chosen exactly), or -inf when I + 1 <= keep
 * Returns PBSA_ERR_INVALID_ARG for null pointers or keep < 1.  NaN tile maxima are not expected.
 */
pbsa_status pbsa_calibrate_thresholds(const pbsa_shape* shape, const float* tile_max, int32_t keep,
                                      float* theta, void* stream);

/* Static description of a status code. */
const char* pbsa_status_string(pbsa_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t pbsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PBSA_H */
