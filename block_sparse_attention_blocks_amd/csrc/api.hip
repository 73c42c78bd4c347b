// C ABI of libpbsa: argument validation, workspace sizing and stream-ordered launches.
// Every check runs before anything is enqueued, so a rejected call leaves all outputs untouched.
#include "pbsa.h"

#include <math.h>
#include <stdint.h>

#include <atomic>

#include "estimate.h"

using pbsa::Geometry;

namespace {

constexpr int kMaxSegment = 8192;  // segment sort holds one segment in LDS
constexpr int kMaxBlocks = 2048;   // block selection holds one row of block scores in LDS
constexpr int kMaxPrefixSegments = 256;       // historical ranking: segments per sequence
constexpr int64_t kMaxRankEntries = 1ll << 31;  // historical ranking: entries over all KV heads

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fill g from the caller's shape.  Returns PBSA_OK or the reason the shape is rejected.
pbsa_status make_geometry(const pbsa_shape* s, Geometry* g) {
  if (!s) return PBSA_ERR_INVALID_ARG;
  if (s->seq_len < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0) return PBSA_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return PBSA_ERR_INVALID_ARG;
  if (s->block_size <= 0 || s->segment_size < 0 || s->head_dim <= 0) return PBSA_ERR_INVALID_ARG;
  if (s->segment_size % s->block_size != 0) return PBSA_ERR_INVALID_ARG;
  if (!(s->softmax_scale == s->softmax_scale) || isinf(s->softmax_scale)) return PBSA_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return PBSA_ERR_UNSUPPORTED;
  if (s->block_size != 64 && s->block_size != 128) return PBSA_ERR_UNSUPPORTED;
  if (s->segment_size > kMaxSegment) return PBSA_ERR_UNSUPPORTED;
  const int64_t nb = ((int64_t)s->seq_len + s->block_size - 1) / s->block_size;
  if (nb > kMaxBlocks) return PBSA_ERR_UNSUPPORTED;
  const int d = s->head_dim;
  // strides: (0, 0) means contiguous [heads][tokens][d]; otherwise token stride >= d, both
  // non-negative and multiples of 8 elements (16-byte rows for bf16, 32-byte for fp32 out)
  auto strides = [&](int64_t sh, int64_t st, int64_t* osh, int64_t* ost) -> bool {
    if (sh == 0 && st == 0) {
      *ost = d;
      *osh = (int64_t)s->seq_len * d;
      return true;
    }
    if (sh < 0 || st < d || (sh % 8) != 0 || (st % 8) != 0) return false;
    *osh = sh;
    *ost = st;
    return true;
  };
  if (!strides(s->q_stride_head, s->q_stride_token, &g->qsh, &g->qst)) return PBSA_ERR_INVALID_ARG;
  if (!strides(s->kv_stride_head, s->kv_stride_token, &g->kvsh, &g->kvst)) return PBSA_ERR_INVALID_ARG;
  if (!strides(s->o_stride_head, s->o_stride_token, &g->osh, &g->ost)) return PBSA_ERR_INVALID_ARG;
  // kernels address one head's rows with 32-bit byte offsets, and a whole tensor with 64-bit ones:
  // the byte extent of one head of q, k, v must stay below 2^31, and that of every tensor (all its
  // heads) below 2^48, more than any device address space holds; computed without overflow
  const int64_t N = s->seq_len;
  auto head_bytes_ok = [&](int64_t st) {
    int64_t b = 0;
    return !__builtin_mul_overflow(N, st, &b) && !__builtin_mul_overflow(b, (int64_t)2, &b) && b < ((int64_t)1 << 31);
  };
  auto extent_ok = [&](int64_t heads, int64_t sh, int64_t st, int64_t elem_bytes) {
    if (N == 0) return true;
    int64_t a = 0, b = 0, e = 0;
    if (__builtin_mul_overflow(heads - 1, sh, &a) || __builtin_mul_overflow(N - 1, st, &b)) return false;
    if (__builtin_add_overflow(a, b, &e) || __builtin_add_overflow(e, (int64_t)d, &e)) return false;
    return !__builtin_mul_overflow(e, elem_bytes, &e) && e < ((int64_t)1 << 48);
  };
  if (!head_bytes_ok(g->qst) || !head_bytes_ok(g->kvst)) return PBSA_ERR_UNSUPPORTED;
  if (!extent_ok(s->num_q_heads, g->qsh, g->qst, 2) || !extent_ok(s->num_kv_heads, g->kvsh, g->kvst, 2) ||
      !extent_ok(s->num_q_heads, g->osh, g->ost, 4))
    return PBSA_ERR_UNSUPPORTED;
  g->N = s->seq_len;
  g->Hq = s->num_q_heads;
  g->Hkv = s->num_kv_heads;
  g->G = s->num_q_heads / s->num_kv_heads;
  g->d = d;
  g->B = s->block_size;
  g->S = s->segment_size;
  g->NB = (int)nb;
  g->scale64 = s->softmax_scale > 0.f ? (double)s->softmax_scale : 1.0 / sqrt((double)d);
  g->scale = (float)g->scale64;
  return PBSA_OK;
}

pbsa_status check_workspace(size_t need, const void* ws, size_t bytes) {
  if (need == 0) return PBSA_OK;
  if (!ws || bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return PBSA_ERR_WORKSPACE;
  return PBSA_OK;
}

pbsa_status from_hip(hipError_t e) { return e == hipSuccess ? PBSA_OK : PBSA_ERR_HIP; }

// Shapes the historical ranking supports: segments on, at most kMaxPrefixSegments of them, and a
// ranking that fits kMaxRankEntries.
bool prefix_rank_ok(const Geometry& g) {
  if (g.S <= 0) return false;
  const int64_t nseg = ((int64_t)g.N + g.S - 1) / g.S;
  if (nseg > kMaxPrefixSegments) return false;
  return (int64_t)g.Hkv * pbsa::prefix_rank_length(g) <= kMaxRankEntries;
}

}  // namespace

extern "C" {

size_t pbsa_workspace_size(const pbsa_shape* shape, int op) {
  Geometry g;
  if (make_geometry(shape, &g) != PBSA_OK) return SIZE_MAX;
  switch (op) {
    case PBSA_OP_PERMUTATION: return pbsa::importance_workspace_bytes(g);
    case PBSA_OP_MASK: return pbsa::mask_workspace_bytes(g);
    case PBSA_OP_ATTENTION: return g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0;
    case PBSA_OP_PREFIX_RANK: return prefix_rank_ok(g) ? pbsa::prefix_rank_workspace_bytes(g) : SIZE_MAX;
    case PBSA_OP_QUERY_PERM: return g.S > 0 ? (g.N > 0 ? pbsa::query_perm_workspace_bytes(g) : 0) : SIZE_MAX;
    default: return SIZE_MAX;
  }
}

int64_t pbsa_prefix_rank_length(const pbsa_shape* shape) {
  Geometry g;
  if (make_geometry(shape, &g) != PBSA_OK || !prefix_rank_ok(g)) return -1;
  return pbsa::prefix_rank_length(g);
}

pbsa_status pbsa_build_prefix_kv_ranking(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         int32_t* kv_rank, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (g.S <= 0) return PBSA_ERR_INVALID_ARG;
  if (!prefix_rank_ok(g)) return PBSA_ERR_UNSUPPORTED;
  if (!q || !k || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  const int64_t L = pbsa::prefix_rank_length(g);
  if (L > 0 && !kv_rank) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(L > 0 ? pbsa::prefix_rank_workspace_bytes(g) : 0, workspace, workspace_bytes)) !=
      PBSA_OK)
    return st;
  if (L == 0) return PBSA_OK;
  return from_hip(pbsa::launch_prefix_rank(g, q, k, kv_rank, workspace, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_build_segment_permutation(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                           int32_t* perm, double* importance, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (g.S <= 0) return PBSA_ERR_INVALID_ARG;
  if (!q || !k || !perm || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  if (importance && (reinterpret_cast<uintptr_t>(importance) & 7u)) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(pbsa::importance_workspace_bytes(g), workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_build_permutation(g, q, k, perm, importance, workspace,
                                                 static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_estimate_block_mask(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                     const int32_t* perm, double mass_tau, uint32_t flags, int32_t* block_count,
                                     int32_t* block_idx, double* block_prob, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (!q || !k || !block_count || !block_idx || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  if (perm && g.S <= 0) return PBSA_ERR_INVALID_ARG;
  if (!(mass_tau > 0.0 && mass_tau <= 1.0)) return PBSA_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(PBSA_FORCE_DIAG | PBSA_FORCE_FIRST | PBSA_MASK_RANKED)) return PBSA_ERR_INVALID_ARG;
  if ((flags & PBSA_MASK_RANKED) && (g.S <= 0 || block_prob)) return PBSA_ERR_INVALID_ARG;
  if (block_prob && (reinterpret_cast<uintptr_t>(block_prob) & 7u)) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(pbsa::mask_workspace_bytes(g), workspace, workspace_bytes)) != PBSA_OK) return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_block_mask(g, q, k, perm, mass_tau, flags, block_count, block_idx, block_prob,
                                          workspace, static_cast<hipStream_t>(stream)));
}

namespace {
pbsa_status check_attn_args(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* perm, const int32_t* block_count, const int32_t* block_idx, float* out,
                            Geometry* g) {
  pbsa_status st = make_geometry(shape, g);
  if (st != PBSA_OK) return st;
  if (!q || !k || !v || !out) return PBSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PBSA_ERR_INVALID_ARG;
  if ((block_count == nullptr) != (block_idx == nullptr)) return PBSA_ERR_INVALID_ARG;
  if (perm && g->S <= 0) return PBSA_ERR_INVALID_ARG;
  return PBSA_OK;
}
}  // namespace

pbsa_status pbsa_block_sparse_attn_prefill(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                           const uint16_t* v, const int32_t* perm, const int32_t* block_count,
                                           const int32_t* block_idx, const float* early_stop_theta, float* out,
                                           float* lse, uint32_t* kept_bitmap, int32_t* device_error,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = check_attn_args(shape, q, k, v, perm, block_count, block_idx, out, &g);
  if (st != PBSA_OK) return st;
  if ((st = check_workspace(g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0, workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_attention(g, q, k, v, perm, block_count, block_idx, early_stop_theta, out, lse,
                                         kept_bitmap, device_error, workspace, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_block_sparse_attn_prefill_ex(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                              const uint16_t* v, const int32_t* perm, const int32_t* block_count,
                                              const int32_t* block_idx, const float* early_stop_theta, float* out,
                                              float* lse, uint32_t* kept_bitmap, int32_t* device_error,
                                              void* workspace, size_t workspace_bytes,
                                              const pbsa_launch_options* options, void* stream) {
  pbsa::LaunchOpts opt;
  if (options) {
    if (options->max_workgroups < 0 || (options->flags & ~PBSA_LAUNCH_CLAIM_BACK) != 0) return PBSA_ERR_INVALID_ARG;
    opt.max_wg = options->max_workgroups;
    opt.claim_back = (options->flags & PBSA_LAUNCH_CLAIM_BACK) != 0;
  }
  Geometry g;
  pbsa_status st = check_attn_args(shape, q, k, v, perm, block_count, block_idx, out, &g);
  if (st != PBSA_OK) return st;
  if ((st = check_workspace(g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0, workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_attention(g, q, k, v, perm, block_count, block_idx, early_stop_theta, out, lse,
                                         kept_bitmap, device_error, workspace, static_cast<hipStream_t>(stream),
                                         opt));
}

pbsa_status pbsa_block_sparse_attn_prefill_bf16out(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                                   const uint16_t* v, const int32_t* perm,
                                                   const int32_t* block_count, const int32_t* block_idx,
                                                   const float* early_stop_theta, uint16_t* out, float* lse,
                                                   uint32_t* kept_bitmap, int32_t* device_error, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  // the kernels take the output as an fp32 pointer and store bf16 through it when out_bf16 is set
  float* out_any = reinterpret_cast<float*>(out);
  Geometry g;
  pbsa_status st = check_attn_args(shape, q, k, v, perm, block_count, block_idx, out_any, &g);
  if (st != PBSA_OK) return st;
  if ((st = check_workspace(g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0, workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  pbsa::LaunchOpts opt;
  opt.out_bf16 = true;
  return from_hip(pbsa::launch_attention(g, q, k, v, perm, block_count, block_idx, early_stop_theta, out_any, lse,
                                         kept_bitmap, device_error, workspace, static_cast<hipStream_t>(stream),
                                         opt));
}

// Device memory of pbsa_block_sparse_attn_prefill_noalloc: the work deques that the pipelined
// attention kernels otherwise keep in the caller's workspace (one 64-bit word per deque, reset by
// a kernel on the stream before every launch).  Every GPU the library runs on holds its own copy
// of this array until the process ends.  On the host, `scratch` is only a stand-in for the symbol:
// its device address is looked up per device with hipGetSymbolAddress and used everywhere instead.
constexpr size_t kNoAllocScratchBytes = 256;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];  // device address of `scratch`, per device ordinal

// Address of the current device's copy of `scratch`: looked up on the first call on that device
// (with the device current) and kept.  Concurrent first calls look up the same address.
pbsa_status scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PBSA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PBSA_ERR_UNSUPPORTED;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return PBSA_ERR_HIP;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PBSA_OK;
}
}  // namespace

pbsa_status pbsa_block_sparse_attn_prefill_noalloc(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                                   const uint16_t* v, const int32_t* perm,
                                                   const int32_t* block_count, const int32_t* block_idx,
                                                   const float* early_stop_theta, float* out, float* lse,
                                                   uint32_t* kept_bitmap, int32_t* device_error, void* stream) {
  Geometry g;
  pbsa_status st = check_attn_args(shape, q, k, v, perm, block_count, block_idx, out, &g);
  if (st != PBSA_OK) return st;
  if (g.N == 0) return PBSA_OK;
  // the deques of this shape (one word per KV group, at most kMaxDeques) must fit the array
  const size_t need = sizeof(unsigned long long) * (size_t)(g.Hkv < pbsa::kMaxDeques ? g.Hkv : pbsa::kMaxDeques);
  if (need > kNoAllocScratchBytes) return PBSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != PBSA_OK) return st;
  return from_hip(pbsa::launch_attention(g, q, k, v, perm, block_count, block_idx, early_stop_theta, out, lse,
                                         kept_bitmap, device_error, ws, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_s2o_attn_prefill(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                  const uint16_t* v, const int32_t* perm, const int32_t* block_count,
                                  const int32_t* block_idx, float gain_tau, float* out, float* lse,
                                  uint32_t* kept_bitmap, int32_t* device_error, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (!q || !k || !v || !out || !block_count || !block_idx) return PBSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PBSA_ERR_INVALID_ARG;
  if (g.S <= 0 || !(gain_tau >= 0.f) || !(gain_tau < INFINITY)) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0, workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_s2o_attention(g, q, k, v, perm, block_count, block_idx, gain_tau, out, lse,
                                             kept_bitmap, device_error, workspace,
                                             static_cast<hipStream_t>(stream)));
}

namespace {
// Trunk sampling needs every one of the n_trunks chunks (ceil(N / n_trunks) positions each, the
// last one shorter) to hold rows_per_trunk positions.
bool trunks_ok(const Geometry& g, int n_trunks, int rpt) {
  if (n_trunks < 1 || rpt < 1 || g.N < 1) return false;
  const int64_t C = ((int64_t)g.N + n_trunks - 1) / n_trunks;
  return (int64_t)(n_trunks - 1) * C + rpt <= g.N;
}
}  // namespace

size_t pbsa_sample_mask_workspace_size(const pbsa_shape* shape, int32_t n_trunks, int32_t rows_per_trunk) {
  Geometry g;
  if (make_geometry(shape, &g) != PBSA_OK) return SIZE_MAX;
  if (g.N == 0) return 0;
  if (!trunks_ok(g, n_trunks, rows_per_trunk)) return SIZE_MAX;
  return pbsa::sample_mask_workspace_bytes(g, n_trunks, rows_per_trunk);
}

pbsa_status pbsa_sample_attention_mask(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k, double cia_tau,
                                       int32_t n_trunks, int32_t rows_per_trunk, uint32_t flags,
                                       int32_t* block_count, int32_t* block_idx, double* col_mass,
                                       double* slash_mass, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (!q || !k || !block_count || !block_idx || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  if (!(cia_tau > 0.0 && cia_tau <= 1.0)) return PBSA_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(PBSA_FORCE_DIAG | PBSA_FORCE_FIRST)) return PBSA_ERR_INVALID_ARG;
  if ((col_mass && (reinterpret_cast<uintptr_t>(col_mass) & 7u)) ||
      (slash_mass && (reinterpret_cast<uintptr_t>(slash_mass) & 7u)))
    return PBSA_ERR_INVALID_ARG;
  if (g.N == 0) return PBSA_OK;
  if (!trunks_ok(g, n_trunks, rows_per_trunk)) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(pbsa::sample_mask_workspace_bytes(g, n_trunks, rows_per_trunk), workspace,
                            workspace_bytes)) != PBSA_OK)
    return st;
  return from_hip(pbsa::launch_sample_mask(g, q, k, cia_tau, n_trunks, rows_per_trunk, flags, block_count,
                                           block_idx, col_mass, slash_mass, workspace,
                                           static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_build_query_permutation(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         int32_t* qperm, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (g.S <= 0) return PBSA_ERR_INVALID_ARG;
  if (!q || !k || !qperm || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(g.N > 0 ? pbsa::query_perm_workspace_bytes(g) : 0, workspace, workspace_bytes)) !=
      PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_query_permutation(g, q, k, qperm, workspace, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_s2o_prefix_attn_prefill(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k,
                                         const uint16_t* v, const int32_t* kv_rank, const int32_t* qperm,
                                         float gain_tau, float* out, float* lse, uint32_t* kept_bitmap,
                                         int32_t* device_error, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (g.S <= 0 || !(gain_tau >= 0.f) || !(gain_tau < INFINITY)) return PBSA_ERR_INVALID_ARG;
  if (!prefix_rank_ok(g)) return PBSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out) return PBSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return PBSA_ERR_INVALID_ARG;
  const int64_t L = pbsa::prefix_rank_length(g);
  if (L > 0 && !kv_rank) return PBSA_ERR_INVALID_ARG;
  if ((st = check_workspace(g.N > 0 ? pbsa::kAttnWorkspaceBytes : 0, workspace, workspace_bytes)) != PBSA_OK)
    return st;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_s2o_prefix_attention(g, q, k, v, kv_rank, L, qperm, gain_tau, out, lse, kept_bitmap,
                                                    device_error, workspace, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_tile_max(const pbsa_shape* shape, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                          float* tile_max, void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (!q || !k || !tile_max || !aligned16(q) || !aligned16(k)) return PBSA_ERR_INVALID_ARG;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_tile_max(g, q, k, perm, tile_max, static_cast<hipStream_t>(stream)));
}

pbsa_status pbsa_calibrate_thresholds(const pbsa_shape* shape, const float* tile_max, int32_t keep, float* theta,
                                      void* stream) {
  Geometry g;
  pbsa_status st = make_geometry(shape, &g);
  if (st != PBSA_OK) return st;
  if (!tile_max || !theta || keep < 1) return PBSA_ERR_INVALID_ARG;
  if (g.N == 0) return PBSA_OK;
  return from_hip(pbsa::launch_calibrate(g.Hq, g.NB, tile_max, keep, theta, static_cast<hipStream_t>(stream)));
}

const char* pbsa_status_string(pbsa_status status) {
  switch (status) {
    case PBSA_OK: return "ok";
    case PBSA_ERR_INVALID_ARG: return "invalid argument";
    case PBSA_ERR_UNSUPPORTED: return "unsupported shape";
    case PBSA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case PBSA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int32_t pbsa_version(void) { return 100; }

}  // extern "C"
