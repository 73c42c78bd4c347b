// Launch-side declarations of the estimation stages of libpbsa (key importance and permutation,
// block masks, S2O rankings, SampleAttention), kept apart from the attention kernels' header.
#pragma once

#include "common.h"

namespace pbsa {

// Stage 1 workspace layout and launches.
size_t importance_workspace_bytes(const Geometry& g);
// Importance (into imp, or into the workspace when imp is NULL) followed by the segment sort.
hipError_t launch_build_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* perm,
                                    double* imp, void* ws, hipStream_t st);

// Sort of fp64 scores [Hkv][N] inside segments of g.S: descending, ties by position, into perm.
hipError_t launch_segment_sort(const Geometry& g, const double* score, int32_t* perm, hipStream_t st);

// SampleAttention stage 1: exact causal softmax rows of trunk-sampled queries, stored as in the
// importance pass (p[r][j] = e[g][r][j] * exp(part_m[g][j / 64][r] - lse[g][r]), e rounded to fp32).
struct SampledRows {
  float* e;        // [Hkv][R][N] chunk-normalised exponentials (0 where j > i), fp32
  double* part_m;  // [Hkv][nchunk][R] chunk maxima (-inf for a chunk wholly past the row)
  double* lse;     // [Hkv][R]
  int R;           // rows per KV head: G * n_trunks * rpt, head-major
  int nchunk;      // key chunks of 64
};
size_t sampled_softmax_workspace_bytes(const Geometry& g, int n_trunks, int rpt);
hipError_t launch_sampled_softmax(const Geometry& g, const uint16_t* q, const uint16_t* k, int n_trunks, int rpt,
                                  void* ws, SampledRows* out, hipStream_t st);
size_t sample_mask_workspace_bytes(const Geometry& g, int n_trunks, int rpt);
hipError_t launch_sample_mask(const Geometry& g, const uint16_t* q, const uint16_t* k, double cia_tau, int n_trunks,
                              int rpt, uint32_t flags, int32_t* count, int32_t* idx, double* col, double* slash,
                              void* ws, hipStream_t st);

// Stage 2.
size_t mask_workspace_bytes(const Geometry& g);
constexpr uint32_t kMaskRanked = 4u;  // PBSA_MASK_RANKED
hipError_t launch_block_mask(const Geometry& g, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                             double tau, uint32_t flags, int32_t* count, int32_t* idx, double* prob,
                             void* ws, hipStream_t st);

// Historical KV ranking of S2O: workspace, entries per KV head, and the launch (kv_rank int32
// [Hkv][rank_len]).
size_t prefix_rank_workspace_bytes(const Geometry& g);
int64_t prefix_rank_length(const Geometry& g);
hipError_t launch_prefix_rank(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* kv_rank, void* ws,
                              hipStream_t st);
// S2O query permutation: workspace and launch (qperm int32 [Hkv][N]).
size_t query_perm_workspace_bytes(const Geometry& g);
hipError_t launch_query_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* qperm, void* ws,
                                    hipStream_t st);

}  // namespace pbsa
