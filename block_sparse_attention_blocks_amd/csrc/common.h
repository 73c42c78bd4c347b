// Shared device helpers and launch-side types of libpbsa (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Problem geometry after validation (strides in elements, defaults filled in).
struct Geometry {
  int N, Hq, Hkv, G, d, B, S, NB;
  double scale64;  // logit scale c for the fp64 estimation stages
  float scale;     // the same c rounded to fp32 for the attention kernels
  int64_t qsh, qst;    // q head / token strides
  int64_t kvsh, kvst;  // k and v head / token strides
  int64_t osh, ost;    // out head / token strides
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Raw buffer access: a 128-bit resource with a byte bound; loads at offsets >= the bound return
// zero without touching memory, which is how out-of-range rows are padded without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset >= every bound the library creates

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

__device__ __forceinline__ int tri_offset(int I) { return (I * (I + 1)) >> 1; }

// Wave64 reductions through cross-lane swizzles.
__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  return x;
}

// ---------------------------------------------------------------- launchers (internal C++ API)

// Stage 1 workspace layout and launches.
size_t importance_workspace_bytes(const Geometry& g);
// Importance (into imp, or into the workspace when imp is NULL) followed by the segment sort.
hipError_t launch_build_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* perm,
                                    double* imp, void* ws, hipStream_t st);

// Sort of fp64 scores [Hkv][N] inside segments of g.S: descending, ties by position, into perm.
hipError_t launch_segment_sort(const Geometry& g, const double* score, int32_t* perm, hipStream_t st);

// SampleAttention stage 1: exact causal softmax rows of trunk-sampled queries, stored as in the
// importance pass (p[r][j] = e[g][r][j] * exp(part_m[g][j / 64][r] - lse[g][r])).
struct SampledRows {
  double* e;       // [Hkv][R][N] chunk-normalised exponentials (0 where j > i)
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

// Stage 3 and calibration.
// Attention workspace: the work deques of the pipelined kernels, one 64-bit word per deque.
constexpr int kMaxDeques = 8;
constexpr size_t kAttnWorkspaceBytes = 256;
hipError_t launch_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* perm, const int32_t* count, const int32_t* idx,
                            const float* theta, float* out, float* lse, uint32_t* kept, int32_t* err,
                            void* ws, hipStream_t st);
hipError_t launch_s2o_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* perm, const int32_t* count, const int32_t* idx, float gain_tau,
                                float* out, float* lse, uint32_t* kept, int32_t* err, void* ws, hipStream_t st);
// Historical KV ranking of S2O: workspace, entries per KV head, and the launch (kv_rank int32
// [Hkv][rank_len]).
size_t prefix_rank_workspace_bytes(const Geometry& g);
int64_t prefix_rank_length(const Geometry& g);
hipError_t launch_prefix_rank(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* kv_rank, void* ws,
                              hipStream_t st);
hipError_t launch_s2o_prefix_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const int32_t* kv_rank, int64_t rank_len, const int32_t* qperm,
                                       float gain_tau, float* out, float* lse, uint32_t* kept, int32_t* err,
                                       void* ws, hipStream_t st);
// S2O query permutation: workspace and launch (qperm int32 [Hkv][N]).
size_t query_perm_workspace_bytes(const Geometry& g);
hipError_t launch_query_permutation(const Geometry& g, const uint16_t* q, const uint16_t* k, int32_t* qperm, void* ws,
                                    hipStream_t st);
hipError_t launch_tile_max(const Geometry& g, const uint16_t* q, const uint16_t* k, float* tmax,
                           hipStream_t st);
hipError_t launch_calibrate(int Hq, int NB, const float* tmax, int keep, float* theta, hipStream_t st);

}  // namespace pbsa
