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

// Max over the 64 lanes, in every lane, with no LDS round trip: four DPP row rotations leave each
// 16-lane row's max in all its lanes, then the partners l ^ 16 (permlane16 swap) and l ^ 32
// (permlane32 swap) are folded in.  A max is exact in any order, so the result is the same value
// the butterfly through ds_bpermute gives, at a fraction of its latency.
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false)));
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Wave64 sums and maxima of doubles through cross-lane swizzles.

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

// Stage 3 and calibration.
// Attention workspace: the work deques of the pipelined kernels, one 64-bit word per deque.
constexpr int kMaxDeques = 8;
constexpr size_t kAttnWorkspaceBytes = 256;
// Launch options of the persistent attention kernels: at most max_wg workgroups (0 = as many as
// fit on the device), and the order in which they take work items.
struct LaunchOpts {
  int max_wg = 0;
  bool claim_back = false;
  bool out_bf16 = false;  // out is bf16 storage (same element strides), rounded to nearest even
};
hipError_t launch_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* perm, const int32_t* count, const int32_t* idx,
                            const float* theta, float* out, float* lse, uint32_t* kept, int32_t* err,
                            void* ws, hipStream_t st, const LaunchOpts& opt = LaunchOpts());
hipError_t launch_s2o_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const int32_t* perm, const int32_t* count, const int32_t* idx, float gain_tau,
                                float* out, float* lse, uint32_t* kept, int32_t* err, void* ws, hipStream_t st);
hipError_t launch_s2o_prefix_attention(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const int32_t* kv_rank, int64_t rank_len, const int32_t* qperm,
                                       float gain_tau, float* out, float* lse, uint32_t* kept, int32_t* err,
                                       void* ws, hipStream_t st);
hipError_t launch_tile_max(const Geometry& g, const uint16_t* q, const uint16_t* k, const int32_t* perm,
                           float* tmax, hipStream_t st);
hipError_t launch_calibrate(int Hq, int NB, const float* tmax, int keep, float* theta, hipStream_t st);

}  // namespace pbsa
