// The argument-validation cases of the C ABI, as a plain C++ program for a host build of the
// library under AddressSanitizer and UndefinedBehaviorSanitizer.  Every call is either rejected
// before the library touches the GPU or is an N = 0 no-op, so the program needs no device; the
// pointers it passes are never dereferenced.  The same cases run through ctypes in test_abi.py.
// Exit status: 0 when every case returns the expected status, 1 otherwise (a sanitizer report
// aborts the program with its own status).
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "pbsa.h"

namespace {

int g_failures = 0;
int g_checks = 0;

#define EXPECT_EQ(expr, want)                                                                  \
  do {                                                                                         \
    ++g_checks;                                                                                \
    const long long got_ = (long long)(expr);                                                  \
    const long long want_ = (long long)(want);                                                 \
    if (got_ != want_) {                                                                       \
      ++g_failures;                                                                            \
      fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #expr, got_, want_); \
    }                                                                                          \
  } while (0)

#define EXPECT_TRUE(cond)                                                      \
  do {                                                                         \
    ++g_checks;                                                                \
    if (!(cond)) {                                                             \
      ++g_failures;                                                            \
      fprintf(stderr, "%s:%d: %s does not hold\n", __FILE__, __LINE__, #cond); \
    }                                                                          \
  } while (0)

// 16-byte aligned addresses that validation accepts as tensors and never dereferences
uint16_t* const FQ = reinterpret_cast<uint16_t*>(0x10000);
int32_t* const FI = reinterpret_cast<int32_t*>(0x10000);
float* const FF = reinterpret_cast<float*>(0x10000);
double* const FD = reinterpret_cast<double*>(0x10000);
void* const FW = reinterpret_cast<void*>(0x10000);  // also 256-byte aligned
const size_t BIG = (size_t)1 << 40;
const size_t SMAX = (size_t)-1;

pbsa_shape shape(int N = 1024, int Hq = 4, int Hkv = 2, int d = 128, int B = 128, int S = 512, float scale = 0.f) {
  pbsa_shape s = {};
  s.seq_len = N;
  s.num_q_heads = Hq;
  s.num_kv_heads = Hkv;
  s.head_dim = d;
  s.block_size = B;
  s.segment_size = S;
  s.softmax_scale = scale;
  return s;
}

void status_strings() {
  for (int st = 0; st < 5; ++st) EXPECT_TRUE(pbsa_status_string((pbsa_status)st)[0] != '\0');
  EXPECT_TRUE(pbsa_version() >= 100);
}

void workspace_sizes_monotone_in_n() {
  const int ops[] = {PBSA_OP_PERMUTATION, PBSA_OP_MASK, PBSA_OP_ATTENTION};
  const int ns[] = {0, 1, 127, 128, 129, 1000, 4096, 32768, 131072};
  for (int op : ops) {
    size_t prev = 0;
    for (int N : ns) {
      pbsa_shape s = shape(N);
      const size_t n = pbsa_workspace_size(&s, op);
      EXPECT_TRUE(n != SMAX);
      EXPECT_TRUE(n >= prev);
      prev = n;
    }
  }
  pbsa_shape s = shape();
  EXPECT_TRUE(pbsa_workspace_size(&s, 7) == SMAX);
}

void shape_validation() {
  struct Case {
    pbsa_shape s;
    pbsa_status want;
  };
  const Case cases[] = {
      {shape(1024, 4, 2, 96), PBSA_ERR_UNSUPPORTED},
      {shape(1024, 4, 2, 128, 32), PBSA_ERR_UNSUPPORTED},
      {shape(1024, 4, 2, 128, 128, 16384), PBSA_ERR_UNSUPPORTED},
      {shape(128 * 2049), PBSA_ERR_UNSUPPORTED},
      {shape(1024, 4, 2, 128, 128, 192), PBSA_ERR_INVALID_ARG},  // S not a multiple of B
      {shape(1024, 6, 4), PBSA_ERR_INVALID_ARG},                 // Hq % Hkv
      {shape(-1), PBSA_ERR_INVALID_ARG},
      {shape(1024, 4, 0), PBSA_ERR_INVALID_ARG},
      {shape(1024, 4, 2, 128, 128, 512, NAN), PBSA_ERR_INVALID_ARG},
  };
  for (const Case& c : cases) {
    const pbsa_shape* s = &c.s;
    EXPECT_TRUE(pbsa_workspace_size(s, 0) == SMAX);
    EXPECT_EQ(pbsa_build_segment_permutation(s, FQ, FQ, FI, nullptr, FW, BIG, nullptr), c.want);
    EXPECT_EQ(pbsa_estimate_block_mask(s, FQ, FQ, nullptr, 0.9, 3, FI, FI, nullptr, FW, BIG, nullptr), c.want);
    EXPECT_EQ(pbsa_block_sparse_attn_prefill(s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                             nullptr, nullptr, 0, nullptr),
              c.want);
    EXPECT_EQ(pbsa_tile_max(s, FQ, FQ, nullptr, FF, nullptr), c.want);
  }
}

void null_shape_and_pointers() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  EXPECT_EQ(pbsa_build_segment_permutation(nullptr, FQ, FQ, FI, nullptr, FW, BIG, nullptr), E);
  pbsa_shape s = shape();
  EXPECT_EQ(pbsa_build_segment_permutation(&s, nullptr, FQ, FI, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_segment_permutation(&s, FQ, FQ, nullptr, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, nullptr, 0.9, 3, nullptr, FI, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, nullptr, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                           nullptr, nullptr, nullptr, 0, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, FI, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, nullptr, 0, nullptr),
            E);  // count without idx
  uint16_t* bad = reinterpret_cast<uint16_t*>(0x10002);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, bad, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, nullptr, 0, nullptr),
            E);  // misaligned tensor
  EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, nullptr, nullptr), E);
  EXPECT_EQ(pbsa_calibrate_thresholds(&s, nullptr, 64, FF, nullptr), E);
  EXPECT_EQ(pbsa_calibrate_thresholds(&s, FF, 64, nullptr, nullptr), E);
  EXPECT_EQ(pbsa_calibrate_thresholds(&s, FF, 0, FF, nullptr), E);
}

void permutation_and_mask_arguments() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  pbsa_shape s0 = shape(1024, 4, 2, 128, 128, 0);
  EXPECT_EQ(pbsa_build_segment_permutation(&s0, FQ, FQ, FI, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_estimate_block_mask(&s0, FQ, FQ, FI, 0.9, 3, FI, FI, nullptr, FW, BIG, nullptr), E);
  pbsa_shape s = shape();
  const double taus[] = {0.0, -0.5, 1.0000001, NAN};
  for (double tau : taus)
    EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, nullptr, tau, 3, FI, FI, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, nullptr, 0.9, 8, FI, FI, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_estimate_block_mask(&s0, FQ, FQ, nullptr, 0.9, PBSA_MASK_RANKED, FI, FI, nullptr, FW, BIG, nullptr),
            E);  // the ranked order needs segments
  EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, FI, 0.9, PBSA_MASK_RANKED, FI, FI, FD, FW, BIG, nullptr),
            E);  // and writes no probabilities
}

void marginal_gain_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  pbsa_shape s = shape();
  auto call = [&](const pbsa_shape& sh, const int32_t* cnt, const int32_t* idx, float tau) {
    return pbsa_s2o_attn_prefill(&sh, FQ, FQ, FQ, nullptr, cnt, idx, tau, FF, nullptr, nullptr, nullptr, FW,
                                 (size_t)1 << 20, nullptr);
  };
  EXPECT_EQ(call(s, nullptr, FI, 0.01f), E);
  EXPECT_EQ(call(s, FI, nullptr, 0.01f), E);
  EXPECT_EQ(call(s, FI, FI, -0.5f), E);
  EXPECT_EQ(call(s, FI, FI, NAN), E);
  EXPECT_EQ(call(s, FI, FI, INFINITY), E);
  EXPECT_EQ(call(shape(1024, 4, 2, 128, 128, 0), FI, FI, 0.01f), E);
  EXPECT_EQ(pbsa_s2o_attn_prefill(&s, FQ, FQ, FQ, nullptr, FI, FI, 0.01f, FF, nullptr, nullptr, nullptr, nullptr, 0,
                                  nullptr),
            PBSA_ERR_WORKSPACE);
  EXPECT_EQ(call(shape(0), FI, FI, 0.01f), PBSA_OK);
}

void workspace_checks() {
  const pbsa_status W = PBSA_ERR_WORKSPACE;
  pbsa_shape s = shape();
  const size_t need = pbsa_workspace_size(&s, PBSA_OP_PERMUTATION);
  EXPECT_TRUE(need > 0);
  EXPECT_EQ(pbsa_build_segment_permutation(&s, FQ, FQ, FI, nullptr, nullptr, need, nullptr), W);
  EXPECT_EQ(pbsa_build_segment_permutation(&s, FQ, FQ, FI, nullptr, FW, need - 1, nullptr), W);
  EXPECT_EQ(pbsa_build_segment_permutation(&s, FQ, FQ, FI, nullptr, reinterpret_cast<void*>(0x10010), need, nullptr),
            W);  // not 256-byte aligned
  const size_t needa = pbsa_workspace_size(&s, PBSA_OP_ATTENTION);
  EXPECT_TRUE(needa > 0);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, nullptr, 0, nullptr),
            W);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, FW, needa - 1, nullptr),
            W);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, reinterpret_cast<void*>(0x10010), needa, nullptr),
            W);
  const size_t needm = pbsa_workspace_size(&s, PBSA_OP_MASK);
  EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, nullptr, 0.9, 3, FI, FI, nullptr, FW, needm - 8, nullptr), W);
}

void stride_validation() {
  pbsa_shape s = shape();
  s.q_stride_head = 1024 * 128;
  s.q_stride_token = 100;  // token stride < d
  EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr), PBSA_ERR_INVALID_ARG);
  s.q_stride_token = 132;  // not a multiple of 8
  EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr), PBSA_ERR_INVALID_ARG);
  s.q_stride_token = 1LL << 40;  // a stride whose byte extent overflows 32-bit buffer offsets
  EXPECT_TRUE(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr) != PBSA_OK);
}

void empty_sequence_is_a_no_op() {
  pbsa_shape s = shape(0);
  EXPECT_EQ(pbsa_build_segment_permutation(&s, FQ, FQ, FI, nullptr, FW, (size_t)1 << 20, nullptr), PBSA_OK);
  EXPECT_EQ(pbsa_estimate_block_mask(&s, FQ, FQ, nullptr, 0.9, 3, FI, FI, nullptr, FW, (size_t)1 << 20, nullptr),
            PBSA_OK);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                           nullptr, nullptr, 0, nullptr),
            PBSA_OK);
  EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr), PBSA_OK);
  EXPECT_EQ(pbsa_calibrate_thresholds(&s, FF, 4, FF, nullptr), PBSA_OK);
}

void prefix_rank_length_and_workspace() {
  pbsa_shape s;
  s = shape(1024, 4, 2, 128, 128, 512);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), 512);
  s = shape(2000, 4, 2, 128, 128, 512);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), 512 * 4 * 3 / 2);
  s = shape(512, 4, 2, 128, 128, 512);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), 0);
  s = shape(0);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), 0);
  s = shape(1024, 4, 2, 128, 128, 0);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), -1);
  s = shape(64 * 300, 4, 2, 128, 64, 64);
  EXPECT_EQ(pbsa_prefix_rank_length(&s), -1);
  s = shape(1024, 4, 2, 128, 128, 0);
  EXPECT_TRUE(pbsa_workspace_size(&s, PBSA_OP_PREFIX_RANK) == SMAX);
  size_t prev = 0;
  const int ns[] = {512, 1024, 2048, 4096, 8192};
  for (int n : ns) {
    s = shape(n, 4, 2, 128, 128, 512);
    const size_t w = pbsa_workspace_size(&s, PBSA_OP_PREFIX_RANK);
    EXPECT_TRUE(w != SMAX && w >= prev);
    prev = w;
  }
}

void prefix_ranking_and_two_pass_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG, W = PBSA_ERR_WORKSPACE, U = PBSA_ERR_UNSUPPORTED;
  pbsa_shape s = shape(2048, 4, 2, 128, 128, 512);
  pbsa_shape s0 = shape(1024, 4, 2, 128, 128, 0);
  pbsa_shape many = shape(64 * 300, 4, 2, 128, 64, 64);
  pbsa_shape empty = shape(0);
  pbsa_shape one_seg = shape(400, 4, 2, 128, 128, 512);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&s0, FQ, FQ, FI, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&s, nullptr, FQ, FI, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&s, FQ, FQ, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&s, FQ, FQ, FI, nullptr, 0, nullptr), W);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&many, FQ, FQ, FI, FW, BIG, nullptr), U);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&empty, FQ, FQ, nullptr, nullptr, 0, nullptr), PBSA_OK);
  EXPECT_EQ(pbsa_build_prefix_kv_ranking(&one_seg, FQ, FQ, nullptr, nullptr, 0, nullptr), PBSA_OK);
  auto att = [&](const pbsa_shape& sh, const int32_t* kvr, float tau, void* w) {
    return pbsa_s2o_prefix_attn_prefill(&sh, FQ, FQ, FQ, kvr, nullptr, tau, FF, nullptr, nullptr, nullptr, w,
                                        w ? BIG : 0, nullptr);
  };
  EXPECT_EQ(att(s, FI, -1.0f, FW), E);
  EXPECT_EQ(att(s, FI, NAN, FW), E);
  EXPECT_EQ(att(s, FI, INFINITY, FW), E);
  EXPECT_EQ(att(s0, FI, 0.01f, FW), E);
  EXPECT_EQ(att(s, nullptr, 0.01f, FW), E);
  EXPECT_EQ(att(s, FI, 0.01f, nullptr), W);
  EXPECT_EQ(att(many, FI, 0.01f, FW), U);
  EXPECT_EQ(att(empty, nullptr, 0.01f, FW), PBSA_OK);
}

void query_permutation_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG, W = PBSA_ERR_WORKSPACE;
  pbsa_shape s = shape(2048, 4, 2, 128, 128, 512);
  pbsa_shape s0 = shape(1024, 4, 2, 128, 128, 0);
  pbsa_shape empty = shape(0);
  EXPECT_TRUE(pbsa_workspace_size(&s0, PBSA_OP_QUERY_PERM) == SMAX);
  EXPECT_TRUE(pbsa_workspace_size(&empty, PBSA_OP_QUERY_PERM) == 0);
  EXPECT_TRUE(pbsa_workspace_size(&s, PBSA_OP_QUERY_PERM) >= (size_t)8 * 2 * 2048);
  EXPECT_EQ(pbsa_build_query_permutation(&s0, FQ, FQ, FI, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_query_permutation(&s, FQ, FQ, nullptr, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_query_permutation(&s, nullptr, FQ, FI, FW, BIG, nullptr), E);
  EXPECT_EQ(pbsa_build_query_permutation(&s, FQ, FQ, FI, nullptr, 0, nullptr), W);
  EXPECT_EQ(pbsa_build_query_permutation(&empty, FQ, FQ, FI, nullptr, 0, nullptr), PBSA_OK);
}

void sample_attention_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG, W = PBSA_ERR_WORKSPACE;
  pbsa_shape s = shape(1000, 4, 2, 128, 128, 0);
  pbsa_shape empty = shape(0);
  const size_t w = pbsa_sample_mask_workspace_size(&s, 4, 8);
  EXPECT_TRUE(w != 0 && w != SMAX);
  EXPECT_TRUE(pbsa_sample_mask_workspace_size(&s, 0, 8) == SMAX);
  EXPECT_TRUE(pbsa_sample_mask_workspace_size(&s, 4, 0) == SMAX);
  EXPECT_TRUE(pbsa_sample_mask_workspace_size(&s, 3, 334) == SMAX);  // chunks of 334: the last holds 332
  EXPECT_TRUE(pbsa_sample_mask_workspace_size(&s, 3, 332) != SMAX);
  EXPECT_TRUE(pbsa_sample_mask_workspace_size(&empty, 4, 8) == 0);
  auto m = [&](const pbsa_shape& sh, double tau, int nt, int rpt, uint32_t fl, void* ws) {
    return pbsa_sample_attention_mask(&sh, FQ, FQ, tau, nt, rpt, fl, FI, FI, nullptr, nullptr, ws, ws ? BIG : 0,
                                      nullptr);
  };
  EXPECT_EQ(m(s, 0.0, 4, 8, 1, FW), E);
  EXPECT_EQ(m(s, 1.5, 4, 8, 1, FW), E);
  EXPECT_EQ(m(s, NAN, 4, 8, 1, FW), E);
  EXPECT_EQ(m(s, 0.9, 0, 8, 1, FW), E);
  EXPECT_EQ(m(s, 0.9, 3, 334, 1, FW), E);
  EXPECT_EQ(m(s, 0.9, 4, 8, 4, FW), E);  // the ranked flag is not accepted here
  EXPECT_EQ(m(s, 0.9, 4, 8, 1, nullptr), W);
  EXPECT_EQ(m(empty, 0.9, 4, 8, 1, nullptr), PBSA_OK);
  EXPECT_EQ(pbsa_sample_attention_mask(&s, FQ, FQ, 0.9, 4, 8, 1, nullptr, FI, nullptr, nullptr, FW, BIG, nullptr), E);
}

void noalloc_attention() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  pbsa_shape s = shape();
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(nullptr, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF,
                                                   nullptr, nullptr, nullptr, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(&s, FQ, FQ, nullptr, nullptr, nullptr, nullptr, nullptr, FF,
                                                   nullptr, nullptr, nullptr, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(&s, FQ, FQ, FQ, nullptr, FI, nullptr, nullptr, FF, nullptr,
                                                   nullptr, nullptr, nullptr),
            E);
  uint16_t* bad = reinterpret_cast<uint16_t*>(0x10002);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(&s, bad, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                                   nullptr, nullptr, nullptr),
            E);
  pbsa_shape s0 = shape(0);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(&s0, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                                   nullptr, nullptr, nullptr),
            PBSA_OK);
  s.head_dim = 96;
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_noalloc(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                                   nullptr, nullptr, nullptr),
            PBSA_ERR_UNSUPPORTED);
}

void launch_options_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  pbsa_shape s = shape();
  const pbsa_launch_options bad[] = {{-1, 0}, {0, 2}, {4, 0x80000000u}};
  for (const pbsa_launch_options& o : bad)
    EXPECT_EQ(pbsa_block_sparse_attn_prefill_ex(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                                nullptr, nullptr, FW, 256, &o, nullptr),
              E);
  const pbsa_launch_options ok = {16, PBSA_LAUNCH_CLAIM_BACK};
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_ex(&s, FQ, FQ, nullptr, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                              nullptr, nullptr, FW, 256, &ok, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_ex(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                              nullptr, nullptr, FW, 8, &ok, nullptr),
            PBSA_ERR_WORKSPACE);
  pbsa_shape s0 = shape(0);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_ex(&s0, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                              nullptr, nullptr, nullptr, 0, nullptr, nullptr),
            PBSA_OK);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_ex(&s0, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                              nullptr, nullptr, nullptr, 0, &ok, nullptr),
            PBSA_OK);
}

void bf16_output_entry() {
  const pbsa_status E = PBSA_ERR_INVALID_ARG;
  pbsa_shape s = shape();
  uint16_t* FO = reinterpret_cast<uint16_t*>(FF);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(nullptr, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FO,
                                                   nullptr, nullptr, nullptr, FW, 256, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                   nullptr, nullptr, nullptr, FW, 256, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s, FQ, FQ, FQ, nullptr, FI, nullptr, nullptr, FO, nullptr,
                                                   nullptr, nullptr, FW, 256, nullptr),
            E);
  uint16_t* bad = reinterpret_cast<uint16_t*>(0x10002);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, bad, nullptr,
                                                   nullptr, nullptr, FW, 256, nullptr),
            E);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FO, nullptr,
                                                   nullptr, nullptr, FW, 8, nullptr),
            PBSA_ERR_WORKSPACE);
  pbsa_shape s0 = shape(0);
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s0, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FO, nullptr,
                                                   nullptr, nullptr, nullptr, 0, nullptr),
            PBSA_OK);
  s.head_dim = 96;
  EXPECT_EQ(pbsa_block_sparse_attn_prefill_bf16out(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FO, nullptr,
                                                   nullptr, nullptr, FW, 256, nullptr),
            PBSA_ERR_UNSUPPORTED);
}

// Extreme shape fields: validation must reject them without overflowing its own arithmetic (a
// signed overflow here is what UndefinedBehaviorSanitizer reports).
void extreme_shapes() {
  const int32_t vals[] = {INT32_MIN, -129, -1, 0, 1, 63, 64, 65, 127, 128, 129, 4096, 262144, 262145, INT32_MAX};
  for (int32_t N : vals)
    for (int32_t H : {INT32_MIN, -1, 0, 1, 2, 3, 64, 65536, INT32_MAX})
      for (int32_t S : {INT32_MIN, -128, 0, 128, 512, 8192, INT32_MAX}) {
        pbsa_shape s = shape(N, H, H > 1 ? H / 2 : H, 128, 128, S);
        (void)pbsa_workspace_size(&s, PBSA_OP_PERMUTATION);
        (void)pbsa_workspace_size(&s, PBSA_OP_MASK);
        (void)pbsa_workspace_size(&s, PBSA_OP_ATTENTION);
        (void)pbsa_workspace_size(&s, PBSA_OP_PREFIX_RANK);
        (void)pbsa_workspace_size(&s, PBSA_OP_QUERY_PERM);
        (void)pbsa_prefix_rank_length(&s);
        (void)pbsa_sample_mask_workspace_size(&s, 4, 8);
        (void)pbsa_sample_mask_workspace_size(&s, INT32_MAX, INT32_MAX);
        // only shapes that validation rejects, or that are empty, may go on to the entry points
        if (pbsa_workspace_size(&s, PBSA_OP_ATTENTION) == SMAX || N == 0) {
          const int st = pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF,
                                                        nullptr, nullptr, nullptr, nullptr, 0, nullptr);
          if (N != 0) EXPECT_TRUE(st != PBSA_OK);
        }
      }
  // strides whose extents overflow 64-bit arithmetic, or exceed what the kernels address
  const int64_t big8 = INT64_MAX & ~(int64_t)7;
  const int64_t strides[][2] = {{big8, big8}, {big8, 128}, {0x4000000000000000ll, 128}, {1024 * 128, big8},
                                {1024 * 128, (int64_t)1 << 21}, {(int64_t)1 << 47, 128}};
  for (const auto& st : strides) {
    pbsa_shape s = shape();
    s.q_stride_head = st[0];
    s.q_stride_token = st[1];
    EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr), PBSA_ERR_UNSUPPORTED);
    s = shape();
    s.kv_stride_head = st[0];
    s.kv_stride_token = st[1];
    EXPECT_EQ(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr), PBSA_ERR_UNSUPPORTED);
    s = shape();
    s.o_stride_head = st[0];
    s.o_stride_token = st[1];
    if (st[1] < ((int64_t)1 << 21))
      EXPECT_EQ(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr,
                                               nullptr, nullptr, nullptr, 0, nullptr),
                PBSA_ERR_UNSUPPORTED);
  }
  pbsa_shape s = shape();
  s.q_stride_head = INT64_MAX;  // not a multiple of 8
  s.q_stride_token = INT64_MAX;
  EXPECT_TRUE(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr) != PBSA_OK);
  s = shape();
  s.kv_stride_head = -128;
  EXPECT_TRUE(pbsa_tile_max(&s, FQ, FQ, nullptr, FF, nullptr) != PBSA_OK);
  s = shape();
  s.o_stride_token = INT64_MIN;
  EXPECT_TRUE(pbsa_block_sparse_attn_prefill(&s, FQ, FQ, FQ, nullptr, nullptr, nullptr, nullptr, FF, nullptr, nullptr,
                                             nullptr, FW, 256, nullptr) != PBSA_OK);
}

}  // namespace

int main() {
  status_strings();
  workspace_sizes_monotone_in_n();
  shape_validation();
  null_shape_and_pointers();
  permutation_and_mask_arguments();
  marginal_gain_entry();
  workspace_checks();
  stride_validation();
  empty_sequence_is_a_no_op();
  prefix_rank_length_and_workspace();
  prefix_ranking_and_two_pass_entry();
  query_permutation_entry();
  sample_attention_entry();
  noalloc_attention();
  launch_options_entry();
  bf16_output_entry();
  extreme_shapes();
  printf("abi_cases: %d checks, %d failures\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
