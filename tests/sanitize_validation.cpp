// Host-side driver for the library's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py builds and runs it; no GPU involved).
//
// Every call below either returns from validation with an error before anything is enqueued, or is
// a pure size query; none reaches a launch (the driver runs without a GPU, and a call that got past
// validation would return a HIP error, which this driver counts as a failure).
// Inputs go to the edges of what the validation guards: group counts, negative and huge split
// sizes, 32-bit extents, widths, NULL pointers, enum values, short workspaces, device-resident split
// sizes, and the allocation-free backward's scratch limit.

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mgs.h"

namespace {

int g_checks = 0, g_fail = 0;

void expect(long long got, long long want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL line %d: %s returned %lld, expected %lld (%s)\n", line, what, got, want, mgs_last_error());
  }
  // the message must be a terminated string within the library's buffer
  const char* msg = mgs_last_error();
  if (std::strlen(msg) > 4096) {
    ++g_fail;
    std::printf("FAIL line %d: error message of %zu bytes\n", line, std::strlen(msg));
  }
}

#define EXPECT(expr, want) expect((long long)(expr), (long long)(want), #expr, __LINE__)

void* const FAKE = reinterpret_cast<void*>(0x1000);  // never dereferenced: validation fails first

mgs_groups host_groups(const std::vector<int64_t>& s) {
  mgs_groups g;
  g.num_groups = (int32_t)s.size();
  g.split_sizes = s.data();
  g.max_rows = 0;
  g.dev_table = nullptr;
  return g;
}

mgs_groups dev_groups(int e, int64_t cap) {
  mgs_groups g;
  g.num_groups = e;
  g.split_sizes = nullptr;
  g.max_rows = cap;
  g.dev_table = FAKE;
  return g;
}

}  // namespace

// Planted faults that show the instrumentation is live: "oob" reads past a heap array (ASan must
// report it), "overflow" overflows a signed int (UBSan must report it).
int planted(const char* which) {
  volatile int n = 4;
  if (std::strcmp(which, "oob") == 0) {
    int* a = new int[n];
    const int v = a[n];  // one past the end
    delete[] a;
    return v;
  }
  volatile int big = INT32_MAX;
  return big + n;  // signed overflow
}

int main(int argc, char** argv) {
  if (argc > 1) return planted(argv[1]);
  const mgs_act_params srelu{MGS_ACT_SRELU, 2.0f, 7.0f, 1.0f, 0.0f};
  const mgs_act_params swiglu{MGS_ACT_SWIGLU, 2.0f, 7.0f, 1.0f, 0.0f};
  mgs_qbuf q{FAKE, FAKE, static_cast<float*>(FAKE), 0u};
  mgs_qbuf q_nogs{FAKE, FAKE, nullptr, 0u};
  float* const F = static_cast<float*>(FAKE);

  EXPECT(mgs_abi_version(), MGS_ABI_VERSION);
  EXPECT(mgs_groups_table_bytes() > 0, 1);

  // ---- group tables
  std::vector<int64_t> ok4{64, 0, 96, 37};
  mgs_groups g4 = host_groups(ok4);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, nullptr, 64, MGS_NBYTES_DATA), MGS_ERR_INVALID_ARG);
  std::vector<int64_t> none;
  mgs_groups g0 = host_groups(none);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g0, 64, MGS_NBYTES_DATA), MGS_ERR_INVALID_ARG);
  std::vector<int64_t> too_many(MGS_MAX_GROUPS + 1, 1);
  mgs_groups g257 = host_groups(too_many);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g257, 64, MGS_NBYTES_DATA), MGS_ERR_INVALID_ARG);
  std::vector<int64_t> max_groups(MGS_MAX_GROUPS, 129);
  mgs_groups g256 = host_groups(max_groups);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 1, &g256, 64, MGS_NBYTES_DATA), (int64_t)256 * 256 * 64);
  std::vector<int64_t> neg{32, -1};
  mgs_groups gneg = host_groups(neg);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gneg, 64, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  std::vector<int64_t> huge{INT64_MAX / 2, INT64_MAX / 2};
  mgs_groups ghuge = host_groups(huge);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &ghuge, 64, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  std::vector<int64_t> over31{(int64_t)1 << 30, (int64_t)1 << 30};
  mgs_groups gover = host_groups(over31);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gover, 64, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  EXPECT(mgs_qtensor_nbytes(7, 0, &g4, 64, MGS_NBYTES_DATA), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, 48, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, 0, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, ((int64_t)1 << 24) + 32, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, 64, 9), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, 64, MGS_NBYTES_DATA), 197 * 64);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_NVFP4, 1, &g4, 64, MGS_NBYTES_DATA), 3 * 128 * 32);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_NVFP4, 0, &g4, 64, MGS_NBYTES_GROUP_SCALE), 16);

  // device-resident split sizes
  mgs_groups gd = dev_groups(4, 300);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gd, 96, MGS_NBYTES_DATA), 300 * 96);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 1, &gd, 96, MGS_NBYTES_DATA), 128 * (3 + 4) * 96);
  mgs_groups gd0 = dev_groups(4, 0);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gd0, 96, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  mgs_groups gdbig = dev_groups(4, INT64_MAX);
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gdbig, 96, MGS_NBYTES_DATA), MGS_ERR_SHAPE);
  mgs_groups gdnull = dev_groups(4, 300);
  gdnull.dev_table = nullptr;
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &gdnull, 96, MGS_NBYTES_DATA), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_groups_update(&g4, static_cast<int64_t*>(FAKE), nullptr, nullptr), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_groups_update(&gd, nullptr, nullptr, nullptr), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_groups_update(nullptr, static_cast<int64_t*>(FAKE), nullptr, nullptr), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_groups_update(&gd0, static_cast<int64_t*>(FAKE), nullptr, nullptr), MGS_ERR_SHAPE);

  // ---- forward
  EXPECT(mgs_grouped_scaled_act_fwd(nullptr, MGS_FMT_MXFP8, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  const mgs_act_params bad_kind{42, 1, 1, 1, 0};
  EXPECT(mgs_grouped_scaled_act_fwd(&bad_kind, MGS_FMT_MXFP8, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  const mgs_act_params bad_kind_neg{-1, 1, 1, 1, 0};
  EXPECT(mgs_grouped_scaled_act_fwd(&bad_kind_neg, MGS_FMT_MXFP8, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  const mgs_act_params tanh_bad{MGS_ACT_TANH_SRELU, 0.0f, 7, 1, 0};
  EXPECT(mgs_grouped_scaled_act_fwd(&tanh_bad, MGS_FMT_MXFP8, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  const mgs_act_params clamp_bad{MGS_ACT_CLAMPED_SWIGLU, 1, -1.0f, 1, 0};
  EXPECT(mgs_grouped_scaled_act_fwd(&clamp_bad, MGS_FMT_MXFP8, &g4, 128, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, 5, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_MXFP8, &g4, 64, nullptr, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_MXFP8, &g4, 64, FAKE, F, nullptr, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd(&swiglu, MGS_FMT_MXFP8, &g4, 96, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, F, &q_nogs, nullptr, F, nullptr),
         MGS_ERR_INVALID_ARG);
  std::vector<int64_t> big1{65536};
  mgs_groups gbig = host_groups(big1);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_MXFP8, &gbig, 32768, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_NVFP4, &gd, 96, FAKE, F, &q, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  mgs_qbuf rht_row{FAKE, FAKE, F, (1u << 16) | 0x1234u};
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, F, &rht_row, nullptr, F, nullptr),
         MGS_ERR_UNSUPPORTED);
  mgs_qbuf rht_bad{FAKE, FAKE, F, 0x1234u};
  EXPECT(mgs_grouped_scaled_act_fwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, F, nullptr, &rht_bad, F, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd_f32(&srelu, MGS_FMT_MXFP8, &g4, 64, F, F, nullptr, nullptr, nullptr, nullptr,
                                        nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_fwd_f32(&srelu, MGS_FMT_MXFP8, &gd, 48, F, F, &q, nullptr, nullptr, nullptr,
                                        nullptr),
         MGS_ERR_SHAPE);

  // ---- backward
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_MXFP8, &g4, 64, FAKE, nullptr, F, FAKE, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_MXFP8, &g4, 64, FAKE, FAKE, F, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, FAKE, F, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, &q, nullptr, nullptr, 0, nullptr),
         MGS_ERR_UNSUPPORTED);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_NVFP4, &g4, 64, FAKE, FAKE, F, nullptr, &q, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  const int64_t need = mgs_act_bwd_workspace_bytes(&srelu, &g4, 256);
  EXPECT(need > 0, 1);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_MXFP8, &g4, 256, FAKE, FAKE, F, nullptr, nullptr, nullptr,
                                    nullptr, F, nullptr, nullptr, nullptr, FAKE, need - 1, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_MXFP8, &g4, 256, FAKE, FAKE, F, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, F, nullptr, nullptr, nullptr, need, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_act_bwd_workspace_bytes(&swiglu, &g4, 96), MGS_ERR_SHAPE);
  EXPECT(mgs_act_bwd_workspace_bytes(nullptr, &g4, 64), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_act_bwd_workspace_bytes(&srelu, &gneg, 64), MGS_ERR_SHAPE);
  std::vector<int64_t> big16(16, 4096);
  mgs_groups gbig16 = host_groups(big16);
  EXPECT(mgs_grouped_scaled_act_bwd_noalloc(&srelu, MGS_FMT_MXFP8, &gbig16, 4096, FAKE, FAKE, F, nullptr, nullptr,
                                            nullptr, nullptr, F, nullptr, nullptr, nullptr, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_scaled_act_bwd_noalloc(&srelu, MGS_FMT_MXFP8, &g4, 64, FAKE, nullptr, F, FAKE, nullptr,
                                            nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_scaled_act_bwd(&srelu, MGS_FMT_NVFP4, &gd, 96, FAKE, FAKE, F, nullptr, &q, nullptr,
                                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);

  // ---- quantize and column sums
  EXPECT(mgs_grouped_mx_quantize(MGS_FMT_MXFP8, &g4, 64, FAKE, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                 nullptr),
         MGS_ERR_INVALID_ARG);
  const int64_t qneed = mgs_grouped_mx_quantize_workspace_bytes(&g4, 64);
  EXPECT(qneed, 4 * 3 * 64);
  EXPECT(mgs_grouped_mx_quantize(MGS_FMT_MXFP8, &g4, 64, FAKE, &q, nullptr, nullptr, F, FAKE, qneed - 1,
                                 nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_mx_quantize(MGS_FMT_NVFP4, &g4, 64, FAKE, &q, nullptr, nullptr, nullptr, nullptr, 0,
                                 nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_mx_quantize_workspace_bytes(&g4, 40), MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_col_sum(&g4, 12, FAKE, F, nullptr), MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_col_sum(&g4, 64, FAKE, nullptr, nullptr), MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_col_sum(&gd, 64, FAKE, nullptr, nullptr), MGS_ERR_INVALID_ARG);

  // ---- GEMMs
  float cbuf[1];
  EXPECT(mgs_grouped_gemm_mx(9, MGS_FMT_MXFP8, &g4, 197, 64, 64, &q, &q, cbuf, MGS_DTYPE_F32, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 196, 64, 64, &q, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 197, 64, 48, &q, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_WGRAD, MGS_FMT_MXFP8, &g4, 64, 64, 198, &q, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_WGRAD, MGS_FMT_MXFP8, &g4, 64, 64, 197, &q, &q, cbuf, MGS_DTYPE_F32, FAKE,
                             0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 197, 64, 64, &q, &q, cbuf, MGS_DTYPE_BF16,
                             nullptr, 1, nullptr),
         MGS_ERR_UNSUPPORTED);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 197, 64, 64, &q, &q, cbuf, 3, nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_NVFP4, &g4, 197, 64, 64, &q_nogs, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 197, 64, 64, nullptr, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &g4, 197, 64, 64, &q, &q, nullptr, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_MXFP8, &gd, 299, 64, 64, &q, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_SHAPE);
  EXPECT(mgs_grouped_gemm_mx(MGS_GEMM_FPROP, MGS_FMT_NVFP4, &gd, 300, 64, 64, &q_nogs, &q, cbuf, MGS_DTYPE_F32,
                             nullptr, 0, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx_fprop_act(&g4, 197, 64, 64, &q, &q, cbuf, nullptr, &swiglu, F, MGS_DTYPE_BF16, &q,
                                       nullptr),
         MGS_ERR_UNSUPPORTED);
  EXPECT(mgs_grouped_gemm_mx_fprop_act(&g4, 197, 64, 64, &q, &q, nullptr, nullptr, &srelu, F, MGS_DTYPE_BF16, &q,
                                       nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx_fprop_act(&g4, 197, 64, 64, &q, &q, cbuf, nullptr, &srelu, F, 5, &q, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx_fprop_act(&g4, 197, 64, 64, &q, &q, cbuf, nullptr, &srelu, F, MGS_DTYPE_BF16,
                                       nullptr, nullptr),
         MGS_ERR_INVALID_ARG);
  EXPECT(mgs_grouped_gemm_mx_fprop_act(&g4, 196, 64, 64, &q, &q, cbuf, nullptr, &srelu, F, MGS_DTYPE_BF16, &q,
                                       nullptr),
         MGS_ERR_SHAPE);

  // a successful query clears the message
  EXPECT(mgs_qtensor_nbytes(MGS_FMT_MXFP8, 0, &g4, 32, MGS_NBYTES_DATA), 197 * 32);
  EXPECT(std::strlen(mgs_last_error()), 0);

  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
