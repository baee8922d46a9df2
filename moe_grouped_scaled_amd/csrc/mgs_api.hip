// C-ABI entry points: argument validation, group bookkeeping and kernel dispatch.
//
// Group bookkeeping (page "Activation + GroupedLinear Fusion for MOE", sequence diagram: the fused
// ops receive split_sizes and derive each group's rows from it): row offsets, padded columnwise
// token offsets and the per-launch tile lists are computed here on the host and passed to the
// kernels by value, so no device memory is allocated and nothing is synchronized.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "mgs_internal.h"

// Scratch of the allocation-free backward (mgs_grouped_scaled_act_bwd_noalloc): the dprobs and
// bias-gradient partial sums and the group maxima of a transformed recompute.  Every device the
// library runs on holds its own copy until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in for the symbol): scratch_address() looks up each
// device's copy once and every later use goes through that pointer.
static __device__ __align__(256) uint8_t scratch[MGS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MGS_OK;
}

bool valid_fmt(int32_t fmt) { return fmt == MGS_FMT_MXFP8 || fmt == MGS_FMT_NVFP4; }

bool is_gated(int kind) { return kind == MGS_ACT_SWIGLU || kind == MGS_ACT_CLAMPED_SWIGLU || kind == MGS_ACT_GLU; }

// Byte offset of the GEMM tile table after the group table in a device table.
constexpr int64_t kDevGemmTableOffset = (sizeof(mgs::GroupTable) + 255) / 256 * 256;

// Validates the groups and fills the panel table.  Returns MGS_OK or an error code.  Device-resident
// split sizes: the table describes the layout for the row capacity (total_rows = max_rows, num_panels
// = the padded-panel bound) and points to the device table holding the actual offsets.
int build_groups(const mgs_groups* groups, mgs::GroupTable* gt, int64_t* total_rows) {
  if (!groups) return fail(MGS_ERR_INVALID_ARG, "groups is NULL");
  if (groups->num_groups < 1 || groups->num_groups > MGS_MAX_GROUPS)
    return fail(MGS_ERR_INVALID_ARG, "num_groups %d outside [1, %d]", groups->num_groups, MGS_MAX_GROUPS);
  std::memset(gt, 0, sizeof *gt);
  gt->num_groups = groups->num_groups;
  if (!groups->split_sizes) {
    if (!groups->dev_table)
      return fail(MGS_ERR_INVALID_ARG, "split_sizes is NULL and no dev_table for device-resident split sizes");
    const int64_t cap = groups->max_rows;
    if (cap <= 0 || cap > INT32_MAX - 64 - (int64_t)mgs::COL_ALIGN * (groups->num_groups + 1))
      return fail(MGS_ERR_SHAPE, "max_rows = %lld outside [1, 2^31 - 64 - 128 (E + 1)]", (long long)cap);
    gt->total_rows = (int32_t)cap;
    gt->num_panels = (int32_t)(((cap + mgs::COL_ALIGN - 1) / mgs::COL_ALIGN + groups->num_groups) *
                               (mgs::COL_ALIGN / mgs::PANEL_ROWS));
    gt->dev = static_cast<const mgs::GroupTable*>(groups->dev_table);
    *total_rows = cap;
    return MGS_OK;
  }
  int64_t rows = 0, panels = 0;
  for (int g = 0; g < groups->num_groups; ++g) {
    const int64_t m = groups->split_sizes[g];
    if (m < 0) return fail(MGS_ERR_SHAPE, "split_sizes[%d] = %lld is negative", g, (long long)m);
    gt->row_off[g] = (int32_t)rows;
    gt->panel_off[g] = (int32_t)panels;
    rows += m;
    panels += (m + mgs::COL_ALIGN - 1) / mgs::COL_ALIGN * (mgs::COL_ALIGN / mgs::PANEL_ROWS);
    if (rows > INT32_MAX - 64) return fail(MGS_ERR_SHAPE, "total rows exceed 2^31 - 64");
  }
  gt->row_off[groups->num_groups] = (int32_t)rows;
  gt->panel_off[groups->num_groups] = (int32_t)panels;
  gt->num_panels = (int32_t)panels;
  gt->total_rows = (int32_t)rows;
  *total_rows = rows;
  return MGS_OK;
}

int check_width(int64_t w, const char* what) {
  if (w <= 0 || w % 32 != 0)
    return fail(MGS_ERR_SHAPE, "%s = %lld must be a positive multiple of 32", what, (long long)w);
  if (w > (int64_t)1 << 24) return fail(MGS_ERR_SHAPE, "%s = %lld is too large", what, (long long)w);
  return MGS_OK;
}

// The quantizing kernels address each output through 32-bit offsets below 2^31 bytes: one group's
// columnwise matrix (padded rows x width codes) and the whole rowwise MXFP8 scale array must fit.
int check_extent(const mgs::GroupTable& gt, int64_t width, const char* what) {
  const int64_t lim = (int64_t)1 << 31;
  if (gt.dev && (int64_t)mgs::PANEL_ROWS * gt.num_panels * width >= lim)
    return fail(MGS_ERR_SHAPE, "max_rows x %s too large: one group's padded columnwise matrix could reach 2^31 "
                "elements", what);
  for (int g = 0; g < gt.num_groups; ++g) {
    const int64_t padded = (int64_t)mgs::PANEL_ROWS * (gt.panel_off[g + 1] - gt.panel_off[g]);
    if (padded * width >= lim)
      return fail(MGS_ERR_SHAPE, "group %d: %lld padded rows x %s %lld reach 2^31 elements", g,
                  (long long)padded, what, (long long)width);
  }
  if (4 * (int64_t)gt.total_rows * ((width + 127) / 128) >= lim)
    return fail(MGS_ERR_SHAPE, "rows x %s too large: the rowwise scale array reaches 2 GiB", what);
  return MGS_OK;
}

bool qbuf_requested(const mgs_qbuf* q) { return q && q->data; }

int check_qbuf(const mgs_qbuf* q, int32_t fmt, const char* what, bool colwise) {
  if (!qbuf_requested(q)) return MGS_OK;
  if (!q->scales) return fail(MGS_ERR_INVALID_ARG, "%s.scales is NULL", what);
  if (fmt == MGS_FMT_NVFP4 && !q->group_scale)
    return fail(MGS_ERR_INVALID_ARG, "%s.group_scale is NULL (required for NVFP4)", what);
  if (q->rht) {
    if (!colwise || fmt != MGS_FMT_NVFP4)
      return fail(MGS_ERR_UNSUPPORTED, "%s.rht: the Hadamard transform applies to NVFP4 columnwise copies only", what);
    if ((q->rht >> 16) != 1u)
      return fail(MGS_ERR_INVALID_ARG, "%s.rht = 0x%x: bit 16 enables the transform, bits 0..15 are the signs",
                  what, q->rht);
  }
  return MGS_OK;
}

uint32_t qbuf_rht(const mgs_qbuf* q) { return qbuf_requested(q) ? q->rht : 0u; }

int check_act(const mgs_act_params* act, mgs::ActHost* out) {
  if (!act) return fail(MGS_ERR_INVALID_ARG, "act is NULL");
  if (act->kind < MGS_ACT_IDENTITY || act->kind > MGS_ACT_GLU)
    return fail(MGS_ERR_INVALID_ARG, "unknown activation kind %d", act->kind);
  if (act->kind == MGS_ACT_TANH_SRELU && !(act->s > 0.0f && std::isfinite(act->s)))
    return fail(MGS_ERR_INVALID_ARG, "TANH_SRELU needs a finite s > 0 (got %g)", (double)act->s);
  if (act->kind == MGS_ACT_CLAMPED_SWIGLU &&
      !(act->limit > 0.0f && std::isfinite(act->limit) && std::isfinite(act->alpha) && std::isfinite(act->beta)))
    return fail(MGS_ERR_INVALID_ARG, "CLAMPED_SWIGLU needs a finite limit > 0 and finite alpha, beta");
  out->kind = act->kind;
  out->s = act->s;
  out->inv_s = act->kind == MGS_ACT_TANH_SRELU ? 1.0f / act->s : 1.0f;
  out->limit = act->limit;
  out->alpha = act->alpha;
  out->beta = act->beta;
  return MGS_OK;
}

mgs::QOut make_qout(const mgs_qbuf* row, const mgs_qbuf* col, int64_t width) {
  mgs::QOut q{};
  if (qbuf_requested(row)) {
    q.row_data = static_cast<uint8_t*>(row->data);
    q.row_scales = static_cast<uint8_t*>(row->scales);
    q.row_gscale = row->group_scale;
  }
  if (qbuf_requested(col)) {
    q.col_data = static_cast<uint8_t*>(col->data);
    q.col_scales = static_cast<uint8_t*>(col->scales);
    q.col_gscale = col->group_scale;
    q.col_rht = col->rht;
  }
  q.width = width;
  return q;
}

bool device_splits(const mgs::GroupTable& gt) { return gt.dev != nullptr; }

mgs::GemmTable* dev_gemm_table(const mgs_groups* groups) {
  return groups->split_sizes ? nullptr
                             : reinterpret_cast<mgs::GemmTable*>(static_cast<uint8_t*>(groups->dev_table) +
                                                                 kDevGemmTableOffset);
}


int hip_status(hipError_t e) {
  if (e != hipSuccess) return fail(MGS_ERR_HIP, "HIP launch error: %s", hipGetErrorString(e));
  return ok();
}

// Device address of `scratch` on the current device, taken with that device current on the first
// call that needs it and kept per device (each device's copy has its own address).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];

int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MGS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MGS_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch covers", dev,
                kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MGS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MGS_OK;
}

// The backward's validation and launch, shared by the entry point with a caller workspace and the
// allocation-free one (whose workspace is the static scratch).
int act_bwd_impl(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups, int64_t width_in,
                 const void* x_bf16, const void* dy_bf16, const float* probs, void* dx_bf16,
                 const mgs_qbuf* dx_row, const mgs_qbuf* dx_col, float* dx_group_amax, float* dprobs,
                 float* dx_col_sum, const mgs_qbuf* act_col, const float* saved_group_amax,
                 void* workspace, int64_t workspace_bytes, bool static_scratch, void* stream) {
  mgs::ActHost ah;
  int rc = check_act(act, &ah);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  mgs::GroupTable gt;
  int64_t rows = 0;
  if ((rc = build_groups(groups, &gt, &rows))) return rc;
  if (is_gated(ah.kind) && width_in % 2 != 0) return fail(MGS_ERR_SHAPE, "gated width_in must be even");
  const int64_t wa = is_gated(ah.kind) ? width_in / 2 : width_in;
  if ((rc = check_width(wa, is_gated(ah.kind) ? "width_in / 2" : "width_in"))) return rc;
  if ((rc = check_extent(gt, width_in, "width_in"))) return rc;
  if (!x_bf16 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "x_bf16 is NULL");
  if (!dy_bf16 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "dy_bf16 is NULL");
  const bool want_dxq = qbuf_requested(dx_row) || qbuf_requested(dx_col);
  if (!dx_bf16 && !want_dxq && !dprobs && !dx_col_sum && !qbuf_requested(act_col))
    return fail(MGS_ERR_INVALID_ARG, "no output requested");
  if ((rc = check_qbuf(dx_row, fmt, "dx_row", false))) return rc;
  if ((rc = check_qbuf(dx_col, fmt, "dx_col", true))) return rc;
  if ((rc = check_qbuf(act_col, fmt, "act_col", true))) return rc;
  if (fmt == MGS_FMT_NVFP4 && want_dxq && !dx_group_amax)
    return fail(MGS_ERR_INVALID_ARG, "dx_group_amax is required to quantize dx to NVFP4");
  const bool act_rht = qbuf_rht(act_col) != 0;
  if (fmt == MGS_FMT_NVFP4 && qbuf_requested(act_col) && !act_rht && !saved_group_amax)
    return fail(MGS_ERR_UNSUPPORTED,
                "NVFP4 recompute (act_col) needs saved_group_amax, the group amax of the forward");
  if (dprobs || dx_col_sum || act_rht) {
    const int64_t need = mgs::act_bwd_workspace_bytes(gt, wa, width_in);
    if (static_scratch) {
      if (need > MGS_NOALLOC_SCRATCH_BYTES)
        return fail(MGS_ERR_SHAPE,
                    "%s needs %lld bytes of scratch, more than the %lld bytes of the allocation-free "
                    "entry point's static scratch (use mgs_grouped_scaled_act_bwd with a workspace)",
                    dprobs ? "dprobs" : dx_col_sum ? "dx_col_sum" : "a transformed act_col", (long long)need,
                    (long long)MGS_NOALLOC_SCRATCH_BYTES);
      if ((rc = scratch_address(&workspace))) return rc;
      workspace_bytes = MGS_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(MGS_ERR_INVALID_ARG, "%s needs a workspace of %lld bytes (got %lld%s)",
                  dprobs ? "dprobs" : dx_col_sum ? "dx_col_sum" : "a transformed act_col", (long long)need,
                  (long long)workspace_bytes, workspace ? "" : ", NULL");
  }
  mgs::QOut dxq = make_qout(dx_row, dx_col, width_in);
  mgs::QOut aq = make_qout(nullptr, act_col, wa);
  aq.amax = saved_group_amax;
  return hip_status(mgs::launch_act_bwd(ah, fmt, gt, width_in, static_cast<const uint16_t*>(x_bf16),
                                        static_cast<const uint16_t*>(dy_bf16), probs,
                                        static_cast<uint16_t*>(dx_bf16), dxq, dx_group_amax, dprobs,
                                        dx_col_sum, workspace, aq, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int mgs_abi_version(void) { return MGS_ABI_VERSION; }

int64_t mgs_groups_table_bytes(void) { return kDevGemmTableOffset + (int64_t)sizeof(mgs::GemmTable); }

int mgs_groups_update(const mgs_groups* groups, const int64_t* split_sizes_dev, int32_t* status_dev,
                      void* stream) {
  if (!groups) return fail(MGS_ERR_INVALID_ARG, "groups is NULL");
  if (groups->split_sizes) return fail(MGS_ERR_INVALID_ARG, "groups has host split sizes (split_sizes must be NULL)");
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if (!split_sizes_dev) return fail(MGS_ERR_INVALID_ARG, "split_sizes_dev is NULL");
  return hip_status(mgs::launch_groups_update(groups->num_groups, split_sizes_dev, groups->max_rows,
                                              static_cast<mgs::GroupTable*>(groups->dev_table), status_dev,
                                              static_cast<hipStream_t>(stream)));
}

const char* mgs_last_error(void) { return g_err; }

int64_t mgs_qtensor_nbytes(int32_t fmt, int32_t colwise, const mgs_groups* groups, int64_t width,
                           int32_t which) {
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if ((rc = check_width(width, "width"))) return rc;
  const int64_t r = colwise ? (int64_t)mgs::PANEL_ROWS * gt.num_panels : rows;
  switch (which) {
    case MGS_NBYTES_DATA: ok(); return fmt == MGS_FMT_MXFP8 ? r * width : r * width / 2;
    case MGS_NBYTES_SCALES:
      ok();
      if (fmt == MGS_FMT_NVFP4) return r * width / 16;
      // MXFP8 scales are grouped per 128-wide K step: 4 bytes per row and step
      return colwise ? r * width / 32 : 4 * r * ((width + 127) / 128);
    case MGS_NBYTES_GROUP_SCALE: ok(); return fmt == MGS_FMT_MXFP8 ? 0 : 4 * (int64_t)gt.num_groups;
    default: return fail(MGS_ERR_INVALID_ARG, "unknown buffer selector %d", which);
  }
}

int mgs_grouped_scaled_act_fwd(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                               int64_t width_in, const void* x_bf16, const float* probs,
                               const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                               void* stream) {
  mgs::ActHost ah;
  int rc = check_act(act, &ah);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  mgs::GroupTable gt;
  int64_t rows = 0;
  if ((rc = build_groups(groups, &gt, &rows))) return rc;
  if (is_gated(ah.kind) && width_in % 2 != 0) return fail(MGS_ERR_SHAPE, "gated width_in must be even");
  const int64_t wa = is_gated(ah.kind) ? width_in / 2 : width_in;
  if ((rc = check_width(wa, is_gated(ah.kind) ? "width_in / 2" : "width_in"))) return rc;
  if ((rc = check_extent(gt, wa, "width"))) return rc;
  if (!x_bf16 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "x_bf16 is NULL");
  if (!qbuf_requested(out_row) && !qbuf_requested(out_col))
    return fail(MGS_ERR_INVALID_ARG, "no output requested (out_row and out_col are both empty)");
  if ((rc = check_qbuf(out_row, fmt, "out_row", false))) return rc;
  if ((rc = check_qbuf(out_col, fmt, "out_col", true))) return rc;
  if (fmt == MGS_FMT_NVFP4 && !group_amax)
    return fail(MGS_ERR_INVALID_ARG, "group_amax is required for NVFP4 (per-group amax pass)");
  const mgs::QOut q = make_qout(out_row, out_col, wa);
  return hip_status(mgs::launch_act_fwd(ah, fmt, gt, width_in, x_bf16, false, probs, q, group_amax,
                                        nullptr, nullptr, nullptr, static_cast<hipStream_t>(stream)));
}

int mgs_grouped_scaled_act_fwd_f32(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                                   int64_t width_in, const float* x_f32, const float* probs,
                                   const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                                   void* x_bf16_out, void* stream) {
  mgs::ActHost ah;
  int rc = check_act(act, &ah);
  if (rc) return rc;
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  mgs::GroupTable gt;
  int64_t rows = 0;
  if ((rc = build_groups(groups, &gt, &rows))) return rc;
  if (is_gated(ah.kind) && width_in % 2 != 0) return fail(MGS_ERR_SHAPE, "gated width_in must be even");
  const int64_t wa = is_gated(ah.kind) ? width_in / 2 : width_in;
  if ((rc = check_width(wa, is_gated(ah.kind) ? "width_in / 2" : "width_in"))) return rc;
  if ((rc = check_extent(gt, wa, "width"))) return rc;
  if ((int64_t)mgs::PANEL_ROWS * width_in * 4 >= ((int64_t)1 << 31))
    return fail(MGS_ERR_SHAPE, "width_in %lld too large for the FP32 input", (long long)width_in);
  if (!x_f32 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "x_f32 is NULL");
  if (!qbuf_requested(out_row) && !qbuf_requested(out_col) && !x_bf16_out)
    return fail(MGS_ERR_INVALID_ARG, "no output requested (out_row, out_col and x_bf16_out are all empty)");
  if ((rc = check_qbuf(out_row, fmt, "out_row", false))) return rc;
  if ((rc = check_qbuf(out_col, fmt, "out_col", true))) return rc;
  const bool quant = qbuf_requested(out_row) || qbuf_requested(out_col);
  if (fmt == MGS_FMT_NVFP4 && quant && !group_amax)
    return fail(MGS_ERR_INVALID_ARG, "group_amax is required for NVFP4 (per-group amax pass)");
  const mgs::QOut q = make_qout(out_row, out_col, wa);
  return hip_status(mgs::launch_act_fwd(ah, fmt, gt, width_in, x_f32, true, probs, q, group_amax,
                                        nullptr, nullptr, static_cast<uint16_t*>(x_bf16_out),
                                        static_cast<hipStream_t>(stream)));
}

int mgs_grouped_scaled_act_bwd(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                               int64_t width_in, const void* x_bf16, const void* dy_bf16,
                               const float* probs, void* dx_bf16, const mgs_qbuf* dx_row,
                               const mgs_qbuf* dx_col, float* dx_group_amax, float* dprobs,
                               float* dx_col_sum, const mgs_qbuf* act_col,
                               const float* saved_group_amax, void* workspace,
                               int64_t workspace_bytes, void* stream) {
  return act_bwd_impl(act, fmt, groups, width_in, x_bf16, dy_bf16, probs, dx_bf16, dx_row, dx_col,
                      dx_group_amax, dprobs, dx_col_sum, act_col, saved_group_amax, workspace,
                      workspace_bytes, false, stream);
}

int mgs_grouped_scaled_act_bwd_noalloc(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                                       int64_t width_in, const void* x_bf16, const void* dy_bf16,
                                       const float* probs, void* dx_bf16, const mgs_qbuf* dx_row,
                                       const mgs_qbuf* dx_col, float* dx_group_amax, float* dprobs,
                                       float* dx_col_sum, const mgs_qbuf* act_col,
                                       const float* saved_group_amax, void* stream) {
  return act_bwd_impl(act, fmt, groups, width_in, x_bf16, dy_bf16, probs, dx_bf16, dx_row, dx_col,
                      dx_group_amax, dprobs, dx_col_sum, act_col, saved_group_amax, nullptr, 0, true,
                      stream);
}

int64_t mgs_act_bwd_workspace_bytes(const mgs_act_params* act, const mgs_groups* groups,
                                    int64_t width_in) {
  mgs::ActHost ah;
  int rc = check_act(act, &ah);
  if (rc) return rc;
  mgs::GroupTable gt;
  int64_t rows = 0;
  if ((rc = build_groups(groups, &gt, &rows))) return rc;
  if (is_gated(ah.kind) && width_in % 2 != 0) return fail(MGS_ERR_SHAPE, "gated width_in must be even");
  const int64_t wa = is_gated(ah.kind) ? width_in / 2 : width_in;
  if ((rc = check_width(wa, is_gated(ah.kind) ? "width_in / 2" : "width_in"))) return rc;
  ok();
  return mgs::act_bwd_workspace_bytes(gt, wa, width_in);
}

int mgs_grouped_mx_quantize(int32_t fmt, const mgs_groups* groups, int64_t width, const void* x_bf16,
                            const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                            float* col_sum, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if ((rc = check_width(width, "width"))) return rc;
  if ((rc = check_extent(gt, width, "width"))) return rc;
  if (!x_bf16 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "x_bf16 is NULL");
  if (!qbuf_requested(out_row) && !qbuf_requested(out_col) && !col_sum)
    return fail(MGS_ERR_INVALID_ARG, "no output requested (out_row, out_col and col_sum are all empty)");
  if ((rc = check_qbuf(out_row, fmt, "out_row", false))) return rc;
  if ((rc = check_qbuf(out_col, fmt, "out_col", true))) return rc;
  const bool quant = qbuf_requested(out_row) || qbuf_requested(out_col);
  if (fmt == MGS_FMT_NVFP4 && quant && !group_amax)
    return fail(MGS_ERR_INVALID_ARG, "group_amax is required for NVFP4 (per-group amax pass)");
  if (col_sum) {
    const int64_t need = mgs::col_sum_part_bytes(gt, width);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(MGS_ERR_INVALID_ARG, "col_sum needs a workspace of %lld bytes (got %lld%s)", (long long)need,
                  (long long)workspace_bytes, workspace ? "" : ", NULL");
  }
  mgs::ActHost ah{};
  ah.kind = MGS_ACT_IDENTITY;
  ah.s = ah.inv_s = ah.limit = ah.alpha = 1.0f;
  ah.beta = 0.0f;
  const mgs::QOut q = make_qout(out_row, out_col, width);
  return hip_status(mgs::launch_act_fwd(ah, fmt, gt, width, x_bf16, false, nullptr, q, group_amax, col_sum,
                                        static_cast<float*>(workspace), nullptr,
                                        static_cast<hipStream_t>(stream)));
}

int64_t mgs_grouped_mx_quantize_workspace_bytes(const mgs_groups* groups, int64_t width) {
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if ((rc = check_width(width, "width"))) return rc;
  ok();
  return mgs::col_sum_part_bytes(gt, width);
}

int mgs_grouped_gemm_mx(int32_t mode, int32_t fmt, const mgs_groups* groups, int64_t m, int64_t n,
                        int64_t k, const mgs_qbuf* a, const mgs_qbuf* b, void* c, int32_t c_dtype,
                        const void* bias_bf16, int32_t accumulate, void* stream) {
  if (mode != MGS_GEMM_FPROP && mode != MGS_GEMM_DGRAD && mode != MGS_GEMM_WGRAD)
    return fail(MGS_ERR_INVALID_ARG, "unknown GEMM mode %d", mode);
  if (!valid_fmt(fmt)) return fail(MGS_ERR_INVALID_ARG, "unknown format %d", fmt);
  if (c_dtype != MGS_DTYPE_BF16 && c_dtype != MGS_DTYPE_F32)
    return fail(MGS_ERR_INVALID_ARG, "unknown output dtype %d", c_dtype);
  if (accumulate && c_dtype != MGS_DTYPE_F32)
    return fail(MGS_ERR_UNSUPPORTED, "accumulate needs an FP32 output");
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if (!a || !a->data || !a->scales) return fail(MGS_ERR_INVALID_ARG, "operand A (data, scales) is NULL");
  if (!b || !b->data || !b->scales) return fail(MGS_ERR_INVALID_ARG, "operand B (data, scales) is NULL");
  if (fmt == MGS_FMT_NVFP4 && (!a->group_scale || !b->group_scale))
    return fail(MGS_ERR_INVALID_ARG, "NVFP4 operands need group_scale");
  if (!c) return fail(MGS_ERR_INVALID_ARG, "c is NULL");
  if ((rc = check_width(n, "n"))) return rc;
  if (mode == MGS_GEMM_WGRAD) {
    if ((rc = check_width(m, "m"))) return rc;
    if (k != rows) return fail(MGS_ERR_SHAPE, "WGRAD k = %lld must equal the split sum %lld", (long long)k, (long long)rows);
    if (bias_bf16) return fail(MGS_ERR_INVALID_ARG, "bias is not defined for WGRAD");
  } else {
    if ((rc = check_width(k, "k"))) return rc;
    if (m != rows) return fail(MGS_ERR_SHAPE, "m = %lld must equal the split sum %lld", (long long)m, (long long)rows);
  }
  mgs::GemmArgs ga{};
  ga.mode = mode;
  ga.fmt = fmt;
  ga.m = m;
  ga.n = n;
  ga.k = k;
  ga.a_data = static_cast<const uint8_t*>(a->data);
  ga.a_scales = static_cast<const uint8_t*>(a->scales);
  ga.a_gscale = a->group_scale;
  ga.b_data = static_cast<const uint8_t*>(b->data);
  ga.b_scales = static_cast<const uint8_t*>(b->scales);
  ga.b_gscale = b->group_scale;
  ga.c = c;
  ga.c_f32 = c_dtype == MGS_DTYPE_F32;
  ga.accumulate = accumulate != 0;
  ga.bias = static_cast<const uint16_t*>(bias_bf16);
  if (mgs::gemm_tile_count(ga, gt) > INT32_MAX / 2) return fail(MGS_ERR_SHAPE, "too many tiles");
  return hip_status(mgs::launch_gemm(ga, gt, static_cast<hipStream_t>(stream), dev_gemm_table(groups)));
}

int mgs_grouped_gemm_mx_fprop_act(const mgs_groups* groups, int64_t m, int64_t n, int64_t k,
                                  const mgs_qbuf* a, const mgs_qbuf* b, void* c_bf16,
                                  const void* bias_bf16, const mgs_act_params* act, const float* probs,
                                  int32_t act_input, const mgs_qbuf* out_row, void* stream) {
  mgs::ActHost ah;
  int rc = check_act(act, &ah);
  if (rc) return rc;
  if (is_gated(ah.kind))
    return fail(MGS_ERR_UNSUPPORTED, "gated activations need both halves of a row: use the separate forward");
  if (act_input != MGS_DTYPE_BF16 && act_input != MGS_DTYPE_F32)
    return fail(MGS_ERR_INVALID_ARG, "unknown act_input %d", act_input);
  if (!out_row || !out_row->data || !out_row->scales)
    return fail(MGS_ERR_INVALID_ARG, "out_row (data, scales) is NULL");
  if (out_row->rht) return fail(MGS_ERR_UNSUPPORTED, "out_row.rht: the Hadamard transform applies to columnwise copies");
  mgs::GroupTable gt;
  int64_t rows = 0;
  if ((rc = build_groups(groups, &gt, &rows))) return rc;
  if (!a || !a->data || !a->scales) return fail(MGS_ERR_INVALID_ARG, "operand A (data, scales) is NULL");
  if (!b || !b->data || !b->scales) return fail(MGS_ERR_INVALID_ARG, "operand B (data, scales) is NULL");
  if (!c_bf16) return fail(MGS_ERR_INVALID_ARG, "c_bf16 is NULL");
  if ((rc = check_width(n, "n"))) return rc;
  if ((rc = check_width(k, "k"))) return rc;
  if (m != rows) return fail(MGS_ERR_SHAPE, "m = %lld must equal the split sum %lld", (long long)m, (long long)rows);
  mgs::GemmArgs ga{};
  ga.mode = MGS_GEMM_FPROP;
  ga.fmt = MGS_FMT_MXFP8;
  ga.m = m;
  ga.n = n;
  ga.k = k;
  ga.a_data = static_cast<const uint8_t*>(a->data);
  ga.a_scales = static_cast<const uint8_t*>(a->scales);
  ga.b_data = static_cast<const uint8_t*>(b->data);
  ga.b_scales = static_cast<const uint8_t*>(b->scales);
  ga.c = c_bf16;
  ga.c_f32 = 0;
  ga.accumulate = 0;
  ga.bias = static_cast<const uint16_t*>(bias_bf16);
  ga.act_enabled = 1;
  ga.act_kind = ah.kind;
  ga.act_on_bf16 = act_input == MGS_DTYPE_BF16;
  ga.act_s = ah.s;
  ga.act_inv_s = ah.inv_s;
  ga.act_limit = ah.limit;
  ga.act_alpha = ah.alpha;
  ga.act_beta = ah.beta;
  ga.probs = probs;
  ga.act_data = static_cast<uint8_t*>(out_row->data);
  ga.act_scales = static_cast<uint8_t*>(out_row->scales);
  if (mgs::gemm_tile_count(ga, gt) > INT32_MAX / 2) return fail(MGS_ERR_SHAPE, "too many tiles");
  return hip_status(mgs::launch_gemm(ga, gt, static_cast<hipStream_t>(stream), dev_gemm_table(groups)));
}

int mgs_grouped_col_sum(const mgs_groups* groups, int64_t width, const void* x_bf16, float* out,
                        void* stream) {
  mgs::GroupTable gt;
  int64_t rows = 0;
  int rc = build_groups(groups, &gt, &rows);
  if (rc) return rc;
  if (width <= 0 || width % 8 != 0) return fail(MGS_ERR_SHAPE, "width must be a positive multiple of 8");
  if (!x_bf16 && rows > 0) return fail(MGS_ERR_INVALID_ARG, "x_bf16 is NULL");
  if (!out) return fail(MGS_ERR_INVALID_ARG, "out is NULL");
  return hip_status(mgs::launch_col_sum(gt, width, static_cast<const uint16_t*>(x_bf16), out,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
