// Internal interface between the C-ABI layer (argument validation, group bookkeeping) and the kernel
// launchers.  Not installed; the public interface is include/mgs.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mgs.h"

namespace mgs {

// Rows of one panel: a panel is 32 consecutive rows of one group, the unit of the columnwise
// quantization blocks (32 for MXFP8, 2 x 16 for NVFP4).
constexpr int PANEL_ROWS = 32;
// The columnwise (token-contiguous) layout pads each group to a multiple of 128 tokens: a whole
// number of 128-wide K steps of the weight-gradient GEMM.
constexpr int COL_ALIGN = 128;

// Group bookkeeping passed by value in the kernel arguments.
//   row_off[g]   = sum_{h<g} m_h                            (E + 1 entries)
//   panel_off[g] = sum_{h<g} roundup(m_h, 128) / 32         (E + 1 entries); the padded columnwise
//                  token offset of group g is 32 * panel_off[g] and its padded length
//                  32 * (panel_off[g+1] - panel_off[g]); panels past a group's last row are padding.
//
// Device-resident split sizes (graph-safe calls): the table passed by value then describes the
// layout for a row capacity -- total_rows = the capacity, num_panels = an upper bound of the padded
// panels -- and `dev` points to a copy in device memory that holds the actual offsets, written by
// groups_update_kernel from the device split sizes.  Kernels take offsets (row_off, panel_off and the
// actual counts) from *dev and layout strides and extents from the by-value table; null `dev`: both
// are the by-value table.
struct GroupTable {
  int32_t num_groups;
  int32_t num_panels;
  int32_t total_rows;
  int32_t row_off[MGS_MAX_GROUPS + 1];
  int32_t panel_off[MGS_MAX_GROUPS + 1];
  const GroupTable* dev;
};

// One quantized output (rowwise and/or columnwise copies) of logical width `width`.
struct QOut {
  uint8_t* row_data;
  uint8_t* row_scales;
  uint8_t* col_data;
  uint8_t* col_scales;
  float* row_gscale;  // NVFP4 S_dec outputs (may be null)
  float* col_gscale;
  const float* amax;  // NVFP4: per-group amax the encode scale derives from
  int64_t width;
  // NVFP4 columnwise copy: its per-group amax (the transformed values' with col_rht, else amax) and
  // the Hadamard transform (bit 16: on; bits 0..15: signs)
  const float* col_amax;
  uint32_t col_rht;
};

struct ActHost {
  int kind;
  float s, inv_s, limit, alpha, beta;
};

// Group table for the GEMM tile scheduler.
struct GemmTable {
  int32_t num_groups;
  int32_t total_tiles;
  int32_t tile_off[MGS_MAX_GROUPS + 1];  // cumulative tiles per group
  int32_t tok_off[MGS_MAX_GROUPS + 1];   // M-grouped: row offsets; K-grouped: padded token offsets
  // Workgroup schedule (workgroups are dealt to the 8 XCDs round-robin by index).
  //   interleave == 0: each XCD takes a contiguous range of the tile sequence (group by group).
  //   interleave == 1 (K-grouped launches, where every group has the same tiles but its own K):
  //     groups in the order `order` (largest K first); group order[s] owns workgroups
  //     s * stride .. s * stride + stride - 1 (stride = the group's tile count rounded up to a
  //     multiple of 8); its workgroup j goes to XCD j % 8 and takes the (j / 8)-th tile of that XCD's
  //     contiguous eighth of the group's tiles; workgroups past the end of an eighth do nothing.
  int32_t interleave;
  int32_t grid;                          // workgroups of the launch
  int32_t stride;
  // rows of the layout the M-grouped operand A's rowwise MXFP8 scales are strided for (the rows in
  // use, or the row capacity with device-resident split sizes)
  int32_t layout_rows;
  uint8_t order[MGS_MAX_GROUPS];
  // device-resident split sizes: the table of this launch in device memory (written by
  // gemm_table_kernel just before it); the by-value fields are then unused
  const GemmTable* dev;
};

struct GemmArgs {
  int mode;  // mgs_gemm_mode
  int fmt;   // mgs_fmt
  int64_t m, n, k;
  const uint8_t* a_data;
  const uint8_t* a_scales;
  const float* a_gscale;
  const uint8_t* b_data;
  const uint8_t* b_scales;
  const float* b_gscale;
  void* c;
  int c_f32;
  int accumulate;
  const uint16_t* bias;
  // FPROP epilogue activation (act_enabled == 0, the zero-initialised default: none).  With it the
  // epilogue also quantizes y = act(c) * probs[row] to MXFP8 rowwise: codes [M x n] at act_data,
  // scales K-step grouped over n at act_scales; c is the FP32 value (act_on_bf16 == 0) or its BF16
  // rounding (1).  C is BF16.
  int act_enabled;
  int act_kind;
  int act_on_bf16;
  float act_s, act_inv_s, act_limit, act_alpha, act_beta;
  const float* probs;
  uint8_t* act_data;
  uint8_t* act_scales;
};

// ---- launchers (return hipGetLastError() after the launches) ----

// x: BF16, or FP32 when x_f32 (then x_copy, nullable, receives its BF16 rounding, same shape).
// col_sum (nullable): per-group column sums of the output values [E x W_a]; cs_part: workspace of
// col_sum_part_bytes(gt, W_a) bytes for the per-block partial sums (used when col_sum is requested).
hipError_t launch_act_fwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const void* x, bool x_f32, const float* probs, QOut out, float* group_amax,
                          float* col_sum, float* cs_part, uint16_t* x_copy, hipStream_t stream);

// workspace: act_bwd_workspace_bytes(gt, activation width, width_in) bytes, used when dprobs or
// dx_col_sum is requested: per-row partial sums of dprobs per 128-column tile at offset 0, then (at
// act_bwd_cs_offset) per-block column partial sums of the dense dx; both are added in a fixed order
// by a second kernel.
hipError_t launch_act_bwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const uint16_t* x, const uint16_t* dy, const float* probs, uint16_t* dx,
                          QOut dxq, float* dx_amax, float* dprobs, float* dx_col_sum, void* workspace,
                          QOut actq, hipStream_t stream);
int64_t act_bwd_cs_offset(int64_t rows, int64_t wa);
int64_t act_bwd_rht_offset(const GroupTable& gt, int64_t wa, int64_t width_in);
int64_t col_sum_part_bytes(const GroupTable& gt, int64_t width);
int64_t act_bwd_workspace_bytes(const GroupTable& gt, int64_t wa, int64_t width_in);

hipError_t launch_col_sum(const GroupTable& gt, int64_t width, const uint16_t* x, float* out,
                          hipStream_t stream);

// Builds the per-group tile table for the kernel variant of `ga.fmt` and launches it.  With
// device-resident split sizes (gt.dev) the table is built on the device into `dev_gemm_table` first.
hipError_t launch_gemm(const GemmArgs& ga, const GroupTable& gt, hipStream_t stream,
                       GemmTable* dev_gemm_table = nullptr);
int64_t gemm_tile_count(const GemmArgs& ga, const GroupTable& gt);

// Device-resident split sizes: the actual group table from `splits` (device int64 [E]) into `out`
// (device), capacity `max_rows`; status (device int32): 0, or 1 when a split is negative or the
// sum exceeds the capacity (the table then describes empty groups, so every call writes nothing).
hipError_t launch_groups_update(int num_groups, const int64_t* splits, int64_t max_rows, GroupTable* out,
                                int32_t* status, hipStream_t stream);

}  // namespace mgs
