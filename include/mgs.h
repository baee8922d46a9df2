/*
 * mgs.h -- C ABI of the MI355X (gfx950) library for the fused MoE expert-MLP hot path:
 * per-row scaled activation + grouped block quantization (MXFP8 / NVFP4) + grouped MX GEMM.
 *
 * Sources (web pages the method is described on):
 *   [P1] "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU" (TransformerEngine PR 3473)
 *   [P2] "Activation + GroupedLinear Fusion for MOE" (TransformerEngine PR 3238)
 *   [P3] "[PyTorch] Preserve FP8 recompute state for inner autocast" (TransformerEngine PR 3284)
 *
 * General conventions (all entry points):
 *   - Every pointer argument named *_bf16, probs, dprobs, group_amax, data, scales, group_scale, c and
 *     bias is a DEVICE pointer; mgs_groups.split_sizes and the mgs_* structs themselves are HOST memory.
 *   - The caller owns every buffer, workspaces included.  The library allocates no memory and keeps no
 *     state between calls, apart from the static device scratch of mgs_grouped_scaled_act_bwd_noalloc
 *     (and the per-device address of that scratch).
 *   - Every call validates its arguments on the host, then enqueues its kernels on `stream` (a
 *     hipStream_t; NULL = the null stream) and returns without synchronizing.
 *   - A NULL output pointer (or an mgs_qbuf with data == NULL) means "not requested": it is not computed.
 *   - Return value: MGS_OK (0) or a negative MGS_ERR_* code; nothing is enqueued when validation
 *     fails.  mgs_last_error() returns a thread-local message describing the last failure.
 *   - Row groups: `groups->split_sizes[g]` rows belong to group (expert) g, stored contiguously in
 *     group order ([P2] sequence diagram: split_sizes).  M = sum of split sizes.
 *   - Quantized widths (the quantized, contiguous dimension) must be multiples of 32, at most 2^24.
 *   - Size limits of the quantizing entry points (MGS_ERR_SHAPE beyond them): one group's columnwise
 *     matrix, roundup(m_g, 128) x W elements, stays below 2^31, and so does the byte size of the
 *     rowwise MXFP8 scale array, 4 * M * ceil(W / 128).
 *   - Arithmetic follows IEEE FP32 with round-to-nearest-even; results are deterministic (no float
 *     atomics, fixed reduction orders).
 *
 * Quantized tensor layouts (mgs_qbuf), for a logical [M x W] tensor quantized along W:
 *   MXFP8 (E4M3 elements, E8M0 scale per 32):
 *     rowwise : data u8 [M, W]                      scales: K-step grouped over [M, W]
 *     colwise : group g at data + W*coff[g]:        data [W, mp_g]   (tokens contiguous)
 *               group g at scales + W*coff[g]/32:   scales: K-step grouped over [W, mp_g]
 *   NVFP4 (E2M1 elements two per byte, element 2i in the low nibble; E4M3 scale per 16; FP32 per group):
 *     rowwise : data u8 [M, W/2]                    scales u8 [M, W/16]   group_scale f32 [E]
 *     colwise : group g at data + W*coff[g]/2:      data [W, mp_g/2]
 *               group g at scales + W*coff[g]/16:   scales [W, mp_g/16]   group_scale f32 [E]
 *   where mp_g = roundup(m_g, 128) and coff[g] = sum_{h<g} mp_h; padding tokens are written as zeros.
 *   "K-step grouped" MXFP8 scales of an [R x K] matrix keep the four 32-block scales of each
 *   128-wide K step together per row, steps outermost: the scale of (row r, block kb) is the byte
 *   ((kb / 4) * R + r) * 4 + kb % 4; 4 * R * ceil(K / 128) bytes, unused bytes of a partial last
 *   step zero.  (One aligned dword per row and K step: what the grouped GEMM stages per step.)
 *   MXFP8 scale of a block with maximum magnitude amax: E8M0 code clamp(floor(log2 amax) - 8 + 127, 0, 254)
 *   (0 for an all-zero block), element = E4M3(y / 2^(code-127)) rounded to nearest-even, saturated at 448.
 *   NVFP4 (per group g, FP32): S_enc = 2688 / amax_g (1 if amax_g == 0, FLT_MAX on overflow);
 *   block scale s_b = E4M3((amax_b / 6) * S_enc); element = E2M1(y * (S_enc / s_b)) (0 if s_b == 0);
 *   group_scale[g] = S_dec = 1 / S_enc; dequantized value = e2m1 * s_b * S_dec.
 */
#ifndef MGS_H
#define MGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MGS_ABI_VERSION 8
#define MGS_MAX_GROUPS 256
/* Size of the static per-device scratch of mgs_grouped_scaled_act_bwd_noalloc (16 MiB). */
#define MGS_NOALLOC_SCRATCH_BYTES ((int64_t)16 << 20)

enum mgs_status {
  MGS_OK = 0,
  MGS_ERR_INVALID_ARG = -1, /* NULL required pointer, unknown enum value, bad group count      */
  MGS_ERR_SHAPE = -2,       /* width not a multiple of 32, negative split, split sum mismatch,
                               size limits (see the conventions above)                          */
  MGS_ERR_UNSUPPORTED = -3, /* a valid but unsupported combination (e.g. NVFP4 recompute
                               without the forward's group amax)                                 */
  MGS_ERR_HIP = -4          /* a HIP launch error                                                */
};

/* Activation kinds.  [P2] Greptile summary (first bullet) and Important Files Changed
 * (csrc/extensions/activation.cpp): scaled SwiGLU, clamped SwiGLU and SReLU; [P1] title:
 * ScaledTanhSReLU.  With x the BF16 FC1 output row and p the row's routing probability:
 *   IDENTITY        a = x                                       (plain grouped quantize)
 *   SRELU           a = relu(x)^2
 *   TANH_SRELU      a = (s * tanh(relu(x) / s))^2               (bounded at s^2, [P1] reviewer comment)
 *   SWIGLU          x = [gate | up], a = silu(gate) * up        (output width = width_in / 2)
 *   CLAMPED_SWIGLU  g = min(gate, limit), u = clamp(up, -limit, limit), a = g * sigmoid(alpha g) * (u + beta)
 * and, through the same fused kernels and recompute path ([P1] review discussion: nothing in the
 * fused recompute is specific to SReLU; GeLU, sigmoid and the GLU family fit the same scheme):
 *   GELU            a = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))   (the exact form, not tanh-approximated)
 *   SIGMOID         a = 1 / (1 + exp(-x))
 *   GLU             x = [gate | up], a = sigmoid(gate) * up          (output width = width_in / 2)
 * The forward output is y = a * p, kept in FP32 until it is quantized. */
typedef enum {
  MGS_ACT_IDENTITY = 0,
  MGS_ACT_SRELU = 1,
  MGS_ACT_TANH_SRELU = 2,
  MGS_ACT_SWIGLU = 3,
  MGS_ACT_CLAMPED_SWIGLU = 4,
  MGS_ACT_GELU = 5,
  MGS_ACT_SIGMOID = 6,
  MGS_ACT_GLU = 7
} mgs_act_kind;

typedef enum { MGS_FMT_MXFP8 = 0, MGS_FMT_NVFP4 = 1 } mgs_fmt;

typedef enum { MGS_DTYPE_BF16 = 0, MGS_DTYPE_F32 = 1 } mgs_dtype;

typedef enum {
  MGS_GEMM_FPROP = 0, /* grouped over M: C[M x N] = A[M x K] . B_g^T, B = [E x N x K]          */
  MGS_GEMM_DGRAD = 1, /* same contraction as FPROP; B is the columnwise copy of the weight     */
  MGS_GEMM_WGRAD = 2  /* grouped over K: C_g[Mc x N] = A_g[Mc x mp_g] . B_g[N x mp_g]^T          */
} mgs_gemm_mode;

typedef enum { MGS_NBYTES_DATA = 0, MGS_NBYTES_SCALES = 1, MGS_NBYTES_GROUP_SCALE = 2 } mgs_nbytes_which;

typedef struct {
  int32_t kind;  /* mgs_act_kind */
  float s;       /* TANH_SRELU bound parameter (> 0) */
  float limit;   /* CLAMPED_SWIGLU clamp (> 0) */
  float alpha;   /* CLAMPED_SWIGLU sigmoid slope (default 1) */
  float beta;    /* CLAMPED_SWIGLU up-projection offset (default 0) */
} mgs_act_params;

/* Row groups.  Host split sizes: split_sizes points to them; max_rows and dev_table are ignored.
 *
 * Device-resident split sizes (split_sizes == NULL): the graph-safe form.  [P2] Greptile summary,
 * third bullet (GroupedLinear's graph-safe forward, _fuser_forward_graph_safe): the split sizes stay in
 * device memory, so a captured HIP graph can be replayed for a different routing without a host sync.
 *   max_rows   row capacity (> 0): every layout is strided for it, so buffer sizes do not depend on the
 *              split sizes -- rowwise tensors have max_rows rows (rows past the sum are neither read nor
 *              written), columnwise tensors a padded token count of 128 * (ceil(max_rows / 128) +
 *              num_groups), rowwise MXFP8 scales are K-step grouped over max_rows rows, and an
 *              M-grouped GEMM's m (a WGRAD's k) is max_rows.  mgs_qtensor_nbytes and the workspace-size
 *              calls return the capacity sizes.
 *   dev_table  DEVICE buffer of mgs_groups_table_bytes() bytes holding the offsets, written on the
 *              stream by mgs_groups_update (call it after every change of the split sizes; kernels of
 *              the calls enqueued after it read them).  Calls sharing a dev_table must not overlap.
 * Every call takes device-resident split sizes, for both formats; NVFP4's per-group amax and S_dec
 * are taken over the rows of each group as the device table holds them at the time of the call. */
typedef struct {
  int32_t num_groups;         /* 1 .. MGS_MAX_GROUPS */
  const int64_t* split_sizes; /* host array [num_groups], each >= 0; NULL: device-resident (above) */
  int64_t max_rows;
  void* dev_table;
} mgs_groups;

/* One orientation (rowwise or columnwise) of a grouped quantized tensor; see the layouts above. */
typedef struct {
  void* data;
  void* scales;
  float* group_scale; /* NVFP4 only: S_dec per group [E]; ignored for MXFP8 */
  /* NVFP4 columnwise copies only (0 elsewhere): random Hadamard transform of every 16-token block
   * of a column before quantization, v -> H16 diag(s) v / 4 (H16[k][n] = (-1)^popcount(k & n)).
   * 0 = off; otherwise bit 16 must be set and bits 0..15 give the signs (bit n set: s_n = -1).
   * [P1] names this recipe NVFP4_RHT for its NVFP4 measurements without defining it; it is for the
   * two operands of a weight-gradient GEMM, made with the same signs, whose product the orthogonal
   * transform leaves unchanged.  The transformed copy's per-group encode scale comes from its own
   * amax (see group_amax below); the GEMM reads such a copy like any other. */
  uint32_t rht;
} mgs_qbuf;

/* Bytes of the device table of device-resident split sizes (mgs_groups.dev_table). */
int64_t mgs_groups_table_bytes(void);

/* Device-resident split sizes: enqueues on `stream` the computation of groups->dev_table from
 * split_sizes_dev (DEVICE int64 [num_groups]).  status_dev (DEVICE int32, nullable) receives 0, or 1
 * when a split size is negative or their sum exceeds max_rows; the table then holds empty groups, so
 * the calls that follow write no output rows (a WGRAD writes zero weight gradients).  The host cannot
 * see this without a synchronization: read status_dev after the step. */
int mgs_groups_update(const mgs_groups* groups, const int64_t* split_sizes_dev, int32_t* status_dev,
                      void* stream);

/* Library ABI version (MGS_ABI_VERSION). */
int mgs_abi_version(void);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* mgs_last_error(void);

/* Byte size of one buffer of a grouped quantized tensor of width `width`:
 * which = DATA, SCALES or GROUP_SCALE (4 * E for NVFP4, 0 for MXFP8).  Negative MGS_ERR_* on error. */
int64_t mgs_qtensor_nbytes(int32_t fmt, int32_t colwise, const mgs_groups* groups, int64_t width,
                           int32_t which);

/* Fused forward: y = act(x) * p, quantized rowwise and/or columnwise in one pass over x.
 * [P2] Greptile summary, first bullet (the per-row scale, the activation and the grouped quantization
 * share one pass) and sequence diagram (the forward activation call takes x, the scales, the
 * quantizer and split_sizes and returns the grouped quantized tensor).
 *   x_bf16     [M x width_in] BF16, row-major (required unless M == 0)
 *   probs      [M] FP32 per-row scale; NULL means 1 for every row
 *   out_row    rowwise qtensor of y [M x W_a] (W_a = width_in, or width_in/2 for gated kinds); nullable
 *   out_col    columnwise qtensor of y; nullable (NULL in the recompute forward, [P1] Description)
 *   group_amax [E] FP32: NVFP4 only, required there; receives max|y| per group (the per-tensor
 *              amax of each expert slice) and must be kept for a later recompute.  Ignored for MXFP8.
 *              [2E] when out_col has the Hadamard transform (mgs_qbuf.rht): entries E..2E-1 receive
 *              the transformed values' amax, which scales the columnwise copy.
 * NVFP4 runs two passes over x (group amax, then quantize). */
int mgs_grouped_scaled_act_fwd(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                               int64_t width_in, const void* x_bf16, const float* probs,
                               const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                               void* stream);

/* Fused forward from the FP32 FC1 output.  [P1] Description and review discussion: in the fused
 * forward the activation is applied to the FP32 accumulator of the FC1 GEMM, while the backward and
 * the recompute read the saved BF16 FC1 output; the regenerated FC2 input therefore differs slightly
 * from the forward's (the deviation that page tabulates for the FC2 weight gradient).  Same outputs
 * and rules as mgs_grouped_scaled_act_fwd, except:
 *   x_f32      [M x width_in] FP32, row-major (required unless M == 0); width_in * 128 < 2^31
 *   x_bf16_out [M x width_in] BF16 nullable: receives x rounded to nearest-even, the tensor the
 *              backward and the recompute take as x_bf16 (written in the same pass)
 * At least one of out_row, out_col, x_bf16_out must be requested. */
int mgs_grouped_scaled_act_fwd_f32(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                                   int64_t width_in, const float* x_f32, const float* probs,
                                   const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                                   void* x_bf16_out, void* stream);

/* Fused backward.  [P2] sequence diagram, backward half: grouped_scaled_d{swiglu,srelu}(grad, input_,
 * scales, quantizer) -> (grouped_dy, dense_dy, grad_scales), where grad = dL/d(act_out * scales);
 * [P1] Description: activation recompute regenerates FC2's input from the saved BF16 FC1 output.
 *   x_bf16        [M x width_in] BF16 saved FC1 output (required unless M == 0)
 *   dy_bf16       [M x W_a] BF16 dL/d(a * p) (required unless M == 0)
 *   probs         [M] FP32; NULL means 1
 *   dx_bf16       [M x width_in] BF16 dense dL/dx = dy * p * a'(x); nullable
 *   dx_row/dx_col quantized dL/dx (rowwise / columnwise); nullable
 *   dx_group_amax [E] FP32: required when dx is quantized to NVFP4 (receives max|dL/dx| per group);
 *                 [2E] when dx_col has the Hadamard transform (transformed amax at E..2E-1)
 *   dprobs        [M] FP32 dL/dp = sum_j dy * a(x); nullable
 *   dx_col_sum    [E x width_in] FP32 per-group column sums of the dense BF16 dL/dx (the values dx_bf16
 *                 holds, whether or not it is requested): the FC1 bias gradient.  [P1] Description,
 *                 second paragraph (bias in the fused step).  Nullable; empty groups give zeros.
 *   act_col       columnwise qtensor of y = a(x) * p regenerated from x (recompute); nullable.  Its bytes
 *                 equal those the forward's out_col would have held.
 *   saved_group_amax [E] FP32 group amax written by the forward; required for an NVFP4 act_col
 *                 without the Hadamard transform.  With it (act_col.rht) the transformed values'
 *                 amax is taken again from x in this call (the same bits the forward's copy used)
 *                 and the workspace is required.
 *   workspace     DEVICE scratch of at least mgs_act_bwd_workspace_bytes() bytes, required when dprobs
 *                 or dx_col_sum is requested, or act_col has the Hadamard transform (else ignored;
 *                 may be NULL); owned by the caller,
 *                 contents undefined before and after the call.  The kernel writes partial sums there
 *                 (dprobs: one per row and 128-column tile; column sums: one per 128-token block and
 *                 column) and second kernels add them in a fixed order, so both are deterministic.
 *                 Calls that share a workspace must not overlap.
 *   workspace_bytes its size; MGS_ERR_INVALID_ARG when it is needed and too small. */
int mgs_grouped_scaled_act_bwd(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                               int64_t width_in, const void* x_bf16, const void* dy_bf16,
                               const float* probs, void* dx_bf16, const mgs_qbuf* dx_row,
                               const mgs_qbuf* dx_col, float* dx_group_amax, float* dprobs,
                               float* dx_col_sum, const mgs_qbuf* act_col,
                               const float* saved_group_amax, void* workspace,
                               int64_t workspace_bytes, void* stream);

/* The fused backward above without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, outputs and results (bit for bit, the same kernels) as mgs_grouped_scaled_act_bwd;
 * the partial sums go to a static scratch array of MGS_NOALLOC_SCRATCH_BYTES (16 MiB) in device
 * memory that each device holds from the first call on it until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 *   - MGS_ERR_SHAPE when the workspace the request needs (mgs_act_bwd_workspace_bytes, counted only
 *     when dprobs, dx_col_sum or a transformed act_col is requested) exceeds the scratch; nothing is
 *     enqueued then.
 *   - Every call on one device shares that device's scratch, and the scratch keeps the last call's
 *     contents (each call writes every partial it reads and zeroes its group maxima itself): calls
 *     that overlap on one device (other streams, other threads) race and must be serialized by the
 *     caller. */
int mgs_grouped_scaled_act_bwd_noalloc(const mgs_act_params* act, int32_t fmt, const mgs_groups* groups,
                                       int64_t width_in, const void* x_bf16, const void* dy_bf16,
                                       const float* probs, void* dx_bf16, const mgs_qbuf* dx_row,
                                       const mgs_qbuf* dx_col, float* dx_group_amax, float* dprobs,
                                       float* dx_col_sum, const mgs_qbuf* act_col,
                                       const float* saved_group_amax, void* stream);

/* Workspace bytes mgs_grouped_scaled_act_bwd needs for dprobs, dx_col_sum and a transformed act_col:
 * roundup(roundup(4 * M * ceil(W_a / 128), 256) + 4 * (P / 128) * width_in, 256) + 8 * E,
 * P = sum_g roundup(m_g, 128).
 * Negative MGS_ERR_* on invalid arguments. */
int64_t mgs_act_bwd_workspace_bytes(const mgs_act_params* act, const mgs_groups* groups,
                                    int64_t width_in);

/* Plain grouped quantization of a BF16 tensor (weights, upstream gradients, FC1 input): the forward
 * above with act = IDENTITY and p = 1.  [P2] Greptile summary, second bullet (GroupedLinear consumes a
 * pre-quantized grouped tensor); [P3] "A behaviour change worth calling out" (columnwise usage).
 *   out_row, out_col, group_amax as in mgs_grouped_scaled_act_fwd (group_amax required for NVFP4 when
 *              a quantized output is requested)
 *   col_sum    [E x width] FP32 per-group column sums of x in the same pass (the FC2 bias gradient when
 *              x is dL/dY2); nullable; empty groups give zeros.  At least one of out_row, out_col,
 *              col_sum must be requested.
 *   workspace  DEVICE scratch of at least mgs_grouped_mx_quantize_workspace_bytes() bytes, required
 *              when col_sum is requested (per-block partial sums, added in block order by a second
 *              kernel); caller-owned, contents undefined before and after; calls sharing it must not
 *              overlap.  workspace_bytes: its size (MGS_ERR_INVALID_ARG when needed and too small). */
int mgs_grouped_mx_quantize(int32_t fmt, const mgs_groups* groups, int64_t width, const void* x_bf16,
                            const mgs_qbuf* out_row, const mgs_qbuf* out_col, float* group_amax,
                            float* col_sum, void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes of mgs_grouped_mx_quantize's col_sum: 4 * (P / 128) * width,
 * P = sum_g roundup(m_g, 128).  Negative MGS_ERR_* on invalid arguments. */
int64_t mgs_grouped_mx_quantize_workspace_bytes(const mgs_groups* groups, int64_t width);

/* Grouped GEMM on quantized operands with FP32 accumulation.  [P2] Greptile summary, second bullet and
 * sequence diagram (GroupedLinear forward / backward on a pre-built grouped tensor).
 *   FPROP, DGRAD (grouped over M; m = M = sum of splits, n, k = reduction width, k % 32 == 0):
 *     A = rowwise qtensor [M x k];
 *     B (FPROP) = rowwise qtensor of the weight [E * n x k] (expert g owns rows g*n .. g*n + n - 1);
 *     B (DGRAD) = columnwise qtensor of the weight [E * k x n] with split_sizes [k] * E (per expert
 *                 [n x roundup(k, 128)], zero padded);
 *     C [M x n] row-major; bias_bf16 [E x n] optional.
 *   WGRAD (grouped over K; k = M = sum of splits; m, n = widths of A and B):
 *     A = columnwise qtensor of width m, B = columnwise qtensor of width n, both over the same groups;
 *     C [E x m x n] row-major (an empty group writes zeros, or leaves C unchanged if accumulating).
 *   c_dtype BF16 or F32; accumulate != 0 adds into C (F32 only).
 *   NVFP4 operands also scale each group's result by A.group_scale[g] * B.group_scale[g]. */
int mgs_grouped_gemm_mx(int32_t mode, int32_t fmt, const mgs_groups* groups, int64_t m, int64_t n,
                        int64_t k, const mgs_qbuf* a, const mgs_qbuf* b, void* c, int32_t c_dtype,
                        const void* bias_bf16, int32_t accumulate, void* stream);

/* FC1's forward GEMM with the scaled activation and MXFP8 rowwise quantization in its epilogue.
 * [P1] Description and review discussion: the fused forward applies the activation to FC1's output
 * inside the GEMM and hands FC2 its quantized input; [P2] Greptile summary (per-row scale, activation
 * and grouped quantization in one pass).  An FPROP of mgs_grouped_gemm_mx (same A, B, groups, m, n, k,
 * bias; MXFP8 only) that also writes
 *   out_row    rowwise MXFP8 qtensor [M x n] of y = act(c) * probs[row], required: the bytes
 *              mgs_grouped_scaled_act_fwd (act_input BF16) or mgs_grouped_scaled_act_fwd_f32
 *              (act_input F32) writes for out_row from this C, bit for bit
 *   c_bf16     [M x n] BF16 FC1 output, required (the tensor the backward and the recompute read)
 *   act        unary kinds only (IDENTITY, SRELU, TANH_SRELU, GELU, SIGMOID); gated kinds return
 *              MGS_ERR_UNSUPPORTED (their two halves lie in different output tiles)
 *   probs      [M] FP32 per-row scale; NULL means 1
 *   act_input  MGS_DTYPE_F32: activate the FP32 value c = A.B^T + bias; MGS_DTYPE_BF16: its BF16 rounding
 * No columnwise copy: the recompute forward needs none; callers wanting one use the separate forward. */
int mgs_grouped_gemm_mx_fprop_act(const mgs_groups* groups, int64_t m, int64_t n, int64_t k,
                                  const mgs_qbuf* a, const mgs_qbuf* b, void* c_bf16,
                                  const void* bias_bf16, const mgs_act_params* act, const float* probs,
                                  int32_t act_input, const mgs_qbuf* out_row, void* stream);

/* Per-group column sums (bias gradient): out[g, j] = sum over group g's rows of x[r, j], FP32,
 * fixed summation order.  [P1] Description, second paragraph: bias changes what wgrad consumes.
 *   x_bf16 [M x width] BF16; out [E x width] FP32 (empty groups give zeros). */
int mgs_grouped_col_sum(const mgs_groups* groups, int64_t width, const void* x_bf16, float* out,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MGS_H */
