// Fused grouped scaled activation + block quantization kernels for gfx950.
//
// The method (page "Activation + GroupedLinear Fusion for MOE", Greptile summary, first bullet):
// per-row scale x activation x grouped quantization in one pass over the FC1 output, forward and
// backward; the backward also returns the per-row scale gradient.  The recompute variant (page
// "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU", Description) regenerates the
// columnwise quantized activation from the saved BF16 input inside the backward launch.
//
// Work decomposition.  A workgroup (4 waves) owns one 32-row panel of one group and 512 output
// columns per iteration; each lane owns an 8 x 8 tile (8 rows x 8 consecutive columns):
//   lane = 4 * cc + rc : rc = row chunk (rows 8rc..8rc+7), cc = column chunk (columns 8cc..8cc+7)
// so the 4 lanes of a quad share a column (columnwise block = 32 rows = the quad: DPP quad_perm),
// and lanes {rc + 4k, k = 0..3} of a 16-lane DPP row share a 32-column rowwise block (DPP row_ror).
// Both block maxima are therefore register-only reductions; nothing goes through LDS except the
// cross-wave sum of the per-row scale gradient.
//
// Memory.  Inputs are read with 16-byte loads (8 BF16 per lane, 256 contiguous bytes per row and
// wave); rowwise codes go out as 8-byte stores (128 contiguous bytes per row and wave), columnwise
// codes as 8-byte stores (32 contiguous token bytes per column and panel).  Consecutive panels of a
// column tile are placed on the same XCD so the columnwise lines they share are merged in one L2.
#include "mgs_device.h"

namespace mgs {
namespace {

struct PanelInfo {
  int g;
  int row0;     // first global row of the panel
  int nrows;    // real rows in the panel (1..32)
  int lpanel;   // panel index within the group
  int64_t coff; // padded columnwise token offset of the group
  int64_t mp;   // padded token count of the group
};

__device__ __forceinline__ PanelInfo find_panel(const GroupTable& gt, int panel) {
  int lo = 0, hi = gt.num_groups;  // panel_off[lo] <= panel < panel_off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (gt.panel_off[mid] <= panel) lo = mid; else hi = mid;
  }
  PanelInfo pi;
  pi.g = lo;
  pi.lpanel = panel - gt.panel_off[lo];
  pi.row0 = gt.row_off[lo] + PANEL_ROWS * pi.lpanel;
  int end = gt.row_off[lo + 1];
  pi.nrows = min(PANEL_ROWS, end - pi.row0);  // <= 0 for the padding panels of the columnwise layout
  pi.coff = (int64_t)PANEL_ROWS * gt.panel_off[lo];
  pi.mp = (int64_t)PANEL_ROWS * (gt.panel_off[lo + 1] - gt.panel_off[lo]);
  return pi;
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of
// logical tiles so neighbouring panels share one L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int q = n >> 3, r = n & 7;
  int x = b & 7, i = b >> 3;
  return x * q + min(x, r) + i;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// ---------------------------------------------------------------------------------- tile emitters

// Rowwise quantization of an 8 x 8 tile: rows r0 + i (i < 8, real when lr0 + i < nrows), columns
// col..col+7 of a quantized tensor of width w.
// MXFP8 scales are grouped per 128-wide K step (the byte of row r, 32-block kb of an R-row matrix
// sits at ((kb / 4) * R + r) * 4 + kb % 4); `srows` is R.  Unused bytes of a partial last step are
// written as zero by the lane that owns the row's last block.
template <int FMT>
__device__ __forceinline__ void emit_row(const float (&y)[8][8], uint8_t* __restrict__ data,
                                         uint8_t* __restrict__ scales, int64_t w, int64_t srows,
                                         int64_t r0, int lr0, int nrows, int64_t col, bool valid,
                                         int lane, float s_enc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(y[i][j]));
    const bool rv = valid && (lr0 + i) < nrows;
    const int64_t r = r0 + i;
    if constexpr (FMT == MGS_FMT_MXFP8) {
      m = row4_max(m);
      const uint32_t c = mx_scale_code(m);
      const float inv = mx_inv_scale(c);
      uint2 q;
      q.x = e4m3x4(y[i][0] * inv, y[i][1] * inv, y[i][2] * inv, y[i][3] * inv);
      q.y = e4m3x4(y[i][4] * inv, y[i][5] * inv, y[i][6] * inv, y[i][7] * inv);
      if (rv) {
        *reinterpret_cast<uint2*>(data + r * w + col) = q;
        if (((lane >> 2) & 3) == 0) {
          const int64_t kb = col >> 5, nkb = w >> 5;
          scales[(((kb >> 2) * srows + r) << 2) + (kb & 3)] = (uint8_t)c;
          if (kb == nkb - 1)
            for (int64_t t = kb + 1; t < ((nkb + 3) & ~(int64_t)3); ++t)
              scales[(((t >> 2) * srows + r) << 2) + (t & 3)] = 0;
        }
      }
    } else {
      m = pair4_max(m);
      const NvBlock b = nv_block(m, s_enc);
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = b.r != 0.0f ? y[i][j] * b.r : 0.0f;
      const uint32_t q = e2m1x8(v);
      if (rv) {
        *reinterpret_cast<uint32_t*>(data + ((r * w + col) >> 1)) = q;
        if (((lane >> 2) & 1) == 0) scales[r * (w >> 4) + (col >> 4)] = (uint8_t)b.code;
      }
    }
  }
}

// Columnwise quantization of an 8 x 8 tile whose rows are tokens lr0..lr0+7 of panel `pi` (rows
// beyond the group are zeros in y and are written as zero padding).
template <int FMT>
__device__ __forceinline__ void emit_col(const float (&y)[8][8], uint8_t* __restrict__ data,
                                         uint8_t* __restrict__ scales, int64_t w,
                                         const PanelInfo& pi, int lr0, int64_t col, bool valid,
                                         float s_enc) {
  const int64_t tok = (int64_t)PANEL_ROWS * pi.lpanel + lr0;  // token index within the group
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(y[i][j]));
    const int64_t cj = col + j;
    if constexpr (FMT == MGS_FMT_MXFP8) {
      m = quad_max(m);
      const uint32_t c = mx_scale_code(m);
      const float inv = mx_inv_scale(c);
      uint2 q;
      q.x = e4m3x4(y[0][j] * inv, y[1][j] * inv, y[2][j] * inv, y[3][j] * inv);
      q.y = e4m3x4(y[4][j] * inv, y[5][j] * inv, y[6][j] * inv, y[7][j] * inv);
      if (valid) {
        *reinterpret_cast<uint2*>(data + w * pi.coff + cj * pi.mp + tok) = q;
        // K-step grouped scales of the group's [w x mp] matrix (mp is a multiple of 128)
        const int64_t tb = tok >> 5;
        if (lr0 == 0) scales[((w * pi.coff) >> 5) + (((tb >> 2) * w + cj) << 2) + (tb & 3)] = (uint8_t)c;
      }
    } else {
      m = pair1_max(m);
      const NvBlock b = nv_block(m, s_enc);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = b.r != 0.0f ? y[i][j] * b.r : 0.0f;
      const uint32_t q = e2m1x8(v);
      if (valid) {
        *reinterpret_cast<uint32_t*>(data + ((w * pi.coff + cj * pi.mp + tok) >> 1)) = q;
        if ((lr0 & 8) == 0) scales[((w * pi.coff) >> 4) + cj * (pi.mp >> 4) + (tok >> 4)] = (uint8_t)b.code;
      }
    }
  }
}

template <int KIND>
constexpr bool is_gated() { return KIND == MGS_ACT_SWIGLU || KIND == MGS_ACT_CLAMPED_SWIGLU; }

// y = a(x) * p for the lane's 8 x 8 tile (zeros for rows outside the panel or invalid columns)
template <int KIND>
__device__ __forceinline__ void compute_y(const ActArgs& aa, const uint16_t* __restrict__ x,
                                          const float* __restrict__ probs, int64_t width_in,
                                          int64_t wa, const PanelInfo& pi, int lr0, int64_t col,
                                          bool valid, float (&y)[8][8]) {
  uint4 xg[8], xu[8];
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < pi.nrows;
    const int64_t r = pi.row0 + lr0 + i;
    xg[i] = rv ? ld16(x + r * width_in + col) : make_uint4(0, 0, 0, 0);
    if constexpr (is_gated<KIND>()) xu[i] = rv ? ld16(x + r * width_in + wa + col) : make_uint4(0, 0, 0, 0);
    p[i] = rv ? (probs ? probs[r] : 1.0f) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float g[8];
    unpack8(xg[i], g);
    if constexpr (is_gated<KIND>()) {
      float u[8];
      unpack8(xu[i], u);
#pragma unroll
      for (int j = 0; j < 8; ++j) y[i][j] = act_gated<KIND>(g[j], u[j], aa) * p[i];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[i][j] = act_unary<KIND>(g[j], aa) * p[i];
    }
  }
}

// ---------------------------------------------------------------------------------- kernels

__global__ void zero_f32_kernel(float* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0.0f;
}

// max|y| per group (NVFP4 first pass): one unsigned atomic max per wave on the FP32 bit pattern of
// a non-negative value, which orders like the value itself; the result is order-independent.
template <int KIND>
__global__ __launch_bounds__(256) void act_amax_kernel(ActArgs aa, GroupTable gt,
                                                       const uint16_t* __restrict__ x,
                                                       const float* __restrict__ probs,
                                                       int64_t width_in, int64_t wa, int n_ct,
                                                       float* __restrict__ amax) {
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = t / n_ct, ct = t - panel * n_ct;
  const PanelInfo pi = find_panel(gt, panel);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr0 = 8 * (lane & 3);
  const int64_t col = (int64_t)ct * TILE_COLS + wave * 128 + 8 * (lane >> 2);
  const bool valid = col < wa;
  float y[8][8];
  compute_y<KIND>(aa, x, probs, width_in, wa, pi, lr0, col, valid, y);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(y[i][j]));
  m = quad_max(m);
  m = row4_max(m);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(amax + pi.g), __float_as_uint(m));
}

// S_dec = 1 / S_enc per group, written once per launch (covers empty groups too)
__device__ __forceinline__ void write_group_scales(const GroupTable& gt, const QOut& q) {
  if (blockIdx.x != 0 || q.amax == nullptr) return;
  for (int g = threadIdx.x; g < gt.num_groups; g += blockDim.x) {
    const float s_dec = 1.0f / nv_encode_scale(q.amax[g]);
    if (q.row_gscale) q.row_gscale[g] = s_dec;
    if (q.col_gscale) q.col_gscale[g] = s_dec;
  }
}

template <int KIND, int FMT>
__global__ __launch_bounds__(256) void act_fwd_kernel(ActArgs aa, GroupTable gt,
                                                      const uint16_t* __restrict__ x,
                                                      const float* __restrict__ probs,
                                                      int64_t width_in, QOut out, int n_ct) {
  const int64_t wa = out.width;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = t / n_ct, ct = t - panel * n_ct;
  const PanelInfo pi = find_panel(gt, panel);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr0 = 8 * (lane & 3);
  const int64_t col = (int64_t)ct * TILE_COLS + wave * 128 + 8 * (lane >> 2);
  const bool valid = col < wa;
  float s_enc = 1.0f;
  if constexpr (FMT == MGS_FMT_NVFP4) {
    write_group_scales(gt, out);
    s_enc = nv_encode_scale(out.amax[pi.g]);
  }
  float y[8][8];
  compute_y<KIND>(aa, x, probs, width_in, wa, pi, lr0, col, valid, y);
  if (out.row_data)
    emit_row<FMT>(y, out.row_data, out.row_scales, wa, gt.total_rows, pi.row0 + lr0, lr0, pi.nrows, col, valid, lane, s_enc);
  if (out.col_data) emit_col<FMT>(y, out.col_data, out.col_scales, wa, pi, lr0, col, valid, s_enc);
}

// Backward tile computation: dx (one or two 8 x 8 tiles), y = a * p (recompute) and dp partials.
template <int KIND>
struct BwdTile {
  float d0[8][8];  // dx for columns col.. (unary) or the gate half (gated)
  float d1[8][8];  // dx for the up half (gated only)
};

template <int KIND, int FMT>
__global__ __launch_bounds__(256) void act_bwd_kernel(ActArgs aa, GroupTable gt,
                                                      const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ dy,
                                                      const float* __restrict__ probs,
                                                      int64_t width_in, int64_t wa,
                                                      uint16_t* __restrict__ dx, QOut dxq,
                                                      float* __restrict__ dprobs, QOut actq,
                                                      int n_ct_total, int ct_per_wg) {
  constexpr bool GATED = is_gated<KIND>();
  __shared__ float dp_lds[4][PANEL_ROWS];
  const int n_grid_ct = (n_ct_total + ct_per_wg - 1) / ct_per_wg;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = t / n_grid_ct, ctg = t - panel * n_grid_ct;
  const PanelInfo pi = find_panel(gt, panel);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr0 = 8 * (lane & 3);
  float s_dx = 1.0f, s_act = 1.0f;
  if constexpr (FMT == MGS_FMT_NVFP4) {
    write_group_scales(gt, dxq);
    write_group_scales(gt, actq);
    if (dxq.amax) s_dx = nv_encode_scale(dxq.amax[pi.g]);
    if (actq.amax) s_act = nv_encode_scale(actq.amax[pi.g]);
  }
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = (lr0 + i) < pi.nrows;
    p[i] = rv ? (probs ? probs[pi.row0 + lr0 + i] : 1.0f) : 0.0f;
  }
  float dpacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dpacc[i] = 0.0f;

  const int ct_end = min(n_ct_total, (ctg + 1) * ct_per_wg);
  for (int ct = ctg * ct_per_wg; ct < ct_end; ++ct) {
    const int64_t col = (int64_t)ct * TILE_COLS + wave * 128 + 8 * (lane >> 2);
    const bool valid = col < wa;
    uint4 xg[8], xu[8], dyv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool rv = valid && (lr0 + i) < pi.nrows;
      const int64_t r = pi.row0 + lr0 + i;
      xg[i] = rv ? ld16(x + r * width_in + col) : make_uint4(0, 0, 0, 0);
      if constexpr (GATED) xu[i] = rv ? ld16(x + r * width_in + wa + col) : make_uint4(0, 0, 0, 0);
      dyv[i] = rv ? ld16(dy + r * wa + col) : make_uint4(0, 0, 0, 0);
    }
    float d0[8][8], yv[8][8];
    float d1[GATED ? 8 : 1][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float g[8], dd[8];
      unpack8(xg[i], g);
      unpack8(dyv[i], dd);
      if constexpr (GATED) {
        float u[8];
        unpack8(xu[i], u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float a, dg, du;
          dact_gated<KIND>(g[j], u[j], aa, a, dg, du);
          d0[i][j] = (dg * dd[j]) * p[i];
          d1[i][j] = (du * dd[j]) * p[i];
          dpacc[i] += dd[j] * a;
          yv[i][j] = a * p[i];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = act_unary<KIND>(g[j], aa);
          d0[i][j] = (dact_unary<KIND>(g[j], aa) * dd[j]) * p[i];
          dpacc[i] += dd[j] * a;
          yv[i][j] = a * p[i];
        }
      }
    }
    const int64_t r0 = pi.row0 + lr0;
    if (dx) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (valid && (lr0 + i) < pi.nrows) {
          *reinterpret_cast<uint4*>(dx + (r0 + i) * width_in + col) = pack8_bf16(d0[i]);
          if constexpr (GATED) *reinterpret_cast<uint4*>(dx + (r0 + i) * width_in + wa + col) = pack8_bf16(d1[i]);
        }
      }
    }
    if (dxq.row_data) {
      emit_row<FMT>(d0, dxq.row_data, dxq.row_scales, width_in, gt.total_rows, r0, lr0, pi.nrows, col, valid, lane, s_dx);
      if constexpr (GATED)
        emit_row<FMT>(d1, dxq.row_data, dxq.row_scales, width_in, gt.total_rows, r0, lr0, pi.nrows, wa + col, valid, lane, s_dx);
    }
    if (dxq.col_data) {
      emit_col<FMT>(d0, dxq.col_data, dxq.col_scales, width_in, pi, lr0, col, valid, s_dx);
      if constexpr (GATED) emit_col<FMT>(d1, dxq.col_data, dxq.col_scales, width_in, pi, lr0, wa + col, valid, s_dx);
    }
    if (actq.col_data) emit_col<FMT>(yv, actq.col_data, actq.col_scales, wa, pi, lr0, col, valid, s_act);
  }

  if (dprobs) {
    // fixed-order reduction: 4 column chunks of a 16-lane row (DPP), the 4 rows of the wave
    // (cross-row shuffles), then the 4 waves in index order
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = dpacc[i];
      v += dpp_f<DPP_ROW_ROR4>(v);
      v += dpp_f<DPP_ROW_ROR8>(v);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      dpacc[i] = v;
    }
    if (lane < 4) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dp_lds[wave][lr0 + i] = dpacc[i];
    }
    __syncthreads();
    if (threadIdx.x < PANEL_ROWS && (int)threadIdx.x < pi.nrows) {
      const int i = threadIdx.x;
      dprobs[pi.row0 + i] = ((dp_lds[0][i] + dp_lds[1][i]) + dp_lds[2][i]) + dp_lds[3][i];
    }
  }
}

// max|dx| per group over the full dx width (NVFP4 first pass of the backward)
template <int KIND>
__global__ __launch_bounds__(256) void act_bwd_amax_kernel(ActArgs aa, GroupTable gt,
                                                           const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ dy,
                                                           const float* __restrict__ probs,
                                                           int64_t width_in, int64_t wa, int n_ct,
                                                           float* __restrict__ amax) {
  constexpr bool GATED = is_gated<KIND>();
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int panel = t / n_ct, ct = t - panel * n_ct;
  const PanelInfo pi = find_panel(gt, panel);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr0 = 8 * (lane & 3);
  const int64_t col = (int64_t)ct * TILE_COLS + wave * 128 + 8 * (lane >> 2);
  const bool valid = col < wa;
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < pi.nrows;
    const int64_t r = pi.row0 + lr0 + i;
    const uint4 xg = rv ? ld16(x + r * width_in + col) : make_uint4(0, 0, 0, 0);
    const uint4 dyv = rv ? ld16(dy + r * wa + col) : make_uint4(0, 0, 0, 0);
    const float pr = rv ? (probs ? probs[r] : 1.0f) : 0.0f;
    float g[8], dd[8];
    unpack8(xg, g);
    unpack8(dyv, dd);
    if constexpr (GATED) {
      const uint4 xu = rv ? ld16(x + r * width_in + wa + col) : make_uint4(0, 0, 0, 0);
      float u[8];
      unpack8(xu, u);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a, dg, du;
        dact_gated<KIND>(g[j], u[j], aa, a, dg, du);
        m = fmaxf(m, fabsf((dg * dd[j]) * pr));
        m = fmaxf(m, fabsf((du * dd[j]) * pr));
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf((dact_unary<KIND>(g[j], aa) * dd[j]) * pr));
    }
  }
  m = quad_max(m);
  m = row4_max(m);
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(amax + pi.g), __float_as_uint(m));
}

__global__ __launch_bounds__(1024) void col_sum_kernel(GroupTable gt, int64_t width,
                                                       const uint16_t* __restrict__ x,
                                                       float* __restrict__ out) {
  // one group x 512 columns per workgroup; 16 waves take rows r = w, w + 16, ... in order, then the
  // 16 partial sums are added in wave order: a fixed summation order
  __shared__ float part[16][512];
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 512 + lane * 8;
  const bool valid = col < width;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const int r_begin = gt.row_off[g], r_end = gt.row_off[g + 1];
  if (valid) {
    for (int r = r_begin + wave; r < r_end; r += 16) {
      float v[8];
      unpack8(ld16(x + (int64_t)r * width + col), v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[wave][lane * 8 + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < 512) {
    const int c = threadIdx.x;
    float s = 0.0f;
    for (int w = 0; w < 16; ++w) s += part[w][c];
    const int64_t oc = (int64_t)blockIdx.x * 512 + c;
    if (oc < width) out[(int64_t)g * width + oc] = s;
  }
}

template <int KIND>
void fwd_dispatch_fmt(int fmt, dim3 grid, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                      const uint16_t* x, const float* probs, int64_t width_in, const QOut& out,
                      int n_ct) {
  if (fmt == MGS_FMT_MXFP8)
    hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_MXFP8>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, n_ct);
  else
    hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_NVFP4>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, n_ct);
}

template <int KIND>
void bwd_dispatch_fmt(int fmt, dim3 grid, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                      const uint16_t* x, const uint16_t* dy, const float* probs, int64_t width_in,
                      int64_t wa, uint16_t* dx, const QOut& dxq, float* dprobs, const QOut& actq,
                      int n_ct, int ct_per_wg) {
  if (fmt == MGS_FMT_MXFP8)
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_MXFP8>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg);
  else
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_NVFP4>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg);
}

ActArgs to_args(const ActHost& a) { return ActArgs{a.kind, a.s, a.inv_s, a.limit, a.alpha, a.beta}; }

}  // namespace

hipError_t launch_act_fwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const uint16_t* x, const float* probs, QOut out, float* group_amax,
                          hipStream_t st) {
  if (gt.num_panels == 0) return hipSuccess;
  const ActArgs aa = to_args(act);
  const int64_t wa = out.width;
  const int n_ct = (int)((wa + TILE_COLS - 1) / TILE_COLS);
  const dim3 grid((unsigned)((int64_t)gt.num_panels * n_ct));
  if (fmt == MGS_FMT_NVFP4) {
    hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(256), 0, st, group_amax, gt.num_groups);
    switch (act.kind) {
      case MGS_ACT_IDENTITY: hipLaunchKernelGGL((act_amax_kernel<MGS_ACT_IDENTITY>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, wa, n_ct, group_amax); break;
      case MGS_ACT_SRELU: hipLaunchKernelGGL((act_amax_kernel<MGS_ACT_SRELU>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, wa, n_ct, group_amax); break;
      case MGS_ACT_TANH_SRELU: hipLaunchKernelGGL((act_amax_kernel<MGS_ACT_TANH_SRELU>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, wa, n_ct, group_amax); break;
      case MGS_ACT_SWIGLU: hipLaunchKernelGGL((act_amax_kernel<MGS_ACT_SWIGLU>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, wa, n_ct, group_amax); break;
      default: hipLaunchKernelGGL((act_amax_kernel<MGS_ACT_CLAMPED_SWIGLU>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, wa, n_ct, group_amax); break;
    }
    out.amax = group_amax;
  }
  switch (act.kind) {
    case MGS_ACT_IDENTITY: fwd_dispatch_fmt<MGS_ACT_IDENTITY>(fmt, grid, st, aa, gt, x, probs, width_in, out, n_ct); break;
    case MGS_ACT_SRELU: fwd_dispatch_fmt<MGS_ACT_SRELU>(fmt, grid, st, aa, gt, x, probs, width_in, out, n_ct); break;
    case MGS_ACT_TANH_SRELU: fwd_dispatch_fmt<MGS_ACT_TANH_SRELU>(fmt, grid, st, aa, gt, x, probs, width_in, out, n_ct); break;
    case MGS_ACT_SWIGLU: fwd_dispatch_fmt<MGS_ACT_SWIGLU>(fmt, grid, st, aa, gt, x, probs, width_in, out, n_ct); break;
    default: fwd_dispatch_fmt<MGS_ACT_CLAMPED_SWIGLU>(fmt, grid, st, aa, gt, x, probs, width_in, out, n_ct); break;
  }
  return hipGetLastError();
}

hipError_t launch_act_bwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const uint16_t* x, const uint16_t* dy, const float* probs, uint16_t* dx,
                          QOut dxq, float* dx_amax, float* dprobs, QOut actq, hipStream_t st) {
  if (gt.num_panels == 0) return hipSuccess;
  const ActArgs aa = to_args(act);
  const bool gated = act.kind == MGS_ACT_SWIGLU || act.kind == MGS_ACT_CLAMPED_SWIGLU;
  const int64_t wa = gated ? width_in / 2 : width_in;
  const int n_ct = (int)((wa + TILE_COLS - 1) / TILE_COLS);
  const bool quant_dx = dxq.row_data || dxq.col_data;
  if (fmt == MGS_FMT_NVFP4 && quant_dx) {
    const dim3 g1((unsigned)((int64_t)gt.num_panels * n_ct));
    hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(256), 0, st, dx_amax, gt.num_groups);
    switch (act.kind) {
      case MGS_ACT_IDENTITY: hipLaunchKernelGGL((act_bwd_amax_kernel<MGS_ACT_IDENTITY>), g1, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, n_ct, dx_amax); break;
      case MGS_ACT_SRELU: hipLaunchKernelGGL((act_bwd_amax_kernel<MGS_ACT_SRELU>), g1, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, n_ct, dx_amax); break;
      case MGS_ACT_TANH_SRELU: hipLaunchKernelGGL((act_bwd_amax_kernel<MGS_ACT_TANH_SRELU>), g1, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, n_ct, dx_amax); break;
      case MGS_ACT_SWIGLU: hipLaunchKernelGGL((act_bwd_amax_kernel<MGS_ACT_SWIGLU>), g1, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, n_ct, dx_amax); break;
      default: hipLaunchKernelGGL((act_bwd_amax_kernel<MGS_ACT_CLAMPED_SWIGLU>), g1, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, n_ct, dx_amax); break;
    }
    dxq.amax = dx_amax;
  }
  // with dprobs requested a workgroup walks the whole row width (fixed-order row sums)
  const int ct_per_wg = dprobs ? n_ct : 1;
  const int n_grid_ct = (n_ct + ct_per_wg - 1) / ct_per_wg;
  const dim3 grid((unsigned)((int64_t)gt.num_panels * n_grid_ct));
  switch (act.kind) {
    case MGS_ACT_IDENTITY: bwd_dispatch_fmt<MGS_ACT_IDENTITY>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg); break;
    case MGS_ACT_SRELU: bwd_dispatch_fmt<MGS_ACT_SRELU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg); break;
    case MGS_ACT_TANH_SRELU: bwd_dispatch_fmt<MGS_ACT_TANH_SRELU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg); break;
    case MGS_ACT_SWIGLU: bwd_dispatch_fmt<MGS_ACT_SWIGLU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg); break;
    default: bwd_dispatch_fmt<MGS_ACT_CLAMPED_SWIGLU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dprobs, actq, n_ct, ct_per_wg); break;
  }
  return hipGetLastError();
}

hipError_t launch_col_sum(const GroupTable& gt, int64_t width, const uint16_t* x, float* out,
                          hipStream_t st) {
  const dim3 grid((unsigned)((width + 511) / 512), (unsigned)gt.num_groups);
  hipLaunchKernelGGL(col_sum_kernel, grid, dim3(1024), 0, st, gt, width, x, out);
  return hipGetLastError();
}

}  // namespace mgs
