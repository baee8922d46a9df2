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

template <typename Table>
__device__ __forceinline__ PanelInfo find_panel_in(const Table& gt, int panel) {
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

// The panel's group and offsets, from the device copy of the table when the split sizes are
// device-resident (DEV), else from the table passed by value.  DEV is a template parameter so that a
// kernel reads one table only (a pointer chosen at run time between the argument and device memory
// made the compiler copy the argument table to scratch).
template <bool DEV>
__device__ __forceinline__ PanelInfo find_panel(const GroupTable& gt, int panel) {
  if constexpr (DEV) return find_panel_in(*gt.dev, panel);
  else return find_panel_in(gt, panel);
}

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a contiguous range of
// logical tiles so neighbouring panels share one L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  int q = n >> 3, r = n & 7;
  int x = b & 7, i = b >> 3;
  return x * q + min(x, r) + i;
}

// ------------------------------------------------------------------------------- buffer views
//
// Every tensor is addressed through a raw buffer descriptor whose base is the current panel (a
// wave-uniform value, so it lives in scalar registers), a 32-bit per-lane offset and a scalar offset
// for the row (or column) step.  This keeps one vector register per tensor instead of a 64-bit
// address per row.  The descriptor's record count ends the view at the end of its allocation.

using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef unsigned int v2u __attribute__((__vector_size__(8)));
typedef unsigned int v4u __attribute__((__vector_size__(16)));

// dword 3 of a gfx9-family buffer descriptor: 32-bit data format, no swizzle
constexpr int RSRC_WORD3 = 0x00020000;
// Views address at most 2^31 - 1 bytes, so a lane offset of 2^31 is always past the record count:
// the buffer unit returns zero for such a load (no memory access), which masks a lane without a
// branch.  Callers keep every real offset below 2^31 (the C-ABI layer checks the extents).
constexpr uint32_t MASKED = 0x80000000u;

// view of bytes [off, total) of an allocation
__device__ __forceinline__ rsrc_t view(const void* base, int64_t off, int64_t total) {
  int64_t n = total - off;
  n = n < 0 ? 0 : (n > 0x7FFFFFFFll ? 0x7FFFFFFFll : n);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base)) + off,
                                           (short)0, (int)n, RSRC_WORD3);
}

__device__ __forceinline__ uint4 bld16(rsrc_t r, uint32_t vo, uint32_t so) {
  const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)so, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// A store of more than 8 bytes reads its data VGPRs after it issues: on gfx950 a VALU write to one
// of them in the very next instruction changed what the last lanes of each 16-lane group stored
// (measured: they stored the new value), and the compiler does not keep the two apart for this
// target.  The empty asm keeps the data registers live until two wait states after the store.
__device__ __forceinline__ void bst16(uint4 d, rsrc_t r, uint32_t vo, uint32_t so) {
  const v4u v = {d.x, d.y, d.z, d.w};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)vo, (int)so, 0);
  asm volatile("s_nop 1" :: "v"(v));
}
__device__ __forceinline__ void bst8(uint2 d, rsrc_t r, uint32_t vo, uint32_t so) {
  const v2u v = {d.x, d.y};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ void bst4(uint32_t d, rsrc_t r, uint32_t vo, uint32_t so) {
  __builtin_amdgcn_raw_buffer_store_b32(d, r, (int)vo, (int)so, 0);
}
__device__ __forceinline__ void bst1(uint32_t d, rsrc_t r, uint32_t vo, uint32_t so) {
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)d, r, (int)vo, (int)so, 0);
}

// A BF16 row-major tensor seen from the panel's first row: element (lr, c) at byte
// ((lr * ld + c) * 2); `vo` is the lane's offset of (lr0, col), `ld2` the row pitch in bytes.
struct Bf16View {
  rsrc_t r;
  uint32_t vo, ld2;
};

__device__ __forceinline__ Bf16View bf16_view(const uint16_t* p, int64_t ld, int64_t row0,
                                              int64_t rows, int lr0, int64_t col) {
  Bf16View v;
  v.r = view(p, row0 * ld * 2, rows * ld * 2);
  v.ld2 = (uint32_t)(ld * 2);
  v.vo = ((uint32_t)lr0 * (uint32_t)ld + (uint32_t)col) * 2u;
  return v;
}

// Rowwise destination of one panel: codes of row lr0 + i at data + dvo + i * dpitch, the lane's
// block scale at scales + svo + i * spitch.
struct RowDst {
  rsrc_t data, scales;
  uint32_t dvo, dpitch, svo, spitch;
  uint32_t pad;     // MXFP8 byte mode: zero bytes to write after the row's last scale (rest of the K step)
  bool sc_lane;     // byte mode: this lane writes its block's scale
  // MXFP8 dword mode (the workgroup's 128 columns are one K step): each row's four scales are
  // gathered into the lane of column chunk 0 (sd_lane), which writes them as one dword
  bool dword_mode, sd_lane;
  bool sd_aligned;  // dword mode: the lane's eight scale dwords start 16-byte aligned
};

// MXFP8 row scales are grouped per 128-wide K step: the byte of row r, 32-block kb of an R-row
// matrix sits at ((kb / 4) * R + r) * 4 + kb % 4 (R = srows).
template <int FMT>
__device__ __forceinline__ RowDst row_dst(const QOut& q, int64_t w, int64_t srows, int64_t row0,
                                          int lr0, int64_t col, int lane) {
  RowDst d;
  if constexpr (FMT == MGS_FMT_MXFP8) {
    const int64_t nkb = w >> 5, nks = (nkb + 3) >> 2, kb = col >> 5;
    d.data = view(q.row_data, row0 * w, srows * w);
    d.scales = view(q.row_scales, row0 * 4, srows * 4 * nks);
    d.dvo = (uint32_t)lr0 * (uint32_t)w + (uint32_t)col;
    d.dpitch = (uint32_t)w;
    d.svo = (uint32_t)(kb >> 2) * (uint32_t)srows * 4u + (uint32_t)lr0 * 4u + (uint32_t)(kb & 3);
    d.spitch = 4;
    d.pad = kb == nkb - 1 ? (uint32_t)(nks * 4 - nkb) : 0u;
    d.sc_lane = ((lane >> 2) & 3) == 0;
    // the workgroup's first column (chunk 0) starts a K step: always for a unary kind or the gate
    // half, for the up half of a gated kind when its offset (the output width) is a multiple of 128
    d.dword_mode = ((col - 8 * (lane >> 2)) & 127) == 0;
    d.sd_lane = (lane >> 2) == 0;
    const uint64_t sbyte = reinterpret_cast<uint64_t>(q.row_scales) + (uint64_t)(row0 * 4) + d.svo;
    d.sd_aligned = (sbyte & 15) == 0;
  } else {
    d.data = view(q.row_data, row0 * w / 2, srows * w / 2);
    d.scales = view(q.row_scales, row0 * (w >> 4), srows * (w >> 4));
    d.dvo = ((uint32_t)lr0 * (uint32_t)w + (uint32_t)col) >> 1;
    d.dpitch = (uint32_t)(w >> 1);
    d.svo = (uint32_t)lr0 * (uint32_t)(w >> 4) + (uint32_t)(col >> 4);
    d.spitch = (uint32_t)(w >> 4);
    d.pad = 0;
    d.dword_mode = false;
    d.sd_lane = false;
    d.sd_aligned = false;
    d.sc_lane = ((lane >> 2) & 1) == 0;
  }
  return d;
}

// Columnwise destination of one panel (tokens 32 * lpanel .. +31 of the group): the codes of
// column col + j at data + dvo + j * dpitch, its block scale at scales + svo + j * spitch.
struct ColDst {
  rsrc_t data, scales;
  uint32_t dvo, dpitch, svo, spitch;
  bool sc_lane;
};

// The group's columnwise matrix is [w x mp] (mp = padded token count, a multiple of 128) at
// element offset w * coff; MXFP8 scales of it use the K-step grouping over tokens.
template <int FMT>
__device__ __forceinline__ ColDst col_dst(const QOut& q, int64_t w, int64_t total_padded,
                                          const PanelInfo& pi, int lr0, int64_t col) {
  ColDst d;
  const int64_t lp = pi.lpanel, e0 = w * pi.coff;
  const uint32_t mp = (uint32_t)pi.mp;
  if constexpr (FMT == MGS_FMT_MXFP8) {
    d.data = view(q.col_data, e0 + 32 * lp, w * total_padded);
    d.scales = view(q.col_scales, (e0 >> 5) + (((lp >> 2) * w) << 2) + (lp & 3), (w * total_padded) >> 5);
    d.dvo = (uint32_t)col * mp + (uint32_t)lr0;
    d.dpitch = mp;
    d.svo = (uint32_t)col * 4u;
    d.spitch = 4;
    d.sc_lane = lr0 == 0;
  } else {
    d.data = view(q.col_data, (e0 + 32 * lp) >> 1, (w * total_padded) >> 1);
    d.scales = view(q.col_scales, (e0 >> 4) + 2 * lp, (w * total_padded) >> 4);
    d.dvo = ((uint32_t)col * mp + (uint32_t)lr0) >> 1;
    d.dpitch = mp >> 1;
    d.svo = (uint32_t)col * (mp >> 4) + (uint32_t)(lr0 >> 4);
    d.spitch = mp >> 4;
    d.sc_lane = (lr0 & 8) == 0;
  }
  return d;
}

// ---------------------------------------------------------------------------------- tile emitters

// MXFP8 row scales of one 128-column K step: block kb's code sits in the lanes of 16-lane row kb
// (column chunks 4 kb .. 4 kb + 3); two lane swaps gather the row's four codes, kb in byte kb, into
// its chunk-0 lane (lane lr0 / 8).  `code` must be 0 for blocks past the tensor's width: their bytes
// are the zero padding of the last K step.
__device__ __forceinline__ uint32_t gather_scale_dword(uint32_t code) {
  const U2 a = swap32(code, code);        // lanes 0..31: blocks (kb, kb + 2)
  const uint32_t w = a.x | (a.y << 16);
  const U2 b = swap16(w, w);              // lanes 0..15: (w of blocks 0, 2; w of blocks 1, 3)
  return b.x | (b.y << 8);
}

// Rowwise quantization of row i (8 values) of the lane's tile; rv: the row is real, valid: the
// lane's columns are.  MXFP8 in dword mode returns the row's scale dword (in the chunk-0 lanes) for
// flush_row_scales; otherwise the lane stores its block's scale byte here.
template <int FMT>
__device__ __forceinline__ uint32_t quant_row(const float (&v)[8], const RowDst& d, int i, bool rv,
                                              bool valid, float s_enc) {
  float m = absmax8(v);
  if constexpr (FMT == MGS_FMT_MXFP8) {
    m = row4_max(m);
    const Mx8 e = mx_encode8(v, m);
    bst8(e.q, d.data, rv ? d.dvo : MASKED, i * d.dpitch);
    if (d.dword_mode) return gather_scale_dword(valid ? e.code : 0u);
    const bool sv = rv && d.sc_lane;
    bst1(e.code, d.scales, sv ? d.svo : MASKED, i * d.spitch);
#pragma unroll
    for (uint32_t t = 1; t <= 3; ++t) bst1(0, d.scales, sv && t <= d.pad ? d.svo + t : MASKED, i * d.spitch);
    return 0u;
  } else {
    m = pair4_max(m);
    const NvBlock b = nv_block(m, s_enc);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = b.r != 0.0f ? v[j] * b.r : 0.0f;
    bst4(e2m1x8(e), d.data, rv ? d.dvo : MASKED, i * d.dpitch);
    bst1(b.code, d.scales, rv && d.sc_lane ? d.svo : MASKED, i * d.spitch);
    return 0u;
  }
}

// MXFP8: the scale dwords of the tile's eight rows (rows lr0 .. lr0 + 7 of the panel, real when
// < nrows) from the chunk-0 lanes: two 16-byte stores when all eight are real and aligned, else one
// dword per real row.
template <int FMT>
__device__ __forceinline__ void flush_row_scales(const RowDst& d, const uint32_t (&sdw)[8], int lr0,
                                                 int nrows) {
  if constexpr (FMT == MGS_FMT_MXFP8) {
    if (!d.dword_mode || !d.sd_lane) return;
    if (d.sd_aligned && lr0 + 8 <= nrows) {
      bst16(make_uint4(sdw[0], sdw[1], sdw[2], sdw[3]), d.scales, d.svo, 0);
      bst16(make_uint4(sdw[4], sdw[5], sdw[6], sdw[7]), d.scales, d.svo + 16u, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) bst4(sdw[i], d.scales, lr0 + i < nrows ? d.svo + 4u * i : MASKED, 0);
    }
  }
}

// Columnwise quantization of column j (8 tokens lr0..lr0+7; rows beyond the group are zeros and
// are written as zero padding).
template <int FMT>
__device__ __forceinline__ void quant_col(const float (&v)[8], const ColDst& d, int j, bool valid,
                                          float s_enc) {
  float m = absmax8(v);
  if constexpr (FMT == MGS_FMT_MXFP8) {
    m = quad_max(m);
    const Mx8 e = mx_encode8(v, m);
    bst8(e.q, d.data, valid ? d.dvo : MASKED, j * d.dpitch);
    bst1(e.code, d.scales, valid && d.sc_lane ? d.svo : MASKED, j * d.spitch);
  } else {
    m = pair1_max(m);
    const NvBlock b = nv_block(m, s_enc);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = b.r != 0.0f ? v[i] * b.r : 0.0f;
    bst4(e2m1x8(e), d.data, valid ? d.dvo : MASKED, j * d.dpitch);
    bst1(b.code, d.scales, valid && d.sc_lane ? d.svo : MASKED, j * d.spitch);
  }
}

// Rowwise quantization of a whole 8 x 8 tile (rows lr0 + i of the panel, real when < nrows).
template <int FMT>
__device__ __forceinline__ void emit_row(const float (&y)[8][8], const RowDst& d, int lr0, int nrows,
                                         bool valid, float s_enc) {
  uint32_t sdw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) sdw[i] = quant_row<FMT>(y[i], d, i, valid && (lr0 + i) < nrows, valid, s_enc);
  flush_row_scales<FMT>(d, sdw, lr0, nrows);
}

// Columnwise quantization of a whole 8 x 8 tile.
template <int FMT>
__device__ __forceinline__ void emit_col(const float (&y)[8][8], const ColDst& d, bool valid,
                                         float s_enc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = y[i][j];
    quant_col<FMT>(v, d, j, valid, s_enc);
  }
}

// element j (0..7) of a packed BF16 octet
__device__ __forceinline__ float bf16_at(const uint4& w, int j) {
  const uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
  return (j & 1) ? bf16hi(x) : bf16lo(x);
}

// An opaque copy of a packed tile row: later phases recompute from it instead of keeping the
// earlier phase's FP32 intermediates alive (common-subexpression reuse would hold 64 extra floats).
__device__ __forceinline__ void launder(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
// Pins a running sum at this point of the program (the compiler would otherwise sink loop-carried
// additions to the end of the iteration and keep all their operands alive until then).
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

template <int KIND>
constexpr bool is_gated() { return KIND == MGS_ACT_SWIGLU || KIND == MGS_ACT_CLAMPED_SWIGLU || KIND == MGS_ACT_GLU; }

// probs of the lane's 8 rows (0 for rows outside the panel, 1 when probs is null)
__device__ __forceinline__ void load_probs(const float* __restrict__ probs, const PanelInfo& pi,
                                           int64_t total_rows, int lr0, float (&p)[8]) {
  if (probs) {
    const rsrc_t r = view(probs, (int64_t)pi.row0 * 4, total_rows * 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t vo = (lr0 + i) < pi.nrows ? (uint32_t)(lr0 + i) * 4u : MASKED;
      p[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)vo, 0, 0));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = (lr0 + i) < pi.nrows ? 1.0f : 0.0f;
  }
}

// The lane's 8 x 8 BF16 input tile(s): gate (or only) half at column col, up half at wa + col.
template <bool GATED>
__device__ __forceinline__ void load_x(const Bf16View& xv, uint32_t up_off, int lr0, int nrows,
                                       bool valid, uint4 (&xg)[8], uint4 (&xu)[GATED ? 8 : 1]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < nrows;
    xg[i] = bld16(xv.r, rv ? xv.vo : MASKED, i * xv.ld2);
    if constexpr (GATED) xu[i] = bld16(xv.r, rv ? xv.vo + up_off : MASKED, i * xv.ld2);
  }
}

// y = a(x) * p for the lane's 8 x 8 tile (zeros for rows outside the panel or invalid columns)
template <int KIND>
__device__ __forceinline__ void compute_y(const ActArgs& aa, const uint4 (&xg)[8],
                                          const uint4 (&xu)[is_gated<KIND>() ? 8 : 1],
                                          const float (&p)[8], float (&y)[8][8]) {
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

// An FP32 row-major tensor seen from the panel's first row, in the same view type: element (lr, c)
// at byte ((lr * ld + c) * 4); a lane's 8 consecutive values are two 16-byte loads.
__device__ __forceinline__ Bf16View f32_view(const float* p, int64_t ld, int64_t row0, int64_t rows,
                                             int lr0, int64_t col) {
  Bf16View v;
  v.r = view(p, row0 * ld * 4, rows * ld * 4);
  v.ld2 = (uint32_t)(ld * 4);
  v.vo = ((uint32_t)lr0 * (uint32_t)ld + (uint32_t)col) * 4u;
  return v;
}

__device__ __forceinline__ void load_row8_f32(const Bf16View& xv, uint32_t vo, uint32_t so, float (&v)[8]) {
  const uint4 a = bld16(xv.r, vo, so);
  const uint4 b = bld16(xv.r, vo == MASKED ? MASKED : vo + 16u, so);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// The lane's 8 x 8 FP32 input tile(s); `up_off` in bytes.
template <bool GATED>
__device__ __forceinline__ void load_x32(const Bf16View& xv, uint32_t up_off, int lr0, int nrows,
                                         bool valid, float (&xg)[8][8], float (&xu)[GATED ? 8 : 1][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < nrows;
    load_row8_f32(xv, rv ? xv.vo : MASKED, i * xv.ld2, xg[i]);
    if constexpr (GATED) load_row8_f32(xv, rv ? xv.vo + up_off : MASKED, i * xv.ld2, xu[i]);
  }
}

template <int KIND>
__device__ __forceinline__ void compute_y32(const ActArgs& aa, const float (&xg)[8][8],
                                            const float (&xu)[is_gated<KIND>() ? 8 : 1][8],
                                            const float (&p)[8], float (&y)[8][8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (is_gated<KIND>()) y[i][j] = act_gated<KIND>(xg[i][j], xu[i][j], aa) * p[i];
      else y[i][j] = act_unary<KIND>(xg[i][j], aa) * p[i];
    }
  }
}

// The input tile and y = a(x) * p of the forward kernels, from a BF16 or (XF32) an FP32 input.  With
// an FP32 input and `x_copy`, the lane also writes the BF16 (round-to-nearest-even) copy of its tile
// into x_copy (same shape as x): the copy the backward and the recompute read.
template <int KIND, bool XF32>
__device__ __forceinline__ void fwd_tile_y(const ActArgs& aa, const GroupTable& gt, const PanelInfo& pi,
                                           const void* x, uint16_t* x_copy, int64_t width_in, int64_t wa,
                                           int lr0, int64_t col, bool valid, const float (&p)[8],
                                           float (&y)[8][8]) {
  constexpr bool GATED = is_gated<KIND>();
  if constexpr (XF32) {
    const Bf16View xv = f32_view(static_cast<const float*>(x), width_in, pi.row0, gt.total_rows, lr0, col);
    float xg[8][8], xu[GATED ? 8 : 1][8];
    load_x32<GATED>(xv, (uint32_t)wa * 4u, lr0, pi.nrows, valid, xg, xu);
    if (x_copy) {
      const Bf16View cv = bf16_view(x_copy, width_in, pi.row0, gt.total_rows, lr0, col);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool rv = valid && (lr0 + i) < pi.nrows;
        bst16(pack8_bf16(xg[i]), cv.r, rv ? cv.vo : MASKED, i * cv.ld2);
        if constexpr (GATED) bst16(pack8_bf16(xu[i]), cv.r, rv ? cv.vo + (uint32_t)wa * 2u : MASKED, i * cv.ld2);
      }
    }
    compute_y32<KIND>(aa, xg, xu, p, y);
  } else {
    const Bf16View xv = bf16_view(static_cast<const uint16_t*>(x), width_in, pi.row0, gt.total_rows, lr0, col);
    uint4 xg[8], xu[GATED ? 8 : 1];
    load_x<GATED>(xv, (uint32_t)wa * 2u, lr0, pi.nrows, valid, xg, xu);
    compute_y<KIND>(aa, xg, xu, p, y);
  }
}

// ---------------------------------------------------------------------------------- kernels

__global__ void zero_f32_kernel(float* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0.0f;
}

// S_dec = 1 / S_enc per group, written once per launch (covers empty groups too)
__device__ __forceinline__ void write_group_scales(const GroupTable& gt, const QOut& q) {
  if (blockIdx.x != 0 || q.amax == nullptr) return;
  for (int g = threadIdx.x; g < gt.num_groups; g += blockDim.x) {
    if (q.row_gscale) q.row_gscale[g] = 1.0f / nv_encode_scale(q.amax[g]);
    if (q.col_gscale) q.col_gscale[g] = 1.0f / nv_encode_scale(q.col_amax[g]);
  }
}

// --------------------------------------------------------------------- 128-token block tiles
//
// The quantizing kernels give a workgroup one 128-token block of one group (groups are padded to a
// multiple of 128 tokens in the columnwise layout, so a block never straddles two groups) and 128
// columns: wave w owns panel 4 b + w (32 rows) and each lane its 8 x 8 tile of it.  Rowwise codes
// go straight to memory (16 lanes write a row's 128 contiguous bytes).  Columnwise codes are staged
// in LDS and written afterwards by the whole workgroup as complete 128-token column segments: one
// 128-byte line per column for MXFP8 (64 bytes for NVFP4) instead of four 32-byte pieces written by
// four workgroups.  The MXFP8 column scales of the block are then the four bytes of one K step, so
// each column's scales leave as one aligned dword.

constexpr int BLOCK_COLS = 128;

template <int FMT>
struct Stage {
  // bytes per staged column: the block's codes plus 8 bytes of padding, which spreads the lanes'
  // 8-byte writes of eight columns apart over four bank groups instead of one
  static constexpr int PITCH = FMT == MGS_FMT_MXFP8 ? 136 : 72;
  static constexpr int SCALES = FMT == MGS_FMT_MXFP8 ? 4 : 8;  // scale bytes per column and block
  static constexpr int BYTES = BLOCK_COLS * (PITCH + SCALES);
};

struct BlockPos {
  bool ok;        // the workgroup has a block (false: it exits at once)
  PanelInfo pi;   // the wave's panel
  int gb;         // 128-token block index over all groups (columnwise padded rows / 128)
  int blk;        // 128-token block index within the group
  int ct;         // 128-column tile
  int lane, wave, lr0, cc;
  int64_t col0;   // first column of the workgroup
  int64_t col;    // the lane's first column
};

template <bool DEV>
__device__ __forceinline__ BlockPos block_pos(const GroupTable& gt, int n_ct) {
  BlockPos bp;
  // Blocks in use: the whole grid, or with device-resident split sizes (a grid sized for the row
  // capacity) those of the actual panels.  Each XCD takes a contiguous range of them (workgroups are
  // dealt to the 8 XCDs round-robin); workgroups past the end of their XCD's range have no block.
  int n;
  if constexpr (DEV) n = n_ct * (gt.dev->num_panels >> 2);
  else n = (int)gridDim.x;
  const int x = blockIdx.x & 7, i = blockIdx.x >> 3, q = n >> 3, r = n & 7;
  bp.ok = i < q + (x < r ? 1 : 0);
  if (!bp.ok) return bp;
  const int t = x * q + min(x, r) + i;
  const int b = t / n_ct;
  bp.ct = t - b * n_ct;
  bp.lane = threadIdx.x & 63;
  bp.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bp.pi = find_panel<DEV>(gt, 4 * b + bp.wave);
  bp.gb = b;
  bp.blk = bp.pi.lpanel >> 2;
  bp.lr0 = 8 * (bp.lane & 3);
  bp.cc = bp.lane >> 2;
  bp.col0 = (int64_t)bp.ct * BLOCK_COLS;
  bp.col = bp.col0 + 8 * bp.cc;
  return bp;
}

// Quantize column j (8 tokens of the lane) into the stage: codes at column c = 8 cc + j, tokens
// 32 w + lr0 .. +7; the block scale at the column's scale slot.
template <int FMT>
__device__ __forceinline__ void stage_col(const float (&v)[8], uint8_t* st, const BlockPos& bp, int j,
                                          float s_enc) {
  constexpr int P = Stage<FMT>::PITCH;
  const int c = 8 * bp.cc + j;
  float m = absmax8(v);
  if constexpr (FMT == MGS_FMT_MXFP8) {
    m = quad_max(m);
    const Mx8 e = mx_encode8(v, m);
    *reinterpret_cast<uint2*>(st + c * P + 32 * bp.wave + bp.lr0) = e.q;
    if (bp.lr0 == 0) st[BLOCK_COLS * P + 4 * c + bp.wave] = (uint8_t)e.code;
  } else {
    m = pair1_max(m);
    const NvBlock b = nv_block(m, s_enc);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = b.r != 0.0f ? v[i] * b.r : 0.0f;
    *reinterpret_cast<uint32_t*>(st + c * P + 16 * bp.wave + (bp.lr0 >> 1)) = e2m1x8(e);
    if ((bp.lr0 & 8) == 0) st[BLOCK_COLS * P + 8 * c + 2 * bp.wave + (bp.lr0 >> 4)] = (uint8_t)b.code;
  }
}

// Random Hadamard transform of a 16-token block of one column (the weight-gradient operands of the
// NVFP4 recipe the recompute page names NVFP4_RHT): v -> H16 diag(s) v / 4, H16[k][n] =
// (-1)^popcount(k & n), s_n = -1 where bit n of `rht` is set.  The block is the lane pair (rc, rc ^ 1)
// of a quad: the lane holds tokens 8 (rc & 1) + i.  Three butterfly stages run in the lane (token bits
// 0..2), the fourth across the pair (DPP quad_perm [1,0,3,2]); the scaling by 1/4 is exact.
__device__ __forceinline__ void rht16_col(float (&v)[8], uint32_t rht, int rc) {
  const int base = 8 * (rc & 1);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((rht >> (base + i)) & 1u) v[i] = -v[i];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float o = dpp_f<DPP_QUAD_XOR1>(v[i]);
    v[i] = ((rc & 1) ? o - v[i] : v[i] + o) * 0.25f;
  }
}

// Columnwise staging of a whole tile; `rht` (NVFP4 only, wave-uniform): bit 16 enables the Hadamard
// transform of each column's 16-token blocks before quantization, bits 0..15 are its signs.
template <int FMT>
__device__ __forceinline__ void stage_tile(const float (&y)[8][8], uint8_t* st, const BlockPos& bp,
                                           float s_enc, uint32_t rht = 0) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = y[i][j];
    if (FMT == MGS_FMT_NVFP4 && rht) rht16_col(v, rht, bp.lane & 3);
    stage_col<FMT>(v, st, bp, j, s_enc);
  }
}

// Write a staged block (after a barrier) to the group's columnwise tensor of width w: the data of
// column cj at w * coff + cj * mp + 128 blk (elements), MXFP8 scales as the K-step dword of
// (blk, cj), NVFP4 scales as 8 bytes at cj * mp / 16 + 8 blk.
template <int FMT>
__device__ __forceinline__ void flush_col(const uint8_t* st, const QOut& q, int64_t w,
                                          int64_t total_padded, const BlockPos& bp) {
  constexpr int P = Stage<FMT>::PITCH;
  const int64_t e0 = w * bp.pi.coff;
  const uint32_t mp = (uint32_t)bp.pi.mp;
  const int t = threadIdx.x;
  if constexpr (FMT == MGS_FMT_MXFP8) {
    const rsrc_t dv = view(q.col_data, e0 + 128 * (int64_t)bp.blk, w * total_padded);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int idx = t + 256 * k, c = idx >> 3, ch = idx & 7;
      const uint2 a = *reinterpret_cast<const uint2*>(st + c * P + 16 * ch);
      const uint2 b = *reinterpret_cast<const uint2*>(st + c * P + 16 * ch + 8);
      const bool ok = bp.col0 + c < w;
      bst16(make_uint4(a.x, a.y, b.x, b.y), dv, ok ? (uint32_t)(bp.col0 + c) * mp + 16u * ch : MASKED, 0);
    }
    const rsrc_t sv = view(q.col_scales, (e0 >> 5) + 4 * ((int64_t)bp.blk * w + bp.col0), (w * total_padded) >> 5);
    if (t < BLOCK_COLS) {
      const uint32_t d = *reinterpret_cast<const uint32_t*>(st + BLOCK_COLS * P + 4 * t);
      bst4(d, sv, bp.col0 + t < w ? 4u * t : MASKED, 0);
    }
  } else {
    const rsrc_t dv = view(q.col_data, (e0 + 128 * (int64_t)bp.blk) >> 1, (w * total_padded) >> 1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = t + 256 * k, c = idx >> 2, ch = idx & 3;
      const uint2 a = *reinterpret_cast<const uint2*>(st + c * P + 16 * ch);
      const uint2 b = *reinterpret_cast<const uint2*>(st + c * P + 16 * ch + 8);
      const bool ok = bp.col0 + c < w;
      bst16(make_uint4(a.x, a.y, b.x, b.y), dv, ok ? ((uint32_t)(bp.col0 + c) * mp >> 1) + 16u * ch : MASKED, 0);
    }
    const rsrc_t sv = view(q.col_scales, (e0 >> 4) + 8 * (int64_t)bp.blk, (w * total_padded) >> 4);
    if (t < BLOCK_COLS) {
      const uint2 d = *reinterpret_cast<const uint2*>(st + BLOCK_COLS * P + 8 * t);
      bst8(d, sv, bp.col0 + t < w ? (uint32_t)(bp.col0 + t) * (mp >> 4) : MASKED, 0);
    }
  }
}

// Per-group column sums (bias gradients) fused into a block pass.  The lane's sums over its 8 rows
// (rows in increasing order), then its quad (the four lanes of a column chunk: (l0 + l1) + (l2 + l3)),
// go to LDS per wave; after a barrier, thread t < 128 adds the four waves' sums of column t in wave
// order and stores the block's partial sum at part[gb * ld + col].  A second kernel adds a group's
// blocks in block order.  Every order is fixed: the result is deterministic.
__device__ __forceinline__ void cs_stage(float (&s)[8], float* lds, const BlockPos& bp) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s[j] += dpp_f<DPP_QUAD_XOR1>(s[j]);
    s[j] += dpp_f<DPP_QUAD_XOR2>(s[j]);
  }
  if ((bp.lane & 3) == 0) {
    float4* d = reinterpret_cast<float4*>(lds + bp.wave * BLOCK_COLS + 8 * bp.cc);
    d[0] = make_float4(s[0], s[1], s[2], s[3]);
    d[1] = make_float4(s[4], s[5], s[6], s[7]);
  }
}

__device__ __forceinline__ void cs_flush(const float* lds, float* __restrict__ part, int64_t ld,
                                         int64_t col0, int64_t w_lim, int64_t out_off, int gb) {
  const int t = threadIdx.x;
  if (t < BLOCK_COLS && col0 + t < w_lim) {
    const float v = ((lds[t] + lds[BLOCK_COLS + t]) + lds[2 * BLOCK_COLS + t]) + lds[3 * BLOCK_COLS + t];
    part[(int64_t)gb * ld + out_off + col0 + t] = v;
  }
}

template <int KIND, int FMT, bool XF32, bool DEV>
__global__ __launch_bounds__(256) void act_fwd_kernel(ActArgs aa, GroupTable gt,
                                                      const void* __restrict__ x,
                                                      const float* __restrict__ probs,
                                                      int64_t width_in, QOut out, float* __restrict__ cs_part,
                                                      int n_ct, uint16_t* __restrict__ x_copy) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[Stage<FMT>::BYTES];
  __shared__ __attribute__((aligned(16))) float cs_lds[4 * BLOCK_COLS];
  const int64_t wa = out.width;
  const BlockPos bp = block_pos<DEV>(gt, n_ct);
  if (!bp.ok) return;
  const PanelInfo& pi = bp.pi;
  const bool valid = bp.col < wa;
  float s_enc = 1.0f, s_enc_col = 1.0f;
  if constexpr (FMT == MGS_FMT_NVFP4) {
    write_group_scales(gt, out);
    s_enc = nv_encode_scale(out.amax[pi.g]);
    s_enc_col = nv_encode_scale(out.col_amax[pi.g]);
  }
  float p[8];
  load_probs(probs, pi, gt.total_rows, bp.lr0, p);
  float y[8][8];
  fwd_tile_y<KIND, XF32>(aa, gt, pi, x, x_copy, width_in, wa, bp.lr0, bp.col, valid, p, y);
  if (out.row_data)
    emit_row<FMT>(y, row_dst<FMT>(out, wa, gt.total_rows, pi.row0, bp.lr0, bp.col, bp.lane), bp.lr0, pi.nrows, valid, s_enc);
  if (cs_part) {
    float cs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      cs[j] = y[0][j];
#pragma unroll
      for (int i = 1; i < 8; ++i) cs[j] += y[i][j];
    }
    cs_stage(cs, cs_lds, bp);
  }
  if (out.col_data) stage_tile<FMT>(y, stage, bp, s_enc_col, out.col_rht);
  if (out.col_data || cs_part) {
    __syncthreads();
    if (out.col_data) flush_col<FMT>(stage, out, wa, (int64_t)PANEL_ROWS * gt.num_panels, bp);
    if (cs_part) cs_flush(cs_lds, cs_part, wa, bp.col0, wa, 0, bp.gb);
  }
}

// Backward.  Per 8 x 8 tile: dx (the gate half for gated kinds) is computed once into an FP32 tile
// by rows (dense BF16 store, rowwise codes and dprobs partial sums as each row completes), then
// staged by columns; gated kinds repeat this for the up half in the same registers; the recompute
// variant then regenerates y = a * p from the packed input by columns.  The packed inputs are
// laundered before a later phase so the compiler evaluates it afresh instead of keeping the first
// phase's values alive.  dprobs leaves as one partial sum per row and 128-column tile in `dp_part`
// ([n_ct x M]); a second kernel adds the partials in tile order.

// dx of element (gate half or the only half): returns (da/dg * dy) * p, and a(x) through `a`
template <int KIND>
__device__ __forceinline__ float dx_gate(const ActArgs& aa, float g, float u, float dd, float p, float& a) {
  if constexpr (is_gated<KIND>()) {
    float dg, du;
    dact_gated<KIND>(g, u, aa, a, dg, du);
    return (dg * dd) * p;
  } else if constexpr (KIND == MGS_ACT_SRELU) {
    // (2 r dy) p computed as (r dy)(2 p): r dy is exact (two BF16 values) and so is 2 p, so both
    // round once, to the same value
    const float r = relu(g);
    a = r * r;
    return (r * dd) * (p + p);
  } else {
    a = act_unary<KIND>(g, aa);
    return (dact_unary<KIND>(g, aa) * dd) * p;
  }
}

// dx of the up half (gated kinds)
template <int KIND>
__device__ __forceinline__ float dx_up(const ActArgs& aa, float g, float u, float dd, float p) {
  float a, dg, du;
  dact_gated<KIND>(g, u, aa, a, dg, du);
  return (du * dd) * p;
}

template <int KIND, int FMT, bool DEV>
__global__ __launch_bounds__(256) void act_bwd_kernel(ActArgs aa, GroupTable gt,
                                                      const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ dy,
                                                      const float* __restrict__ probs,
                                                      int64_t width_in, int64_t wa,
                                                      uint16_t* __restrict__ dx, QOut dxq,
                                                      float* __restrict__ dp_part, float* __restrict__ cs_part,
                                                      QOut actq, int n_ct) {
  constexpr bool GATED = is_gated<KIND>();
  constexpr int SB = Stage<FMT>::BYTES;
  // stages: dx columnwise (gate half), dx columnwise (up half, gated kinds), recomputed activation
  __shared__ __attribute__((aligned(16))) uint8_t stage[(GATED ? 3 : 2) * SB];
  // column sums of the dense BF16 dx: gate half (or the only half), up half
  __shared__ __attribute__((aligned(16))) float cs_lds[(GATED ? 2 : 1) * 4 * BLOCK_COLS];
  uint8_t* st_dx = stage;
  uint8_t* st_up = stage + SB;
  uint8_t* st_act = stage + (GATED ? 2 : 1) * SB;
  const BlockPos bp = block_pos<DEV>(gt, n_ct);
  if (!bp.ok) return;
  const PanelInfo& pi = bp.pi;
  const int lr0 = bp.lr0;
  const int64_t col = bp.col;
  const bool valid = col < wa;
  const int64_t total_padded = (int64_t)PANEL_ROWS * gt.num_panels;
  float s_dx = 1.0f, s_dx_col = 1.0f, s_act = 1.0f;
  if constexpr (FMT == MGS_FMT_NVFP4) {
    write_group_scales(gt, dxq);
    write_group_scales(gt, actq);
    if (dxq.amax) s_dx = nv_encode_scale(dxq.amax[pi.g]);
    if (dxq.amax) s_dx_col = nv_encode_scale(dxq.col_amax[pi.g]);
    if (actq.col_data && actq.col_amax) s_act = nv_encode_scale(actq.col_amax[pi.g]);
  }
  const uint32_t up2 = (uint32_t)wa * 2u;  // byte offset of the up half in a BF16 row

  const Bf16View xv = bf16_view(x, width_in, pi.row0, gt.total_rows, lr0, col);
  const Bf16View dyv = bf16_view(dy, wa, pi.row0, gt.total_rows, lr0, col);
  uint4 xg[8], xu[GATED ? 8 : 1], dyt[8];
  load_x<GATED>(xv, up2, lr0, pi.nrows, valid, xg, xu);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < pi.nrows;
    dyt[i] = bld16(dyv.r, rv ? dyv.vo : MASKED, i * dyv.ld2);
  }
  float p[8];
  load_probs(probs, pi, gt.total_rows, lr0, p);
  const Bf16View dxv = bf16_view(dx, width_in, pi.row0, gt.total_rows, lr0, col);
  const RowDst rd = row_dst<FMT>(dxq, width_in, gt.total_rows, pi.row0, lr0, col, bp.lane);

  // recompute first: y = a * p -> columnwise codes of the activation, one column of the lane's tile
  // at a time, so that the inputs (not 64 FP32 results) are what stays live into the dx phase; the
  // inputs are laundered afterwards so that phase evaluates a(x) afresh instead of keeping these
  if (actq.col_data) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (GATED) v[i] = act_gated<KIND>(bf16_at(xg[i], j), bf16_at(xu[GATED ? i : 0], j), aa) * p[i];
        else v[i] = act_unary<KIND>(bf16_at(xg[i], j), aa) * p[i];
      }
      if (FMT == MGS_FMT_NVFP4 && actq.col_rht) rht16_col(v, actq.col_rht, bp.lane & 3);
      stage_col<FMT>(v, st_act, bp, j, s_act);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      launder(xg[i]);
      if constexpr (GATED) launder(xu[GATED ? i : 0]);
    }
  }

  float d[8][8], dpacc[8];
  uint32_t sdw[8];
  // column sums over the lane's rows (in row order) of the BF16-rounded dx, the values the dense
  // output holds; taken from the finished tile so that no accumulators live through the row loop
  auto col_sums = [&](float* lds) {
    float cs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t w = bf16x2(d[i][j], d[i + 1][j]);
        cs[j] = i == 0 ? bf16lo(w) : cs[j] + bf16lo(w);
        cs[j] += bf16hi(w);
      }
    }
    cs_stage(cs, lds, bp);
  };
  // rows: dx (gate half) -> dense store, rowwise codes, dprobs partials
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool rv = valid && (lr0 + i) < pi.nrows;
    dpacc[i] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a;
      const float dd = bf16_at(dyt[i], j);
      d[i][j] = dx_gate<KIND>(aa, bf16_at(xg[i], j), GATED ? bf16_at(xu[GATED ? i : 0], j) : 0.0f, dd, p[i], a);
      dpacc[i] = __builtin_fmaf(dd, a, dpacc[i]);
    }
    pin(dpacc[i]);
    if (dx) bst16(pack8_bf16(d[i]), dxv.r, rv ? dxv.vo : MASKED, i * dxv.ld2);
    if (dxq.row_data) sdw[i] = quant_row<FMT>(d[i], rd, i, rv, valid, s_dx);
  }
  if (dxq.row_data) flush_row_scales<FMT>(rd, sdw, lr0, pi.nrows);
  if (cs_part) col_sums(cs_lds);
  if (dxq.col_data) stage_tile<FMT>(d, st_dx, bp, s_dx_col, dxq.col_rht);
  // gated: the up half in the same registers
  if constexpr (GATED) {
    const RowDst ru = row_dst<FMT>(dxq, width_in, gt.total_rows, pi.row0, lr0, wa + col, bp.lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      launder(xg[i]);
      launder(xu[GATED ? i : 0]);
      launder(dyt[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool rv = valid && (lr0 + i) < pi.nrows;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        d[i][j] = dx_up<KIND>(aa, bf16_at(xg[i], j), bf16_at(xu[GATED ? i : 0], j), bf16_at(dyt[i], j), p[i]);
      if (dx) bst16(pack8_bf16(d[i]), dxv.r, rv ? dxv.vo + up2 : MASKED, i * dxv.ld2);
      if (dxq.row_data) sdw[i] = quant_row<FMT>(d[i], ru, i, rv, valid, s_dx);
    }
    if (dxq.row_data) flush_row_scales<FMT>(ru, sdw, lr0, pi.nrows);
    if (cs_part) col_sums(cs_lds + 4 * BLOCK_COLS);
    if (dxq.col_data) stage_tile<FMT>(d, st_up, bp, s_dx_col, dxq.col_rht);
  }

  if (dp_part) {
    // fixed-order sum over the tile's 16 column chunks: DPP within a 16-lane row, then the rows
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = dpacc[i];
      v += dpp_f<DPP_ROW_ROR4>(v);
      v += dpp_f<DPP_ROW_ROR8>(v);
      // + the lane 16 apart, then + the lane 32 apart (lane swaps: a + b is the same either way round)
      const U2 h = swap16(__float_as_uint(v), __float_as_uint(v));
      v = __uint_as_float(h.x) + __uint_as_float(h.y);
      const U2 w = swap32(__float_as_uint(v), __float_as_uint(v));
      v = __uint_as_float(w.x) + __uint_as_float(w.y);
      dpacc[i] = v;
    }
    if (bp.lane < 4) {
      const int64_t first = (int64_t)bp.ct * gt.total_rows + pi.row0;
      const rsrc_t r = view(dp_part, first * 4, (int64_t)n_ct * gt.total_rows * 4);
      // the lane's eight rows are contiguous: two 16-byte stores when all are real and aligned
      if (((reinterpret_cast<uintptr_t>(dp_part) >> 2) + first + lr0) % 4 == 0 &&
          (reinterpret_cast<uintptr_t>(dp_part) & 3) == 0 && lr0 + 8 <= pi.nrows) {
        bst16(make_uint4(__float_as_uint(dpacc[0]), __float_as_uint(dpacc[1]), __float_as_uint(dpacc[2]),
                         __float_as_uint(dpacc[3])), r, (uint32_t)lr0 * 4u, 0);
        bst16(make_uint4(__float_as_uint(dpacc[4]), __float_as_uint(dpacc[5]), __float_as_uint(dpacc[6]),
                         __float_as_uint(dpacc[7])), r, (uint32_t)lr0 * 4u + 16u, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          bst4(__float_as_uint(dpacc[i]), r, (lr0 + i) < pi.nrows ? (uint32_t)(lr0 + i) * 4u : MASKED, 0);
      }
    }
  }

  if (dxq.col_data || actq.col_data || cs_part) {
    __syncthreads();
    if (cs_part) {
      cs_flush(cs_lds, cs_part, width_in, bp.col0, wa, 0, bp.gb);
      if constexpr (GATED) cs_flush(cs_lds + 4 * BLOCK_COLS, cs_part, width_in, bp.col0, wa, wa, bp.gb);
    }
    if (dxq.col_data) {
      flush_col<FMT>(st_dx, dxq, width_in, total_padded, bp);
      if constexpr (GATED) {
        BlockPos bu = bp;
        bu.col0 += wa;
        flush_col<FMT>(st_up, dxq, width_in, total_padded, bu);
      }
    }
    if (actq.col_data) flush_col<FMT>(st_act, actq, wa, total_padded, bp);
  }
}

// Sum of n partials p[0], p[stride], ... in index order.  The loads go out eight at a time so that a
// thread waits for one memory round trip per eight partials rather than one per partial.
__device__ __forceinline__ float ordered_sum(const float* __restrict__ p, int64_t stride, int n) {
  float s = 0.0f;
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(i + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; i < n; ++i) s += p[(int64_t)i * stride];
  return s;
}

// The fixed-order sums of the partials, in one launch.  Workgroups [0, dp_blocks): dprobs[r] = the sum
// over the column tiles of dp_part[ct * rows + r], in tile order (`rows` is the row stride; with
// device-resident split sizes only the rows in use are written).  The rest, one per group and 256
// columns (cs_bx per group): cs_out[g, c] = the sum of group g's 128-token block partials
// cs_part[block * width + c], in block order.
template <bool DEV>
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ dp_part, int n_ct, int rows,
                                                     float* __restrict__ dprobs, int dp_blocks,
                                                     const float* __restrict__ cs_part, GroupTable gt,
                                                     int64_t width, float* __restrict__ cs_out, int cs_bx) {
  const int b = blockIdx.x;
  if (b < dp_blocks) {
    const int r = b * 256 + threadIdx.x;
    int used;
    if constexpr (DEV) used = gt.dev->total_rows;
    else used = rows;
    if (r < used) dprobs[r] = ordered_sum(dp_part + r, rows, n_ct);
    return;
  }
  const int k = b - dp_blocks, g = k / cs_bx;
  const int64_t c = (int64_t)(k - g * cs_bx) * 256 + threadIdx.x;
  if (c >= width) return;
  int b0, b1;
  if constexpr (DEV) {
    b0 = gt.dev->panel_off[g] >> 2;
    b1 = gt.dev->panel_off[g + 1] >> 2;
  } else {
    b0 = gt.panel_off[g] >> 2;
    b1 = gt.panel_off[g + 1] >> 2;
  }
  cs_out[(int64_t)g * width + c] = ordered_sum(cs_part + (int64_t)b0 * width + c, width, b1 - b0);
}

// Per-group column sums.  A workgroup owns one group x 128 columns; lane (rs = lane / 16,
// cc = lane % 16) of wave w adds rows 16 t + 4 w + rs (t = 0, 1, ...) of columns 8 cc..8 cc+7 in
// increasing t, then the 16 partial sums of a column are added in (w, rs) order: a fixed order.
constexpr int CS_COLS = 128;
constexpr int CS_UNROLL = 8;

template <bool DEV>
__global__ __launch_bounds__(256) void col_sum_kernel(GroupTable gt, int64_t width,
                                                      const uint16_t* __restrict__ x,
                                                      float* __restrict__ out) {
  __shared__ float part[16][CS_COLS];
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rs = lane >> 4, cc = lane & 15;
  const int slot = 4 * wave + rs;
  const int64_t col = (int64_t)blockIdx.x * CS_COLS + 8 * cc;
  const bool valid = col < width;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int r_begin, r_end;
  if constexpr (DEV) {
    r_begin = gt.dev->row_off[g];
    r_end = gt.dev->row_off[g + 1];
  } else {
    r_begin = gt.row_off[g];
    r_end = gt.row_off[g + 1];
  }
  const uint32_t ld2 = (uint32_t)width * 2u;
  const uint32_t vo = (uint32_t)slot * ld2 + (uint32_t)col * 2u;
  for (int rb = r_begin; rb < r_end; rb += 16 * CS_UNROLL) {
    const rsrc_t r = view(x, (int64_t)rb * width * 2, (int64_t)gt.total_rows * width * 2);
    uint4 v[CS_UNROLL];
#pragma unroll
    for (int u = 0; u < CS_UNROLL; ++u) {
      const bool ok = valid && rb + 16 * u + slot < r_end;
      v[u] = bld16(r, ok ? vo : MASKED, (uint32_t)(16 * u) * ld2);
    }
#pragma unroll
    for (int u = 0; u < CS_UNROLL; ++u) {
      float f[8];
      unpack8(v[u], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += f[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) part[slot][8 * cc + j] = acc[j];
  __syncthreads();
  if (threadIdx.x < CS_COLS) {
    const int c = threadIdx.x;
    float s = 0.0f;
    for (int k = 0; k < 16; ++k) s += part[k][c];
    const int64_t oc = (int64_t)blockIdx.x * CS_COLS + c;
    if (oc < width) out[(int64_t)g * width + oc] = s;
  }
}

// Group amax for NVFP4 (first pass).  A workgroup owns one 128-token block (wave w: panel 4b + w)
// and a run of `cpw` 128-column chunks, takes max |value| over them in registers (DPP and shuffles
// over the wave, LDS over the four waves) and adds one unsigned atomic max of the FP32 bits to its
// group's entry: far fewer atomics on the per-group array (one cache line for all groups) than one
// per wave.  BWD: the value is dx = (da/dg * dy) * p (both halves for gated kinds); else y = a * p.
// With `rht` (bit 16 set) the pass also takes the maximum of the Hadamard-transformed columns (the
// columnwise copy's values) into amax[E + g].
template <int KIND, bool BWD, bool XF32, bool DEV>
__global__ __launch_bounds__(256) void group_amax_kernel(ActArgs aa, GroupTable gt,
                                                         const void* __restrict__ xp,
                                                         const uint16_t* __restrict__ dy,
                                                         const float* __restrict__ probs,
                                                         int64_t width_in, int64_t wa, int n_chunks,
                                                         int cpw, float* __restrict__ amax, uint32_t rht) {
  constexpr bool GATED = is_gated<KIND>();
  __shared__ float wmax[2][4];
  const BlockPos bp = block_pos<DEV>(gt, (n_chunks + cpw - 1) / cpw);
  if (!bp.ok) return;
  const PanelInfo& pi = bp.pi;
  const int lr0 = bp.lr0;
  float p[8];
  load_probs(probs, pi, gt.total_rows, lr0, p);
  float m = 0.0f, mt = 0.0f;
  // max |.| of a tile, and of its transformed columns
  auto take = [&](const float (&t)[8][8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(t[i][j]));
    if (rht) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = t[i][j];
        rht16_col(v, rht, bp.lane & 3);
#pragma unroll
        for (int i = 0; i < 8; ++i) mt = fmaxf(mt, fabsf(v[i]));
      }
    }
  };
  const int c_end = min(n_chunks, (bp.ct + 1) * cpw);
  for (int c = bp.ct * cpw; c < c_end; ++c) {
    const int64_t col = (int64_t)c * BLOCK_COLS + 8 * bp.cc;
    const bool valid = col < wa;
    if constexpr (BWD) {
      const uint16_t* x = static_cast<const uint16_t*>(xp);
      const Bf16View xv = bf16_view(x, width_in, pi.row0, gt.total_rows, lr0, col);
      uint4 xg[8], xu[GATED ? 8 : 1];
      load_x<GATED>(xv, (uint32_t)wa * 2u, lr0, pi.nrows, valid, xg, xu);
      const Bf16View dyv = bf16_view(dy, wa, pi.row0, gt.total_rows, lr0, col);
      uint4 dyt[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool rv = valid && (lr0 + i) < pi.nrows;
        dyt[i] = bld16(dyv.r, rv ? dyv.vo : MASKED, i * dyv.ld2);
      }
      float dg[8][8], du[GATED ? 8 : 1][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float dd = bf16_at(dyt[i], j), g = bf16_at(xg[i], j);
          if constexpr (GATED) {
            const float u = bf16_at(xu[GATED ? i : 0], j);
            float a, dgv, duv;
            dact_gated<KIND>(g, u, aa, a, dgv, duv);
            dg[i][j] = (dgv * dd) * p[i];
            du[GATED ? i : 0][j] = (duv * dd) * p[i];
          } else {
            dg[i][j] = (dact_unary<KIND>(g, aa) * dd) * p[i];
          }
        }
      }
      take(dg);
      if constexpr (GATED) take(du);
    } else {
      float y[8][8];
      fwd_tile_y<KIND, XF32>(aa, gt, pi, xp, nullptr, width_in, wa, lr0, col, valid, p, y);
      take(y);
    }
  }
  auto reduce = [&](float v) {
    v = quad_max(v);
    v = row4_max(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
  };
  m = reduce(m);
  if (rht) mt = reduce(mt);
  if (bp.lane == 0) {
    wmax[0][bp.wave] = m;
    wmax[1][bp.wave] = mt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(wmax[0][0], wmax[0][1]), fmaxf(wmax[0][2], wmax[0][3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax + pi.g), __float_as_uint(b));
    if (rht) {
      const float bt = fmaxf(fmaxf(wmax[1][0], wmax[1][1]), fmaxf(wmax[1][2], wmax[1][3]));
      atomicMax(reinterpret_cast<unsigned int*>(amax + gt.num_groups + pi.g), __float_as_uint(bt));
    }
  }
}

// chunks per workgroup of the amax pass: about 1024 workgroups for small inputs, at most 8 chunks each
// for large ones (measured on 32k x 4096 and 64k x 4096 inputs: 4 or 16 chunks per workgroup are both
// slower than 8)
int amax_cpw(const GroupTable& gt, int n_chunks) {
  const int64_t units = (int64_t)(gt.num_panels / 4) * n_chunks;
  int64_t c = units / 1024;
  return (int)(c < 1 ? 1 : (c > 8 ? 8 : c));
}

template <int KIND, bool BWD>
void launch_group_amax(hipStream_t st, const ActArgs& aa, const GroupTable& gt, const void* x, bool x_f32,
                       const uint16_t* dy, const float* probs, int64_t width_in, int64_t wa,
                       float* amax, uint32_t rht) {
  const int n_chunks = (int)((wa + BLOCK_COLS - 1) / BLOCK_COLS);
  const int cpw = amax_cpw(gt, n_chunks);
  const dim3 grid((unsigned)((int64_t)(gt.num_panels / 4) * ((n_chunks + cpw - 1) / cpw)));
  if (gt.dev) {
    if (!BWD && x_f32)
      hipLaunchKernelGGL((group_amax_kernel<KIND, false, true, true>), grid, dim3(256), 0, st, aa, gt, x, dy, probs,
                         width_in, wa, n_chunks, cpw, amax, rht);
    else
      hipLaunchKernelGGL((group_amax_kernel<KIND, BWD, false, true>), grid, dim3(256), 0, st, aa, gt, x, dy, probs,
                         width_in, wa, n_chunks, cpw, amax, rht);
  } else if (!BWD && x_f32) {
    hipLaunchKernelGGL((group_amax_kernel<KIND, false, true, false>), grid, dim3(256), 0, st, aa, gt, x, dy, probs,
                       width_in, wa, n_chunks, cpw, amax, rht);
  } else {
    hipLaunchKernelGGL((group_amax_kernel<KIND, BWD, false, false>), grid, dim3(256), 0, st, aa, gt, x, dy, probs,
                       width_in, wa, n_chunks, cpw, amax, rht);
  }
}

// Zeroes `amax` (E entries, 2E with rht) and takes the group maxima into it.
template <bool BWD>
void group_amax_dispatch(int kind, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                         const void* x, bool x_f32, const uint16_t* dy, const float* probs,
                         int64_t width_in, int64_t wa, float* amax, uint32_t rht) {
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(256), 0, st, amax, (rht ? 2 : 1) * gt.num_groups);
  switch (kind) {
    case MGS_ACT_IDENTITY: launch_group_amax<MGS_ACT_IDENTITY, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_SRELU: launch_group_amax<MGS_ACT_SRELU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_TANH_SRELU: launch_group_amax<MGS_ACT_TANH_SRELU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_SWIGLU: launch_group_amax<MGS_ACT_SWIGLU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_GELU: launch_group_amax<MGS_ACT_GELU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_SIGMOID: launch_group_amax<MGS_ACT_SIGMOID, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    case MGS_ACT_GLU: launch_group_amax<MGS_ACT_GLU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
    default: launch_group_amax<MGS_ACT_CLAMPED_SWIGLU, BWD>(st, aa, gt, x, x_f32, dy, probs, width_in, wa, amax, rht); break;
  }
}

template <int KIND, bool XF32>
void fwd_dispatch_fmt(int fmt, dim3 grid, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                      const void* x, const float* probs, int64_t width_in, const QOut& out,
                      float* cs_part, int n_ct, uint16_t* x_copy) {
  if (gt.dev) {
    // device-resident split sizes: the offsets come from the device table
    if (fmt == MGS_FMT_MXFP8)
      hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_MXFP8, XF32, true>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, x_copy);
    else
      hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_NVFP4, XF32, true>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, x_copy);
  } else if (fmt == MGS_FMT_MXFP8) {
    hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_MXFP8, XF32, false>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, x_copy);
  } else {
    hipLaunchKernelGGL((act_fwd_kernel<KIND, MGS_FMT_NVFP4, XF32, false>), grid, dim3(256), 0, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, x_copy);
  }
}

template <int KIND>
void fwd_dispatch(int fmt, bool x_f32, dim3 grid, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                  const void* x, const float* probs, int64_t width_in, const QOut& out, float* cs_part,
                  int n_ct, uint16_t* x_copy) {
  if (x_f32) fwd_dispatch_fmt<KIND, true>(fmt, grid, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, x_copy);
  else fwd_dispatch_fmt<KIND, false>(fmt, grid, st, aa, gt, x, probs, width_in, out, cs_part, n_ct, nullptr);
}

template <int KIND>
void bwd_dispatch_fmt(int fmt, dim3 grid, hipStream_t st, const ActArgs& aa, const GroupTable& gt,
                      const uint16_t* x, const uint16_t* dy, const float* probs, int64_t width_in,
                      int64_t wa, uint16_t* dx, const QOut& dxq, float* dp_part, float* cs_part,
                      const QOut& actq, int n_ct) {
  if (gt.dev && fmt == MGS_FMT_MXFP8)  // device-resident split sizes
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_MXFP8, true>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dp_part, cs_part, actq, n_ct);
  else if (gt.dev)
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_NVFP4, true>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dp_part, cs_part, actq, n_ct);
  else if (fmt == MGS_FMT_MXFP8)
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_MXFP8, false>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dp_part, cs_part, actq, n_ct);
  else
    hipLaunchKernelGGL((act_bwd_kernel<KIND, MGS_FMT_NVFP4, false>), grid, dim3(256), 0, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, dp_part, cs_part, actq, n_ct);
}

// dprobs from its partials (when dprobs is non-null) and the column sums from theirs (when cs_out is
// non-null), in one launch of reduce_kernel.
void launch_reduce(const GroupTable& gt, const float* dp_part, int n_ct, float* dprobs, const float* cs_part,
                   int64_t width, float* cs_out, hipStream_t st) {
  const int dp_blocks = dprobs ? (gt.total_rows + 255) / 256 : 0;
  const int cs_bx = cs_out ? (int)((width + 255) / 256) : 0;
  const int64_t grid = (int64_t)dp_blocks + (int64_t)cs_bx * gt.num_groups;
  if (grid == 0) return;
  if (gt.dev)
    hipLaunchKernelGGL(reduce_kernel<true>, dim3((unsigned)grid), dim3(256), 0, st, dp_part, n_ct, gt.total_rows,
                       dprobs, dp_blocks, cs_part, gt, width, cs_out, cs_bx);
  else
    hipLaunchKernelGGL(reduce_kernel<false>, dim3((unsigned)grid), dim3(256), 0, st, dp_part, n_ct, gt.total_rows,
                       dprobs, dp_blocks, cs_part, gt, width, cs_out, cs_bx);
}
void launch_col_sum_reduce(const GroupTable& gt, int64_t width, const float* part, float* out, hipStream_t st) {
  launch_reduce(gt, nullptr, 0, nullptr, part, width, out, st);
}

ActArgs to_args(const ActHost& a) { return ActArgs{a.kind, a.s, a.inv_s, a.limit, a.alpha, a.beta}; }

}  // namespace

hipError_t launch_act_fwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const void* x, bool x_f32, const float* probs, QOut out, float* group_amax,
                          float* col_sum, float* cs_part, uint16_t* x_copy, hipStream_t st) {
  if (gt.num_panels == 0) {
    // every group is empty: its column sums are zeros
    if (col_sum) launch_col_sum_reduce(gt, out.width, cs_part, col_sum, st);
    return hipGetLastError();
  }
  const ActArgs aa = to_args(act);
  const int64_t wa = out.width;
  const int n_ct = (int)((wa + BLOCK_COLS - 1) / BLOCK_COLS);
  const dim3 grid((unsigned)((int64_t)(gt.num_panels / 4) * n_ct));
  float* cs = col_sum ? cs_part : nullptr;
  // column sums alone: no quantized output, so no group amax pass and no format-specific work
  if (!out.row_data && !out.col_data) fmt = MGS_FMT_MXFP8;
  if (fmt == MGS_FMT_NVFP4) {
    const uint32_t rht = out.col_data ? out.col_rht : 0u;
    group_amax_dispatch<false>(act.kind, st, aa, gt, x, x_f32, nullptr, probs, width_in, wa, group_amax, rht);
    out.amax = group_amax;
    out.col_amax = rht ? group_amax + gt.num_groups : group_amax;
  }
  switch (act.kind) {
    case MGS_ACT_IDENTITY: fwd_dispatch<MGS_ACT_IDENTITY>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_SRELU: fwd_dispatch<MGS_ACT_SRELU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_TANH_SRELU: fwd_dispatch<MGS_ACT_TANH_SRELU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_SWIGLU: fwd_dispatch<MGS_ACT_SWIGLU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_GELU: fwd_dispatch<MGS_ACT_GELU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_SIGMOID: fwd_dispatch<MGS_ACT_SIGMOID>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    case MGS_ACT_GLU: fwd_dispatch<MGS_ACT_GLU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
    default: fwd_dispatch<MGS_ACT_CLAMPED_SWIGLU>(fmt, x_f32, grid, st, aa, gt, x, probs, width_in, out, cs, n_ct, x_copy); break;
  }
  if (col_sum) launch_col_sum_reduce(gt, wa, cs_part, col_sum, st);
  return hipGetLastError();
}

hipError_t launch_act_bwd(const ActHost& act, int fmt, const GroupTable& gt, int64_t width_in,
                          const uint16_t* x, const uint16_t* dy, const float* probs, uint16_t* dx,
                          QOut dxq, float* dx_amax, float* dprobs, float* dx_col_sum, void* workspace,
                          QOut actq, hipStream_t st) {
  const bool gated = act.kind == MGS_ACT_SWIGLU || act.kind == MGS_ACT_CLAMPED_SWIGLU || act.kind == MGS_ACT_GLU;
  const int64_t wa = gated ? width_in / 2 : width_in;
  float* cs_part = dx_col_sum ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                                         act_bwd_cs_offset(gt.total_rows, wa))
                              : nullptr;
  if (gt.num_panels == 0) {
    if (dx_col_sum) launch_col_sum_reduce(gt, width_in, cs_part, dx_col_sum, st);
    return hipGetLastError();
  }
  const ActArgs aa = to_args(act);
  const bool quant_dx = dxq.row_data || dxq.col_data;
  if (fmt == MGS_FMT_NVFP4 && quant_dx) {
    const uint32_t rht = dxq.col_data ? dxq.col_rht : 0u;
    group_amax_dispatch<true>(act.kind, st, aa, gt, x, false, dy, probs, width_in, wa, dx_amax, rht);
    dxq.amax = dx_amax;
    dxq.col_amax = rht ? dx_amax + gt.num_groups : dx_amax;
  }
  actq.col_amax = actq.amax;
  if (fmt == MGS_FMT_NVFP4 && actq.col_data) {
    if (actq.col_rht) {
      // the transformed copy's amax is not the forward's saved one: take it again from x into the
      // workspace (the same inputs as the forward's, so the same bits)
      float* ra = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + act_bwd_rht_offset(gt, wa, width_in));
      group_amax_dispatch<false>(act.kind, st, aa, gt, x, false, nullptr, probs, width_in, wa, ra, actq.col_rht);
      actq.amax = ra;
      actq.col_amax = ra + gt.num_groups;
    }
  }
  const int n_ct = (int)((wa + BLOCK_COLS - 1) / BLOCK_COLS);
  const dim3 grid((unsigned)((int64_t)(gt.num_panels / 4) * n_ct));
  float* part = dprobs ? static_cast<float*>(workspace) : nullptr;
  switch (act.kind) {
    case MGS_ACT_IDENTITY: bwd_dispatch_fmt<MGS_ACT_IDENTITY>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_SRELU: bwd_dispatch_fmt<MGS_ACT_SRELU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_TANH_SRELU: bwd_dispatch_fmt<MGS_ACT_TANH_SRELU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_SWIGLU: bwd_dispatch_fmt<MGS_ACT_SWIGLU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_GELU: bwd_dispatch_fmt<MGS_ACT_GELU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_SIGMOID: bwd_dispatch_fmt<MGS_ACT_SIGMOID>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    case MGS_ACT_GLU: bwd_dispatch_fmt<MGS_ACT_GLU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
    default: bwd_dispatch_fmt<MGS_ACT_CLAMPED_SWIGLU>(fmt, grid, st, aa, gt, x, dy, probs, width_in, wa, dx, dxq, part, cs_part, actq, n_ct); break;
  }
  launch_reduce(gt, part, n_ct, gt.total_rows > 0 ? dprobs : nullptr, cs_part, width_in, dx_col_sum, st);
  return hipGetLastError();
}

int64_t act_bwd_cs_offset(int64_t rows, int64_t wa) {
  const int64_t dp = 4 * rows * ((wa + BLOCK_COLS - 1) / BLOCK_COLS);
  return (dp + 255) & ~(int64_t)255;
}

int64_t col_sum_part_bytes(const GroupTable& gt, int64_t width) {
  return 4 * (int64_t)(gt.num_panels / 4) * width;
}

int64_t act_bwd_rht_offset(const GroupTable& gt, int64_t wa, int64_t width_in) {
  const int64_t o = act_bwd_cs_offset(gt.total_rows, wa) + col_sum_part_bytes(gt, width_in);
  return (o + 255) & ~(int64_t)255;
}

int64_t act_bwd_workspace_bytes(const GroupTable& gt, int64_t wa, int64_t width_in) {
  return act_bwd_rht_offset(gt, wa, width_in) + 8 * (int64_t)gt.num_groups;
}

namespace {

// Group table from device-resident split sizes (one workgroup): row offsets, padded columnwise panel
// offsets and their totals, for the calls of a captured graph whose routing changes between replays.
// A negative split or a sum above the capacity sets status 1 and leaves every group empty.
__global__ __launch_bounds__(256) void groups_update_kernel(int e, const int64_t* __restrict__ splits,
                                                            int64_t max_rows, GroupTable* __restrict__ out,
                                                            int32_t* __restrict__ status) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int g = threadIdx.x; g < e; g += blockDim.x)
    if (splits[g] < 0) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x != 0) return;
  int64_t rows = 0, panels = 0;
  if (!bad) {
    for (int g = 0; g < e; ++g) rows += splits[g];
    if (rows > max_rows) bad = 1;
  }
  rows = 0;
  for (int g = 0; g < e; ++g) {
    out->row_off[g] = (int32_t)rows;
    out->panel_off[g] = (int32_t)panels;
    const int64_t m = bad ? 0 : splits[g];
    rows += m;
    panels += (m + COL_ALIGN - 1) / COL_ALIGN * (COL_ALIGN / PANEL_ROWS);
  }
  out->row_off[e] = (int32_t)rows;
  out->panel_off[e] = (int32_t)panels;
  out->num_groups = e;
  out->num_panels = (int32_t)panels;
  out->total_rows = (int32_t)rows;
  out->dev = nullptr;
  if (status) *status = bad;
}

}  // namespace

hipError_t launch_groups_update(int num_groups, const int64_t* splits, int64_t max_rows, GroupTable* out,
                                int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(groups_update_kernel, dim3(1), dim3(256), 0, st, num_groups, splits, max_rows, out, status);
  return hipGetLastError();
}

hipError_t launch_col_sum(const GroupTable& gt, int64_t width, const uint16_t* x, float* out,
                          hipStream_t st) {
  const dim3 grid((unsigned)((width + CS_COLS - 1) / CS_COLS), (unsigned)gt.num_groups);
  if (gt.dev) hipLaunchKernelGGL(col_sum_kernel<true>, grid, dim3(256), 0, st, gt, width, x, out);
  else hipLaunchKernelGGL(col_sum_kernel<false>, grid, dim3(256), 0, st, gt, width, x, out);
  return hipGetLastError();
}

}  // namespace mgs
