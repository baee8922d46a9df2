// Grouped GEMM on block-quantized operands for gfx950: C_g = A_g . B_g^T, FP32 accumulation.
//
// The method (page "Activation + GroupedLinear Fusion for MOE", Greptile summary second bullet and
// sequence diagram): GroupedLinear runs its forward and backward GEMMs per expert group directly on
// the pre-quantized grouped tensor produced by the fused activation kernel.  Every mode is written
// as C_g = A_g . B_g^T with both operands K-contiguous:
//   FPROP / DGRAD: grouped over M (A rows of group g, B = weight g [N x K]);
//   WGRAD:         grouped over K (the group's padded tokens), C_g = dW_g.
//
// MXFP8 operands go straight into the gfx950 block-scaled MFMA (V_MFMA_SCALE_F32_16X16X128_F8F6F4):
// E4M3 codes with one E8M0 scale per 32 K values per row, which is exactly the MX operand format.
// Measured operand layout of that instruction for 8-bit elements (16 x 16 x 128): lane l holds row
// l % 16; its bytes 0..15 are K[16q, 16q + 16) and bytes 16..31 are K[64 + 16q, 64 + 16q + 16) with
// q = l / 16; the scale VGPR of lane l applies to K block q (K[32q, 32q + 32)) of row l % 16.
//
// NVFP4 operands (E2M1 with an E4M3 scale per 16) cannot use the E8M0-scaled MFMA: the product of
// an E2M1 value and an E4M3 scale needs up to 6 significant bits.  The packed codes and scales are
// staged in LDS as they are; each wave dequantizes its fragments exactly to FP16 in registers
// (e2m1 * s_b is exact in FP16) and multiplies them with V_MFMA_F32_32X32X16_F16; the two per-group
// FP32 factors are applied in the epilogue.
//
// Both formats use 256 x 256 tiles per workgroup (4 waves in 2 x 2, each 128 x 128 with 256 FP32
// accumulators per lane in AGPRs), K steps of 128 and double-buffered direct-to-LDS loads.  The MFMA
// is issued with B as its first operand so each lane's accumulator holds runs of 4 consecutive output
// columns of one row (one 16-byte FP32 / 8-byte BF16 store each).
#include <algorithm>
#include <type_traits>

#include "mgs_device.h"

namespace mgs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BK = 128;                  // K elements per step

// One operand of a tile: `rows` valid rows starting at `data` (row stride `ld` bytes).  Scales:
// MXFP8 keeps them grouped per 128-wide K step -- the byte of (row r, 32-block kb) of the scale
// matrix is at sbase[((kb / 4) * srows + srow0 + r) * 4 + kb % 4]; NVFP4 keeps them row-major with
// `sld` bytes per row starting at sbase + srow0 * sld.
struct Operand {
  const uint8_t* data;
  int64_t ld;
  const uint8_t* sbase;
  int64_t srows, srow0, sld;
  int rows;
  int64_t avail;   // bytes of the operand tensor from `data` to its end
  int64_t savail;  // bytes of the scale array from `sbase` to its end
};

struct TileJob {
  int g;
  Operand a, b;
  int64_t k;          // reduction length (elements)
  int64_t crow0, ccol0;
  float* c32;
  uint16_t* c16;
  int64_t ldc;
  float gfactor;
  const uint16_t* bias;  // bias row of the group (length N) or null
};

constexpr int TILE_BLOCK_N = 4;

// Operand layouts by mode (E groups, elements per byte 1 for MXFP8 and 2 for NVFP4):
//   FPROP / DGRAD A: rowwise qtensor [M x k]                 (scale matrix: all M rows)
//   FPROP B:         rowwise qtensor [E * n x k]             (scale matrix: all E * n rows)
//   DGRAD B:         columnwise qtensor of an [E * k x n] weight: per group [n x kp], kp = roundup(k, 128)
//   WGRAD A / B:     columnwise qtensors of widths m / n: per group [m x mp_g] / [n x mp_g]
template <int TM, int TN, typename Table>
__device__ __forceinline__ TileJob make_job(const GemmArgs& ga, const Table& tt, int tile) {
  int lo = 0, hi = tt.num_groups;  // tile_off[lo] <= tile < tile_off[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (tt.tile_off[mid] <= tile) lo = mid; else hi = mid;
  }
  TileJob j;
  const int g = lo;
  j.g = g;
  const int lt = tile - tt.tile_off[g];
  const bool nv = ga.fmt == MGS_FMT_NVFP4;
  const int ediv = nv ? 2 : 1;            // elements per byte
  const int sblk = nv ? 16 : 32;          // elements per scale
  // Tiles of a group run in column blocks of TILE_BLOCK_N tile columns, row-major inside a block:
  // the workgroups in flight on one XCD (dispatched together) then share each K slice of A with
  // TILE_BLOCK_N tiles and each K slice of B with all tile rows of the block, which keeps the slices
  // the XCD's L2 must hold small.
  const int ntn = (int)((ga.n + TN - 1) / TN);
  const int64_t mrows = ga.mode == MGS_GEMM_WGRAD ? ga.m : tt.tok_off[g + 1] - tt.tok_off[g];
  const int ntm = (int)((mrows + TM - 1) / TM);
  const int full = ntn / TILE_BLOCK_N;
  const int blk = lt / (ntm * TILE_BLOCK_N);
  int tm, tn;
  if (blk < full) {
    const int r = lt - blk * ntm * TILE_BLOCK_N;
    tm = r / TILE_BLOCK_N;
    tn = blk * TILE_BLOCK_N + (r - tm * TILE_BLOCK_N);
  } else {
    const int wl = ntn - full * TILE_BLOCK_N;  // width of the last, partial block
    const int r = lt - full * ntm * TILE_BLOCK_N;
    tm = r / wl;
    tn = full * TILE_BLOCK_N + (r - tm * wl);
  }
  const int64_t brow0 = (int64_t)tn * TN;
  int64_t arows_total;
  if (ga.mode == MGS_GEMM_WGRAD) {
    const int64_t coff = tt.tok_off[g];
    const int64_t mp = tt.tok_off[g + 1] - coff;
    const int64_t arow0 = (int64_t)tm * TM;
    j.k = mp;
    j.a.ld = j.b.ld = mp / ediv;
    j.a.data = ga.a_data + ga.m * coff / ediv + arow0 * j.a.ld;
    j.b.data = ga.b_data + ga.n * coff / ediv + brow0 * j.b.ld;
    j.a.sbase = ga.a_scales + ga.m * coff / sblk;
    j.b.sbase = ga.b_scales + ga.n * coff / sblk;
    j.a.srows = ga.m; j.a.srow0 = arow0;
    j.b.srows = ga.n; j.b.srow0 = brow0;
    j.a.sld = j.b.sld = mp / sblk;
    const int64_t tot = tt.tok_off[tt.num_groups];  // padded tokens of all groups
    j.a.avail = ga.m * tot / ediv - (ga.m * coff / ediv + arow0 * j.a.ld);
    j.b.avail = ga.n * tot / ediv - (ga.n * coff / ediv + brow0 * j.b.ld);
    j.a.savail = ga.m * tot / sblk - ga.m * coff / sblk;
    j.b.savail = ga.n * tot / sblk - ga.n * coff / sblk;
    arows_total = ga.m - arow0;
    j.crow0 = arow0;
    j.ldc = ga.n;
    const int64_t cbase = (int64_t)g * ga.m * ga.n;
    j.c32 = ga.c_f32 ? reinterpret_cast<float*>(ga.c) + cbase : nullptr;
    j.c16 = ga.c_f32 ? nullptr : reinterpret_cast<uint16_t*>(ga.c) + cbase;
    j.bias = nullptr;
  } else {
    const int64_t r0 = tt.tok_off[g];
    const int64_t mg = tt.tok_off[g + 1] - r0;
    const int64_t arow0 = r0 + (int64_t)tm * TM;
    j.k = ga.k;
    j.a.ld = ga.k / ediv;
    j.a.data = ga.a_data + arow0 * j.a.ld;
    j.a.sbase = ga.a_scales;
    j.a.srows = tt.layout_rows;   // the K-step grouped scales are strided for the layout's rows
    j.a.srow0 = arow0;
    j.a.sld = ga.k / sblk;
    const int64_t rows_all = tt.tok_off[tt.num_groups];
    const int64_t nks = (ga.k + BK - 1) / BK;  // K steps (rowwise MXFP8 scales: 4 bytes per row and step)
    j.a.avail = (rows_all - arow0) * j.a.ld;
    j.a.savail = nv ? rows_all * j.a.sld : 4 * (int64_t)tt.layout_rows * nks;
    if (ga.mode == MGS_GEMM_FPROP) {
      j.b.ld = ga.k / ediv;
      j.b.data = ga.b_data + ((int64_t)g * ga.n + brow0) * j.b.ld;
      j.b.sbase = ga.b_scales;
      j.b.srows = (int64_t)tt.num_groups * ga.n;
      j.b.srow0 = (int64_t)g * ga.n + brow0;
      j.b.sld = ga.k / sblk;
      j.b.avail = ((int64_t)tt.num_groups * ga.n - ((int64_t)g * ga.n + brow0)) * j.b.ld;
      j.b.savail = nv ? j.b.srows * j.b.sld : 4 * j.b.srows * nks;
    } else {
      const int64_t kp = (ga.k + COL_ALIGN - 1) / COL_ALIGN * COL_ALIGN;
      j.b.ld = kp / ediv;
      j.b.data = ga.b_data + (int64_t)g * ga.n * j.b.ld + brow0 * j.b.ld;
      j.b.sbase = ga.b_scales + (int64_t)g * ga.n * kp / sblk;
      j.b.srows = ga.n;
      j.b.srow0 = brow0;
      j.b.sld = kp / sblk;
      j.b.avail = ((int64_t)tt.num_groups * ga.n - ((int64_t)g * ga.n + brow0)) * j.b.ld;
      j.b.savail = ((int64_t)tt.num_groups - g) * ga.n * kp / sblk;
    }
    arows_total = mg - (int64_t)tm * TM;
    j.crow0 = arow0;
    j.ldc = ga.n;
    j.c32 = ga.c_f32 ? reinterpret_cast<float*>(ga.c) : nullptr;
    j.c16 = ga.c_f32 ? nullptr : reinterpret_cast<uint16_t*>(ga.c);
    j.bias = ga.bias ? ga.bias + (int64_t)g * ga.n : nullptr;
  }
  j.ccol0 = brow0;
  j.a.rows = (int)min<int64_t>(TM, arows_total);
  j.b.rows = (int)min<int64_t>(TN, ga.n - brow0);
  j.gfactor = nv ? ga.a_gscale[g] * ga.b_gscale[g] : 1.0f;
  return j;
}

// max over the lanes l, l ^ 16, l ^ 32, l ^ 48 of a non-negative value (its bits order like
// unsigned integers)
__device__ __forceinline__ float max_over_rows(float m) {
  U2 r = swap16(__float_as_uint(m), __float_as_uint(m));
  const uint32_t u = umax(r.x, r.y);
  r = swap32(u, u);
  return __uint_as_float(umax(r.x, r.y));
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
// 16-byte global store that keeps its data registers live through two wait states: a store wider
// than 8 bytes reads its data after it issues, and a VALU write to them in the next instruction
// changed what part of the wave stored (observed on gfx950).
__device__ __forceinline__ void st16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const v4u v = {a, b, c, d};
  *reinterpret_cast<v4u*>(p) = v;
  asm volatile("s_nop 1" :: "v"(v));
}

// Epilogue value of one 16 x 16 fragment held as C[row][col0 .. col0 + 3] in each lane: the group
// factor, then the bias (four BF16 values, already fetched).
__device__ __forceinline__ void frag_values(const TileJob& j, v4f acc, uint2 bw, float (&v)[4]) {
  v[0] = acc[0] * j.gfactor; v[1] = acc[1] * j.gfactor; v[2] = acc[2] * j.gfactor; v[3] = acc[3] * j.gfactor;
  if (j.bias) {
    v[0] += bf16lo(bw.x); v[1] += bf16hi(bw.x); v[2] += bf16lo(bw.y); v[3] += bf16hi(bw.y);
  }
}

__device__ __forceinline__ void store_values(const TileJob& j, int row, int col, const float (&v)[4]) {
  if (row >= j.a.rows || col >= j.b.rows) return;  // b.rows is a multiple of 4 (N % 32 == 0)
  const int64_t gr = j.crow0 + row, gc = j.ccol0 + col;
  if (j.c32) {
    st16(j.c32 + gr * j.ldc + gc, __float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
         __float_as_uint(v[3]));
  } else {
    uint2 w;
    w.x = bf16x2(v[0], v[1]);
    w.y = bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(j.c16 + gr * j.ldc + gc) = w;
  }
}

template <int TM, int TN>
__device__ __forceinline__ void write_zero_tile(const TileJob& j, const GemmArgs& ga) {
  // empty group in WGRAD: dW_g = 0 (unchanged when accumulating); four columns per store (the
  // tile's valid column count, like N, is a multiple of 32)
  if (ga.accumulate) return;
  for (int idx = threadIdx.x; idx < TM * (TN / 4); idx += blockDim.x) {
    const int r = idx / (TN / 4), c = 4 * (idx - r * (TN / 4));
    if (r >= j.a.rows || c >= j.b.rows) continue;
    const int64_t gr = j.crow0 + r, gc = j.ccol0 + c;
    if (j.c32) st16(j.c32 + gr * j.ldc + gc, 0u, 0u, 0u, 0u);
    else *reinterpret_cast<uint2*>(j.c16 + gr * j.ldc + gc) = make_uint2(0u, 0u);
  }
}

// ------------------------------------------------------------------------------------ MXFP8, large tile
//
// 256 x 256 output tile per workgroup (4 waves in 2 x 2, each 128 x 128 = 8 x 8 MFMA fragments, 256
// FP32 accumulators per lane held in AGPRs), K step 128.  Operands and their E8M0 scales go from
// global memory straight into LDS with the direct-to-LDS loads (no VGPR staging), double-buffered:
// the loads of step s + 1 are in flight while step s is multiplied (a scheduling barrier keeps the
// MFMAs ahead of the wait for those loads).  LDS data rows are 128 bytes; the 16-byte chunk c of row
// r is stored at chunk position c ^ (r & 7) so the 16 lanes reading one fragment column spread over
// all banks.  Scales are staged as [row][4] bytes per step.  Rows past the tile edge load a clamped
// in-range row (their outputs are not stored); K past the end of the reduction is zeroed in
// registers in a peeled last step.
constexpr int BM2 = 256, BN2 = 256;
constexpr int DATA_BYTES = (BM2 + BN2) * BK;           // 64 KiB of operand data per stage
constexpr int STAGE_BYTES = DATA_BYTES + (BM2 + BN2) * 4;  // + 2 KiB of scales

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer descriptor of `bytes` bytes at `p` (record count capped at 2^31 - 1; gfx9 descriptor
// word 3), as four scalar registers.  The arguments are wave-uniform (they derive from the tile
// index); the compiler cannot prove it for values read from the kernel's group tables, so they are
// moved to scalar registers explicitly.
typedef int sdesc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sdesc_t gemm_view(const uint8_t* p, int64_t bytes) {
  bytes = bytes < 0 ? 0 : (bytes > 0x7FFFFFFFll ? 0x7FFFFFFFll : bytes);
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return sdesc_t{(int)lo, (int)(hi & 0xffffu), n, 0x00020000};
}

// Direct-to-LDS buffer loads (16 or 4 bytes per lane) to LDS byte address `lds` + 16 (or 4) x lane.
// Issued as inline assembly: the compiler's LDS-alias tracking would otherwise make later reads of
// the other stage wait for these loads.  It therefore does not count them either; every wait for
// them is an explicit s_waitcnt in the kernel.
// The scalar operands are wave-uniform by construction; readfirstlane tells the compiler so (values
// derived from the group tables are not provably uniform to it).
__device__ __forceinline__ void dma16(const sdesc_t& d, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(d), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const sdesc_t& d, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(d), "s"(__builtin_amdgcn_readfirstlane(soff)),
                  "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ int xcd_remap_gemm(int b, int n) {
  int q = n >> 3, r = n & 7;
  int x = b & 7, i = b >> 3;
  return x * q + min(x, r) + i;
}

// The tile workgroup b takes under the table's schedule (see GemmTable); false: none.  Contiguous
// schedule: XCD b % 8 takes its eighth of the tile sequence; with device-resident split sizes the grid
// is sized for the capacity, so workgroups past the end of their XCD's eighth have no tile.
template <typename Table>
__device__ __forceinline__ bool schedule_tile(const Table& tt, int b, int* tile) {
  if (!tt.interleave) {
    const int n = tt.total_tiles, q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
    if (i >= q + (x < r ? 1 : 0)) return false;
    *tile = x * q + min(x, r) + i;
    return true;
  }
  const int s = b / tt.stride;
  if (s >= tt.num_groups) return false;
  const int g = tt.order[s];
  const int j = b - s * tt.stride;
  const int t = tt.tile_off[g + 1] - tt.tile_off[g];
  const int q = t >> 3, r = t & 7, x = j & 7, i = j >> 3;
  if (i >= q + (x < r ? 1 : 0)) return false;
  *tile = tt.tile_off[g] + x * q + min(x, r) + i;
  return true;
}

// Scaled FP8 MFMA with the accumulator pinned to AGPRs.  Written as inline assembly because the
// register allocator otherwise keeps part of the 256 accumulators of a wave in VGPRs and spills the
// fragments.  The compiler does not see these as MFMAs, so code around them supplies the wait states
// it would insert: mfma_valu_gap() after VALU writes of operands (the masking of a partial K step;
// the values are pinned ahead of it so the compiler cannot sink the masking past it), and
// mfma_drain() before anything reads the accumulators.  tests/test_mfma_hazard.py checks the
// built code for both kinds of hazard.
__device__ __forceinline__ void mfma_scale_fp8(v4f& acc, const v8i& b, const v8i& a, int sb, int sa) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc)
               : "v"(b), "v"(a), "v"(sb), "v"(sa));
}
__device__ __forceinline__ void mfma_valu_gap() { asm volatile("s_nop 7"); }
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
}

// FPROP epilogue with the scaled activation and MXFP8 rowwise quantization of its result (page
// "[PyTorch] Enable fused activation recompute for ScaledTanhSReLU", Description and review
// discussion: the fused forward activates FC1's output in the GEMM epilogue and quantizes it for FC2).
// Lane l = 16 q + r16 holds, for fragment row fm and fragment column fn, C[row][16 fn + 4 q .. + 3]
// (row = 16 fm + r16 within the wave's 128 rows).  Per row the lane evaluates y = act(x) * p with x the
// FP32 value or its BF16 rounding; a 32-column block b (fragment columns 2b, 2b + 1) of a row lies in
// the 4 lanes l, l ^ 16, l ^ 32, l ^ 48, 8 values each, so its maximum is two lane swaps.  The scale
// code, its reciprocal power of two and the saturating E4M3 convert are the helpers the fused
// activation kernels use, so the codes equal theirs on the same x bit for bit.  Stores are regrouped
// by lane swaps so every lane writes 16 contiguous bytes: for a block b the lane holds code dwords
// 4q and 16 + 4q (bytes of the block); a 16-swap leaves lane q the 8 bytes at {16, 0, 24, 8}[q], a
// 32-swap with block b + 1 then 16 bytes of block b + q / 2 at 16 (1 - q % 2).  The BF16 values of C
// are regrouped the same way by one 16-swap per block (16 bytes at 64 b + {32, 0, 48, 16}[q]).  The
// four scales of the wave's 128 columns (one K step of FC2's operand) go out as one dword per row.
template <int KIND>
__device__ __forceinline__ void epilogue_act(const TileJob& j, const GemmArgs& ga, v4f (&acc)[8][8],
                                             const uint2 (&bw)[8], int wm, int wn, int q, int r16) {
  const ActArgs aa{ga.act_kind, ga.act_s, ga.act_inv_s, ga.act_limit, ga.act_alpha, ga.act_beta};
  const int cw = wn * 128;                          // the wave's first column within the tile
  const int64_t col0 = j.ccol0 + cw;                // ... within C
  const int64_t srows = j.a.srows;                  // all M rows: the scale matrix's row count
  const bool wave_cols = cw < j.b.rows;             // the wave's columns reach into C
  const bool odd = q & 1;
  const int c16_off = 16 * (odd ? (q >> 1) : 2 + (q >> 1));   // BF16 bytes within a 64-byte block
#pragma unroll
  for (int fm = 0; fm < 8; ++fm) {
    const int row = wm * 128 + fm * 16 + r16;
    const bool rok = row < j.a.rows;
    const int64_t gr = j.crow0 + row;
    const float p = !rok ? 0.0f : ga.probs ? ga.probs[gr] : 1.0f;
    uint16_t* crow = j.c16 + gr * j.ldc + col0;
    uint8_t* arow = ga.act_data + gr * ga.n + col0;
    uint32_t sdw = 0;
    U2 pr[4];                                       // per block: the lane's 8 code bytes after the 16-swap
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool bok = cw + 32 * b < j.b.rows;      // n % 32 == 0: a block is all in or all out
      float y[8];
      uint2 w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int fn = 2 * b + h;
        float v[4];
        frag_values(j, acc[fm][fn], bw[fn], v);
        w[h].x = bf16x2(v[0], v[1]);
        w[h].y = bf16x2(v[2], v[3]);
        float x[4];
        if (ga.act_on_bf16) {
          x[0] = bf16lo(w[h].x); x[1] = bf16hi(w[h].x); x[2] = bf16lo(w[h].y); x[3] = bf16hi(w[h].y);
        } else {
          x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) y[4 * h + t] = bok ? act_unary<KIND>(x[t], aa) * p : 0.0f;
      }
      // C: 16 contiguous bytes of the block's 64 per lane
      const U2 cx = swap16(w[1].x, w[0].x), cy = swap16(w[1].y, w[0].y);
      if (rok && bok) st16(reinterpret_cast<uint8_t*>(crow) + 64 * b + c16_off, cx.x, cy.x, cx.y, cy.y);
      const Mx8 enc = mx_encode8(y, max_over_rows(absmax8(y)));
      pr[b] = swap16(enc.q.y, enc.q.x);
      sdw |= (bok ? enc.code : 0u) << (8 * b);
    }
    // codes: blocks (0, 1) and (2, 3); lane q writes 16 bytes of block b + q / 2
#pragma unroll
    for (int b = 0; b < 4; b += 2) {
      const U2 lo = swap32(pr[b].x, pr[b + 1].x), hi = swap32(pr[b].y, pr[b + 1].y);
      const int blk = b + (q >> 1);
      if (rok && cw + 32 * blk < j.b.rows)
        st16(arow + 32 * blk + (odd ? 0 : 16), lo.x, hi.x, lo.y, hi.y);
    }
    if (rok && wave_cols && q == 0)
      *reinterpret_cast<uint32_t*>(ga.act_scales + ((col0 / 128) * srows + gr) * 4) = sdw;
  }
}

// BF16 epilogue: per fragment row, one 16-swap per 32-column block regroups the lane's two 8-byte
// pieces (fragment columns 2b, 2b + 1) so it writes 16 contiguous bytes at 64 b + {32, 0, 48, 16}[q]:
// four 16-byte stores per row of fragments instead of eight 8-byte ones.
__device__ __forceinline__ void epilogue_bf16(const TileJob& j, v4f (&acc)[8][8], const uint2 (&bw)[8],
                                              int wm, int wn, int q, int r16) {
  const int cw = wn * 128;
  const int c16_off = 16 * ((q & 1) ? (q >> 1) : 2 + (q >> 1));
#pragma unroll
  for (int fm = 0; fm < 8; ++fm) {
    const int row = wm * 128 + fm * 16 + r16;
    const bool rok = row < j.a.rows;
    uint8_t* crow = reinterpret_cast<uint8_t*>(j.c16 + (j.crow0 + row) * j.ldc + j.ccol0 + cw);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint2 w[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[4];
        frag_values(j, acc[fm][2 * b + h], bw[2 * b + h], v);
        w[h].x = bf16x2(v[0], v[1]);
        w[h].y = bf16x2(v[2], v[3]);
      }
      const U2 cx = swap16(w[1].x, w[0].x), cy = swap16(w[1].y, w[0].y);
      if (rok && cw + 32 * b < j.b.rows) st16(crow + 64 * b + c16_off, cx.x, cy.x, cx.y, cy.y);
    }
  }
}

// Epilogue of the 256 x 256 kernel: group factor, bias (from LDS), optional FP32 accumulation, store.
__device__ __forceinline__ void epilogue_256(const TileJob& j, const GemmArgs& ga, v4f (&acc)[8][8],
                                             const uint2* bias_lds, int wm, int wn, int q, int r16) {
  // epilogue: bias from LDS; one straight-line variant per output kind, so that stores never wait
  // for each other
  uint2 bw[8];
#pragma unroll
  for (int fn = 0; fn < 8; ++fn)
    bw[fn] = j.bias ? bias_lds[(wn * 128 + fn * 16 + 4 * q) >> 2] : make_uint2(0, 0);
  // FP32 output (optionally accumulating): the eight C fragments of a fragment row are loaded together
  // before any of them is stored, one memory round trip per fragment row
  auto epilogue_f32 = [&](auto acc_tag) {
    constexpr bool ACC = decltype(acc_tag)::value;
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      const int row = wm * 128 + fm * 16 + r16;
      const bool rok = row < j.a.rows;
      const int64_t gr = j.crow0 + row;
      float4 old[8];
      if constexpr (ACC) {
#pragma unroll
        for (int fn = 0; fn < 8; ++fn) {
          const int col = wn * 128 + fn * 16 + 4 * q;
          old[fn] = rok && col < j.b.rows ? *reinterpret_cast<const float4*>(j.c32 + gr * j.ldc + j.ccol0 + col)
                                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
      }
      if constexpr (ACC) {
#pragma unroll
        for (int fn = 0; fn < 8; ++fn) {
          const int col = wn * 128 + fn * 16 + 4 * q;
          float v[4];
          frag_values(j, acc[fm][fn], bw[fn], v);
          v[0] += old[fn].x; v[1] += old[fn].y; v[2] += old[fn].z; v[3] += old[fn].w;
          if (rok && col < j.b.rows)
            st16(j.c32 + gr * j.ldc + j.ccol0 + col, __float_as_uint(v[0]), __float_as_uint(v[1]),
                 __float_as_uint(v[2]), __float_as_uint(v[3]));
        }
      } else {
        // fragment pair (2b, 2b + 1) = 32 columns = one 128-byte line per row: lanes r16 and r16 ^ 8
        // trade values so that the first store writes rows 0..7 of the 16-row block as whole lines
        // (lane r16 < 8: its own fragment-2b chunk; r16 >= 8: the chunk of fragment 2b + 1 of row
        // r16 - 8) and the second store rows 8..15
        const bool hi = r16 >= 8;
        const int rlo = wm * 128 + fm * 16 + (r16 & 7);
        const bool ok_a = rlo < j.a.rows, ok_b = rlo + 8 < j.a.rows;
        const int64_t ga_ = j.crow0 + rlo;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v0[4], v1[4], rv[4];
          frag_values(j, acc[fm][2 * b], bw[2 * b], v0);
          frag_values(j, acc[fm][2 * b + 1], bw[2 * b + 1], v1);
#pragma unroll
          for (int t = 0; t < 4; ++t) rv[t] = dpp_f<DPP_ROW_ROR8>(hi ? v0[t] : v1[t]);
          const int col = wn * 128 + 32 * b + (hi ? 16 : 0) + 4 * q;
          if (col < j.b.rows) {
            float* pa_ = j.c32 + ga_ * j.ldc + j.ccol0 + col;
            if (ok_a)
              st16(pa_, __float_as_uint(hi ? rv[0] : v0[0]), __float_as_uint(hi ? rv[1] : v0[1]),
                   __float_as_uint(hi ? rv[2] : v0[2]), __float_as_uint(hi ? rv[3] : v0[3]));
            if (ok_b)
              st16(pa_ + 8 * j.ldc, __float_as_uint(hi ? v1[0] : rv[0]), __float_as_uint(hi ? v1[1] : rv[1]),
                   __float_as_uint(hi ? v1[2] : rv[2]), __float_as_uint(hi ? v1[3] : rv[3]));
          }
        }
      }
    }
  };
  if (ga.act_enabled) {
    switch (ga.act_kind) {
      case MGS_ACT_SRELU: epilogue_act<MGS_ACT_SRELU>(j, ga, acc, bw, wm, wn, q, r16); break;
      case MGS_ACT_TANH_SRELU: epilogue_act<MGS_ACT_TANH_SRELU>(j, ga, acc, bw, wm, wn, q, r16); break;
      case MGS_ACT_GELU: epilogue_act<MGS_ACT_GELU>(j, ga, acc, bw, wm, wn, q, r16); break;
      case MGS_ACT_SIGMOID: epilogue_act<MGS_ACT_SIGMOID>(j, ga, acc, bw, wm, wn, q, r16); break;
      default: epilogue_act<MGS_ACT_IDENTITY>(j, ga, acc, bw, wm, wn, q, r16); break;
    }
  } else if (!j.c32) {
    epilogue_bf16(j, acc, bw, wm, wn, q, r16);
  } else if (!ga.accumulate) {
    epilogue_f32(std::false_type{});
  } else {
    epilogue_f32(std::true_type{});
  }
}

// Per-tile state of the direct-to-LDS loads: buffer descriptors of the operands, their scales and the
// bias, and the offsets that locate the tile's rows.  Lanes differ only in voa / vob.
struct TileDma {
  sdesc_t ad, bd, as, bs, bias;
  uint32_t voa, vob;      // lane offset of the lane's first data row (+ its chunk swizzle)
  uint32_t a_ld8, b_ld8;  // bytes between successive 8-row groups
  uint32_t a_s4, b_s4;    // bytes per K step of the scale arrays
  uint32_t a_sr, b_sr;    // scale byte offset of the tile's first row
  bool has_bias;
};

__device__ __forceinline__ TileDma tile_dma(const TileJob& j, int wave, int lane) {
  TileDma d;
  d.ad = gemm_view(j.a.data, j.a.avail);
  d.bd = gemm_view(j.b.data, j.b.avail);
  d.as = gemm_view(j.a.sbase, j.a.savail);
  d.bs = gemm_view(j.b.sbase, j.b.savail);
  const int lrow = lane >> 3, pchunk = lane & 7;
  const uint32_t lswz = (uint32_t)((pchunk ^ (lrow & 7)) << 4);
  d.voa = (uint32_t)((wave * 64 + lrow) * j.a.ld) + lswz;
  d.vob = (uint32_t)((wave * 64 + lrow) * j.b.ld) + lswz;
  d.a_ld8 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * j.a.ld));
  d.b_ld8 = __builtin_amdgcn_readfirstlane((uint32_t)(8 * j.b.ld));
  d.a_s4 = __builtin_amdgcn_readfirstlane((uint32_t)(j.a.srows * 4));
  d.b_s4 = __builtin_amdgcn_readfirstlane((uint32_t)(j.b.srows * 4));
  d.a_sr = __builtin_amdgcn_readfirstlane((uint32_t)(j.a.srow0 * 4));
  d.b_sr = __builtin_amdgcn_readfirstlane((uint32_t)(j.b.srow0 * 4));
  d.has_bias = j.bias != nullptr;
  d.bias = gemm_view(reinterpret_cast<const uint8_t*>(j.bias + j.ccol0), 2 * (int64_t)j.b.rows);
  return d;
}

// One workgroup per 256 x 256 output tile.  (A persistent variant that walks several tiles per
// workgroup and prefetches the next tile during the last K step measured slower: on this GPU one
// vector-memory counter covers loads and stores in issue order, so waiting for the next step's
// operands also waits for the previous tile's output stores.)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mxfp8_256_kernel(GemmArgs ga, GemmTable tt) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint2 bias_lds[BN2 / 4];
  int tile;
  TileJob j;
  if (tt.dev) {
    if (!schedule_tile(*tt.dev, blockIdx.x, &tile)) return;
    j = make_job<BM2, BN2>(ga, *tt.dev, tile);
  } else {
    if (!schedule_tile(tt, blockIdx.x, &tile)) return;
    j = make_job<BM2, BN2>(ga, tt, tile);
  }
  if (j.k == 0) {
    write_zero_tile<BM2, BN2>(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int swz_lo = (q ^ (r16 & 7)) << 4, swz_hi = ((4 + q) ^ (r16 & 7)) << 4;
  const uint32_t vs = (uint32_t)((wave * 64 + lane) * 4);  // scale dword of the lane's row
  const TileDma d = tile_dma(j, wave, lane);

  // direct-to-LDS loads of step `st` into stage buffer `stg`: wave w fills data rows 64w .. 64w + 63
  // of A and of B (8 instructions of 8 rows x 128 bytes each per operand) and their scale dwords
  // (one per row; the K-step scale dword of row r and step st sits at ((st * srows) + srow0 + r) * 4).
  // Each operand is read through a buffer descriptor based at the tile's first row whose record
  // count ends at the end of the operand tensor: rows past the tile edge read the following rows or
  // zeros (their outputs are not stored), and a partial last K step reads past the row end (those
  // chunks are zeroed in registers).  Rows 8 apart share the 16-byte chunk swizzle c ^ (row & 7).
  // Loads are issued one 1 KB instruction at a time: the wave cannot issue past a load the memory
  // pipeline has no room for, so a burst of them would stall the MFMAs behind it.
  // instruction n of step st: n < 8: B rows 8n of the wave's 64; 8 <= n < 16: A rows 8(n - 8)
  auto issue_one = [&](int st, uint8_t* stg, int n) {
    const uint32_t k0 = (uint32_t)st * BK;
    const uint32_t sa = lds_addr(stg) + wave * 8 * 1024;
    const uint32_t sb = sa + BM2 * BK;
    if (n < 8) dma16(d.bd, d.vob, n * d.b_ld8 + k0, sb + n * 1024);
    else dma16(d.ad, d.voa, (n - 8) * d.a_ld8 + k0, sa + (n - 8) * 1024);
  };
  auto issue_scales = [&](int st, uint8_t* stg) {
    const uint32_t ssa = lds_addr(stg) + DATA_BYTES + wave * 256;
    const uint32_t ssb = ssa + BM2 * 4;
    dma4(d.as, vs, (uint32_t)st * d.a_s4 + d.a_sr, ssa);
    dma4(d.bs, vs, (uint32_t)st * d.b_s4 + d.b_sr, ssb);
  };
  auto issue = [&](int st, uint8_t* stg) {
    for (int n = 0; n < 16; ++n) issue_one(st, stg, n);
    issue_scales(st, stg);
  };

  v4f acc[8][8];
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
#pragma unroll
    for (int fn = 0; fn < 8; ++fn) acc[fm][fn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  __builtin_amdgcn_sched_barrier(0);
  mfma_valu_gap();
  __builtin_amdgcn_sched_barrier(0);

  // One K step from stage buffer `stg` while the next step's loads go into the other buffer: four of
  // its load instructions before the fragment reads, the scales after the first MFMA and the other
  // twelve after every third MFMA, spread over the first 36 of the step's 64 (a pace the load pipeline
  // absorbs without stalling the wave; every second MFMA measured ~1% slower).
  // A fragment row 0 and the eight B fragments are read up front (the first MFMA waits only for the
  // first of them); A fragments then stream: the reads of fragment row fm + 1 are issued between the
  // first MFMAs of row fm, so most LDS reads overlap the matrix cores and 80 fragment registers are
  // live.  With `tail`, K chunks at or past `rem` are zeroed.
  constexpr int PRE_LOADS = 4, LOAD_PACE = 3;
  auto step = [&](const uint8_t* stg, bool tail, int64_t rem, int next_st, uint8_t* next_stg) {
    if (next_st >= 0)
      for (int n = 0; n < PRE_LOADS; ++n) issue_one(next_st, next_stg, n);
    const uint8_t* sa = stg;
    const uint8_t* sb = stg + BM2 * BK;
    const uint8_t* ssa = stg + DATA_BYTES;
    const uint8_t* ssb = ssa + BM2 * 4;
    const bool lo_ok = !tail || 16 * q < rem, hi_ok = !tail || 64 + 16 * q < rem;
    const uint32_t mlo = lo_ok ? 0xffffffffu : 0u, mhi = hi_ok ? 0xffffffffu : 0u;
    // fragment f of a wave's 128 rows starts at row (128 w + 16 f + r16); rows 16 f apart share the
    // chunk swizzle (r16 & 7), so the fragment index only moves the address by an immediate
    const uint8_t* pb = sb + (wn * 128 + r16) * BK;
    const uint8_t* pa = sa + (wm * 128 + r16) * BK;
    const uint8_t* psb = ssb + (wn * 128 + r16) * 4 + q;
    const uint8_t* psa = ssa + (wm * 128 + r16) * 4 + q;
    auto half = [&](const uint8_t* p, int f, int swz) {
      return *reinterpret_cast<const uint4*>(p + f * 16 * BK + swz);
    };
    auto join = [&](uint4 x0, uint4 x1) {
      return v8i{(int)(x0.x & mlo), (int)(x0.y & mlo), (int)(x0.z & mlo), (int)(x0.w & mlo),
                 (int)(x1.x & mhi), (int)(x1.y & mhi), (int)(x1.z & mhi), (int)(x1.w & mhi)};
    };
    // the step's first reads in the order the MFMAs of fragment row 0 use them, scales first (the
    // scheduling fences keep that order): each of those MFMAs then waits only for its own B fragment
    // instead of all eight
    int csn = psa[0];
    int csb[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) csb[f] = psb[f * 64];
    __builtin_amdgcn_sched_barrier(0);
    uint4 alo = half(pa, 0, swz_lo), ahi = half(pa, 0, swz_hi);
    v8i bfr[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      __builtin_amdgcn_sched_barrier(0);
      bfr[f] = join(half(pb, f, swz_lo), half(pb, f, swz_hi));
    }
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      v8i afr = join(alo, ahi);
      const int csa = csn;
      if (tail) {
        // the masked fragments are final before the wait states (the compiler would otherwise be
        // free to sink some of the masking past them, right up to the MFMA)
        asm volatile("" : "+v"(afr));
        if (fm == 0)
          for (int f = 0; f < 8; ++f) asm volatile("" : "+v"(bfr[f]));
        __builtin_amdgcn_sched_barrier(0);
        mfma_valu_gap();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int fn = 0; fn < 8; ++fn) {
        mfma_scale_fp8(acc[fm][fn], bfr[fn], afr, csb[fn], csa);
        if (next_st >= 0) {
          const int m = fm * 8 + fn;
          if (m == 0) issue_scales(next_st, next_stg);
          if (m % LOAD_PACE == LOAD_PACE - 1 && PRE_LOADS + m / LOAD_PACE < 16)
            issue_one(next_st, next_stg, PRE_LOADS + m / LOAD_PACE);
        }
        // the next A fragment row streams in behind the first three MFMAs of this row
        if (fm < 7) {
          if (fn == 0) alo = half(pa, fm + 1, swz_lo);
          if (fn == 1) ahi = half(pa, fm + 1, swz_hi);
          if (fn == 2) csn = psa[(fm + 1) * 64];
        }
      }
    }
    // the tile's last MFMAs are waited out here, on each path: the compiler may copy accumulators
    // out where the full-step loop and the partial last step join, before the drain after it
    if (next_st < 0) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_drain();
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(0, smem);
  // the tile's bias (BN2 BF16 values = 512 bytes) goes to LDS with the first step, by waves 0 and 1
  if (d.has_bias && wave < 2) dma4(d.bias, (uint32_t)(wave * 256 + lane * 4), 0, lds_addr(bias_lds) + wave * 256);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nsteps = __builtin_amdgcn_readfirstlane((int)((j.k + BK - 1) / BK));
  const int64_t last_rem = j.k - (int64_t)(nsteps - 1) * BK;
  const bool tail_step = last_rem < BK;
  const int full_steps = tail_step ? nsteps - 1 : nsteps;
  for (int st = 0; st < full_steps; ++st) {
    const int nx = st + 1 < nsteps ? st + 1 : -1;
    step(smem + (st & 1) * STAGE_BYTES, false, BK, nx, smem + ((st + 1) & 1) * STAGE_BYTES);
  }
  if (tail_step) step(smem + ((nsteps - 1) & 1) * STAGE_BYTES, true, last_rem, -1, nullptr);
  __builtin_amdgcn_sched_barrier(0);
  mfma_drain();
  __builtin_amdgcn_sched_barrier(0);
  epilogue_256(j, ga, acc, bias_lds, wm, wn, q, r16);
}

// ------------------------------------------------------------------------------------ NVFP4 path

// eight E2M1 codes (a dword, element 2i in the low nibble of byte i) times an exact FP16 block
// scale -> eight FP16 values.  V_CVT_SCALEF32_PK_F16_FP4 converts the two codes of one byte (low
// nibble first) to FP16, times the power of two of its FP32 scale operand (measured on the device:
// exact for all 256 bytes and every byte select); with scale 1 the values are the E2M1 values.  The
// product with the block scale is exact: at most 6 significant bits, magnitudes in [2^-10, 2688], all
// normal FP16 numbers.
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t w, v2h scale) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * scale;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * scale;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * scale;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * scale;
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// ------------------------------------------------------------------------------------ NVFP4, large tile
//
// 256 x 256 output tile per workgroup, 4 waves of 128 x 128 (4 x 4 fragments of 32 x 32, 256 FP32
// accumulators per lane in AGPRs), K step 128 elements.  The packed E2M1 codes (64 bytes per row and
// step) and the E4M3 block scales (8 bytes per row and step) go from global memory straight into LDS
// with direct-to-LDS loads, double-buffered (36 KiB per stage); each wave dequantizes its own
// fragments to FP16 in registers (exact, as in the staging path above) and feeds
// V_MFMA_F32_32X32X16_F16.  Fragment reads are 4x smaller than FP16 tiles in LDS would need.
//
// K order inside a step: the MFMA's K slots are a permutation of the step's 128 K indices, the same
// for both operands, so the dot products are unchanged.  Lane half h = l / 32 takes the contiguous
// K range [64 h, 64 h + 64) of the step, 8 elements per 16-wide MFMA (substep s: 64 h + 8 s .. + 7).
// A lane's codes for a whole step are then 32 contiguous bytes of its row (two 16-byte LDS reads)
// and its four block scales one dword.  Data rows are 64 bytes in LDS with the 16-byte chunk c of
// row r stored at slot c ^ ((r >> 1) & 3), so the 32 rows a fragment read touches fall on distinct
// banks; the direct-to-LDS loads realise the swizzle by loading the permuted chunk per lane.
// Scales: a row's 8 bytes of a step start at byte row * (K / 16) + 8 st, which is only 2-byte
// aligned when K % 64 != 0; each row therefore stages the 16 aligned bytes around them (one
// dwordx4 load per lane) and the reader extracts its dword at the row's byte misalignment (0 or 2).
constexpr int RSRC_WORD3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int NV_ROWB = BK / 2;                   // code bytes per row and step
constexpr int NV_DATA = BM2 * NV_ROWB;             // per operand and stage
constexpr int NV_SCB = BK / 16;                    // scale bytes per row and step
constexpr int NV_SCROW = 16;                       // staged scale bytes per row
constexpr int NV_SC = BM2 * NV_SCROW;
constexpr int NV_STAGE = 2 * (NV_DATA + NV_SC);    // A data, B data, A scales, B scales

typedef int v4i32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mfma_f16_32(v16f& acc, const uint4& b, const uint4& a) {
  const v4i32 vb = v4i32{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  const v4i32 va = v4i32{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(vb), "v"(va));
}

// E4M3 block scales (four bytes of a dword) as exact FP16 pairs: the code's bits shifted into an
// FP16 are its value times 2^-8 (the exponent bias differs by 8; E4M3 subnormals land on FP16
// subnormals consistently), so one multiplication by 256 makes them exact normal FP16 numbers.
__device__ __forceinline__ void nv_scales_f16(uint32_t w, v2h& s01, v2h& s23) {
  const uint32_t lo = ((w & 0x7fu) << 7) | ((w & 0x7f00u) << 15);
  const uint32_t hi = ((w >> 9) & 0x3f80u) | ((w >> 1) & 0x3f800000u);
  const v2h k256 = v2h{(_Float16)256.0f, (_Float16)256.0f};
  s01 = __builtin_bit_cast(v2h, lo) * k256;
  s23 = __builtin_bit_cast(v2h, hi) * k256;
}

__device__ __forceinline__ v2h scale_pair(const v2h& s01, const v2h& s23, int blk) {
  const _Float16 v = blk == 0 ? s01[0] : blk == 1 ? s01[1] : blk == 2 ? s23[0] : s23[1];
  return v2h{v, v};
}

// Epilogue of the NVFP4 256 x 256 tile: lane (r32, h32) of wave (wm, wn) holds, for fragment
// (fm, fn) and register group g, output row 128 wm + 32 fm + r32 and the four columns
// 128 wn + 32 fn + 8 g + 4 h32 .. + 3.
__device__ __forceinline__ void epilogue_nv256(const TileJob& j, const GemmArgs& ga, v16f (&acc)[4][4],
                                               const uint2* bias_lds, int wm, int wn, int r32, int h32) {
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    const int row = wm * 128 + fm * 32 + r32;
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * 128 + fn * 32 + 8 * g + 4 * h32;
        const uint2 bw = j.bias ? bias_lds[col >> 2] : make_uint2(0, 0);
        float v[4];
        frag_values(j, v4f{acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2], acc[fm][fn][4 * g + 3]},
                    bw, v);
        if (j.c32 && ga.accumulate && row < j.a.rows && col < j.b.rows) {
          const float4 o = *reinterpret_cast<const float4*>(j.c32 + (j.crow0 + row) * j.ldc + j.ccol0 + col);
          v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
        }
        store_values(j, row, col, v);
      }
    }
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_nvfp4_256_kernel(GemmArgs ga, GemmTable tt) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * NV_STAGE];
  __shared__ __attribute__((aligned(16))) uint2 bias_lds[BN2 / 4];
  int tile;
  TileJob j;
  if (tt.dev) {
    if (!schedule_tile(*tt.dev, blockIdx.x, &tile)) return;
    j = make_job<BM2, BN2>(ga, *tt.dev, tile);
  } else {
    if (!schedule_tile(tt, blockIdx.x, &tile)) return;
    j = make_job<BM2, BN2>(ga, tt, tile);
  }
  if (j.k == 0) {
    write_zero_tile<BM2, BN2>(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int r32 = lane & 31, h32 = lane >> 5;

  // load descriptors: data based at the tile's first row (record count to the end of the tensor),
  // scales at the tile's first scale row
  const sdesc_t ad = gemm_view(j.a.data, j.a.avail), bd = gemm_view(j.b.data, j.b.avail);
  // scale arrays viewed from their 4-aligned base; `sa0` / `sb0` is the array start's offset from it
  const int64_t sa0 = (int64_t)(reinterpret_cast<uintptr_t>(j.a.sbase) & 3u);
  const int64_t sb0 = (int64_t)(reinterpret_cast<uintptr_t>(j.b.sbase) & 3u);
  const sdesc_t as = gemm_view(j.a.sbase - sa0, j.a.savail + sa0), bs = gemm_view(j.b.sbase - sb0, j.b.savail + sb0);
  const sdesc_t biasd = gemm_view(reinterpret_cast<const uint8_t*>(j.bias + j.ccol0), 2 * (int64_t)j.b.rows);
  // data instruction n (0..3) of wave w: rows 64 w + 16 n + lane / 4, LDS slot lane % 4 holding chunk
  // (lane % 4) ^ ((row >> 1) & 3) = (lane % 4) ^ ((lane >> 3) & 3)
  const uint32_t dchunk = (uint32_t)(((lane & 3) ^ ((lane >> 3) & 3)) << 4);
  const uint32_t voa = (uint32_t)((wave * 64 + (lane >> 2)) * j.a.ld) + dchunk;
  const uint32_t vob = (uint32_t)((wave * 64 + (lane >> 2)) * j.b.ld) + dchunk;
  const uint32_t a16 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * j.a.ld));
  const uint32_t b16 = __builtin_amdgcn_readfirstlane((uint32_t)(16 * j.b.ld));
  // scale load of wave w: lane l stages the 16 aligned bytes around the step's 8 scale bytes of row
  // 64 w + l (the step offset 8 st keeps the alignment)
  const uint32_t vsa = (uint32_t)((sa0 + (j.a.srow0 + wave * 64 + lane) * j.a.sld) & ~(int64_t)3);
  const uint32_t vsb = (uint32_t)((sb0 + (j.b.srow0 + wave * 64 + lane) * j.b.sld) & ~(int64_t)3);

  // load instruction n (0..9) of step st into stage `stg`: 0..3 A data, 4..7 B data, 8 A scales,
  // 9 B scales
  constexpr int NLOADS = 10;
  auto issue_one = [&](int st, uint8_t* stg, int n) {
    const uint32_t base = lds_addr(stg);
    if (n < 4) {
      dma16(ad, voa, n * a16 + (uint32_t)st * NV_ROWB, base + (wave * 64 + 16 * n) * NV_ROWB);
    } else if (n < 8) {
      dma16(bd, vob, (n - 4) * b16 + (uint32_t)st * NV_ROWB, base + NV_DATA + (wave * 64 + 16 * (n - 4)) * NV_ROWB);
    } else if (n == 8) {
      dma16(as, vsa, (uint32_t)st * NV_SCB, base + 2 * NV_DATA + wave * 64 * NV_SCROW);
    } else {
      dma16(bs, vsb, (uint32_t)st * NV_SCB, base + 2 * NV_DATA + NV_SC + wave * 64 * NV_SCROW);
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = v16f{};
  __builtin_amdgcn_sched_barrier(0);
  mfma_valu_gap();
  __builtin_amdgcn_sched_barrier(0);

  // the lane's fragment rows: A 128 wm + 32 f + r32, B 128 wn + 32 f + r32 (f = 0..3)
  const int sw = (r32 >> 1) & 3;
  const uint32_t c0 = (uint32_t)(((2 * h32) ^ sw) << 4), c1 = (uint32_t)(((2 * h32 + 1) ^ sw) << 4);
  // byte misalignment (0 or 2) of the scale bytes of the lane's fragment rows
  uint32_t misa[4], misb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    misa[f] = (uint32_t)(sa0 + (j.a.srow0 + wm * 128 + f * 32 + r32) * j.a.sld) & 3u;
    misb[f] = (uint32_t)(sb0 + (j.b.srow0 + wn * 128 + f * 32 + r32) * j.b.sld) & 3u;
  }
  // the lane's scale dword (bytes 4 h .. 4 h + 3 of the row's step) from its staged 16 bytes
  auto scale_word = [&](const uint8_t* row16, uint32_t mis) {
    const uint4 d = *reinterpret_cast<const uint4*>(row16);
    const uint32_t lo = h32 ? d.y : d.x, hi = h32 ? d.z : d.y;
    return __builtin_amdgcn_alignbyte(hi, lo, mis);
  };
  // In a partial last step (K % 128 != 0) the scale array can end inside a dword, which a dword load
  // returns as zero; there the lane reads its bytes directly, two 2-byte loads each fully in or out
  // of the array (the bytes past it belong to K indices the step masks anyway).
  const __amdgpu_buffer_rsrc_t sra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(j.a.sbase), 0, (int)std::min<int64_t>(j.a.savail, 0x7fffffff), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t srb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(j.b.sbase), 0, (int)std::min<int64_t>(j.b.savail, 0x7fffffff), RSRC_WORD3);
  auto scale_word_direct = [&](const __amdgpu_buffer_rsrc_t& r, int64_t srow, int64_t sld, int st) {
    const uint32_t o = (uint32_t)(srow * sld) + (uint32_t)(st * NV_SCB + 4 * h32);
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, (int)(o + 2), 0, 0);
    return lo | (hi << 16);
  };
  // next step's loads: 2 before the fragment reads, then one after every third MFMA (issuing them
  // early measured best: one per 16 MFMAs was 5% slower, one per 8 about 2%, one per 4 0.7%, one per 2 1%)
  constexpr int PRE = 2, PACE = 3;
  auto step = [&](const uint8_t* stg, bool tail, int64_t rem, int next_st, uint8_t* next_stg, int st) {
    if (next_st >= 0)
      for (int n = 0; n < PRE; ++n) issue_one(next_st, next_stg, n);
    const uint8_t* pa = stg + (wm * 128 + r32) * NV_ROWB;
    const uint8_t* pb = stg + NV_DATA + (wn * 128 + r32) * NV_ROWB;
    const uint8_t* psa = stg + 2 * NV_DATA + (wm * 128 + r32) * NV_SCROW;
    const uint8_t* psb = stg + 2 * NV_DATA + NV_SC + (wn * 128 + r32) * NV_SCROW;
    // raw codes (8 dwords per fragment: dword s = substep s) and scales of the step
    uint32_t ra[4][8], rb[4][8];
    v2h sa01[4], sa23[4], sb01[4], sb23[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint4 x0 = *reinterpret_cast<const uint4*>(pa + f * 32 * NV_ROWB + c0);
      const uint4 x1 = *reinterpret_cast<const uint4*>(pa + f * 32 * NV_ROWB + c1);
      const uint4 y0 = *reinterpret_cast<const uint4*>(pb + f * 32 * NV_ROWB + c0);
      const uint4 y1 = *reinterpret_cast<const uint4*>(pb + f * 32 * NV_ROWB + c1);
      ra[f][0] = x0.x; ra[f][1] = x0.y; ra[f][2] = x0.z; ra[f][3] = x0.w;
      ra[f][4] = x1.x; ra[f][5] = x1.y; ra[f][6] = x1.z; ra[f][7] = x1.w;
      rb[f][0] = y0.x; rb[f][1] = y0.y; rb[f][2] = y0.z; rb[f][3] = y0.w;
      rb[f][4] = y1.x; rb[f][5] = y1.y; rb[f][6] = y1.z; rb[f][7] = y1.w;
      const uint32_t wa = tail ? scale_word_direct(sra, j.a.srow0 + wm * 128 + f * 32 + r32, j.a.sld, st)
                               : scale_word(psa + f * 32 * NV_SCROW, misa[f]);
      const uint32_t wb = tail ? scale_word_direct(srb, j.b.srow0 + wn * 128 + f * 32 + r32, j.b.sld, st)
                               : scale_word(psb + f * 32 * NV_SCROW, misb[f]);
      nv_scales_f16(wa, sa01[f], sa23[f]);
      nv_scales_f16(wb, sb01[f], sb23[f]);
    }
    // operands of substep s, zeroed where the K index is past the end (partial last step)
    auto dq = [&](const uint32_t (&r)[8], const v2h& s01, const v2h& s23, int sub) {
      uint4 v = fp4x8_to_f16(r[sub], scale_pair(s01, s23, sub >> 1));
      if (tail && !(64 * h32 + 8 * sub < rem)) v = make_uint4(0, 0, 0, 0);
      return v;
    };
    uint4 fa[2][4], fb[2][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      fa[0][f] = dq(ra[f], sa01[f], sa23[f], 0);
      fb[0][f] = dq(rb[f], sb01[f], sb23[f], 0);
      // computed here, ahead of the first substep's wait states (left free, the compiler sank part
      // of it to just before the fragment's first MFMA)
      asm volatile("" : "+v"(fa[0][f].x), "+v"(fa[0][f].y), "+v"(fa[0][f].z), "+v"(fa[0][f].w));
      asm volatile("" : "+v"(fb[0][f].x), "+v"(fb[0][f].y), "+v"(fb[0][f].z), "+v"(fb[0][f].w));
    }
#pragma unroll
    for (int sub = 0; sub < BK / 16; ++sub) {
      const int cur = sub & 1, nxt = cur ^ 1;
      __builtin_amdgcn_sched_barrier(0);
      mfma_valu_gap();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fm = 0; fm < 4; ++fm) {
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          mfma_f16_32(acc[fm][fn], fb[cur][fn], fa[cur][fm]);
          const int m = sub * 16 + fm * 4 + fn;
          // one fragment of the next substep is dequantized after every second MFMA
          // (the empty asm pins the result here: the compiler would otherwise sink the
          // dequantization to just before the next substep and serialize it with the MFMAs)
          if (sub + 1 < BK / 16 && (m & 1)) {
            const int f = (fm * 4 + fn) >> 1;  // 0..7
            uint4& dst = f < 4 ? fa[nxt][f] : fb[nxt][f - 4];
            dst = f < 4 ? dq(ra[f], sa01[f], sa23[f], sub + 1) : dq(rb[f - 4], sb01[f - 4], sb23[f - 4], sub + 1);
            asm volatile("" : "+v"(dst.x), "+v"(dst.y), "+v"(dst.z), "+v"(dst.w));
          }
          if (next_st >= 0 && m % PACE == PACE - 1 && PRE + m / PACE < NLOADS)
            issue_one(next_st, next_stg, PRE + m / PACE);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the tile's last MFMAs are waited out on each path (accumulator copies may follow the join)
    if (next_st < 0) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_drain();
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int n = 0; n < NLOADS; ++n) issue_one(0, smem, n);
  if (j.bias && wave < 2) dma4(biasd, (uint32_t)(wave * 256 + lane * 4), 0, lds_addr(bias_lds) + wave * 256);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nsteps = __builtin_amdgcn_readfirstlane((int)((j.k + BK - 1) / BK));
  const int64_t last_rem = j.k - (int64_t)(nsteps - 1) * BK;
  const bool tail_step = last_rem < BK;
  const int full_steps = tail_step ? nsteps - 1 : nsteps;
  for (int st = 0; st < full_steps; ++st) {
    const int nx = st + 1 < nsteps ? st + 1 : -1;
    step(smem + (st & 1) * NV_STAGE, false, BK, nx, smem + ((st + 1) & 1) * NV_STAGE, st);
  }
  if (tail_step) step(smem + ((nsteps - 1) & 1) * NV_STAGE, true, last_rem, -1, nullptr, nsteps - 1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_drain();
  __builtin_amdgcn_sched_barrier(0);
  epilogue_nv256(j, ga, acc, bias_lds, wm, wn, r32, h32);
}

}  // namespace

namespace {

// Schedule of a K-grouped (WGRAD) launch.  Every group has the same tiles but its own K, so a
// contiguous range of the tile sequence per XCD can leave one XCD with several times the mean work
// (a Zipf-skewed split puts a third of the tokens in one expert).  Cost of a tile in K steps, plus
// about four steps for the epilogue (one for an empty group's zero tile); when the heaviest XCD's
// contiguous range costs more than 5 % above the mean, the groups are dealt over all XCDs instead,
// largest K first, so each XCD holds an eighth of every group (greedy largest-first list scheduling
// over the XCDs' CUs, within about one tile of the ideal on such splits) while the tiles it has in
// flight still form a compact block of one group.
void schedule_k_grouped(GemmTable& tt) {
  const int e = tt.num_groups;
  int64_t cost[MGS_MAX_GROUPS];
  for (int g = 0; g < e; ++g) {
    const int64_t steps = (tt.tok_off[g + 1] - tt.tok_off[g] + BK - 1) / BK;
    cost[g] = steps ? steps + 4 : 1;
  }
  // the contiguous schedule: XCD x takes tiles [x q + min(x, r), (x + 1) q + min(x + 1, r))
  const int64_t n = tt.total_tiles, q = n / 8, r = n % 8;
  int64_t total = 0, worst = 0;
  for (int g = 0; g < e; ++g) total += cost[g] * (tt.tile_off[g + 1] - tt.tile_off[g]);
  for (int x = 0; x < 8; ++x) {
    const int64_t a = x * q + std::min<int64_t>(x, r), b = (x + 1) * q + std::min<int64_t>(x + 1, r);
    int64_t c = 0;
    for (int g = 0; g < e; ++g) {
      const int64_t lo = std::max<int64_t>(a, tt.tile_off[g]), hi = std::min<int64_t>(b, tt.tile_off[g + 1]);
      if (hi > lo) c += cost[g] * (hi - lo);
    }
    worst = std::max(worst, c);
  }
  if (e < 2 || 8 * worst * 100 <= total * 105) return;
  int order[MGS_MAX_GROUPS];
  for (int g = 0; g < e; ++g) order[g] = g;
  std::stable_sort(order, order + e, [&](int a, int b) { return cost[a] > cost[b]; });
  for (int s = 0; s < e; ++s) tt.order[s] = (uint8_t)order[s];
  // every group of a K-grouped launch has the same tile count
  tt.stride = (tt.tile_off[1] - tt.tile_off[0] + 7) / 8 * 8;
  tt.interleave = 1;
  tt.grid = tt.stride * e;
}

// Tile table for one launch: tiles of group g are [tile_off[g], tile_off[g+1]), ordered row-tile
// major (column tiles fastest) so neighbouring tiles share their A rows.
GemmTable make_table(const GemmArgs& ga, const GroupTable& gt, int tm, int tn) {
  GemmTable tt{};
  tt.num_groups = gt.num_groups;
  const int64_t ntn = (ga.n + tn - 1) / tn;
  int64_t tiles = 0;
  for (int g = 0; g < gt.num_groups; ++g) {
    tt.tile_off[g] = (int32_t)tiles;
    if (ga.mode == MGS_GEMM_WGRAD) {
      tt.tok_off[g] = PANEL_ROWS * gt.panel_off[g];
      tiles += ((ga.m + tm - 1) / tm) * ntn;
    } else {
      tt.tok_off[g] = gt.row_off[g];
      const int64_t mg = gt.row_off[g + 1] - gt.row_off[g];
      tiles += ((mg + tm - 1) / tm) * ntn;
    }
  }
  tt.tok_off[gt.num_groups] = ga.mode == MGS_GEMM_WGRAD ? PANEL_ROWS * gt.panel_off[gt.num_groups]
                                                         : gt.row_off[gt.num_groups];
  tt.tile_off[gt.num_groups] = (int32_t)tiles;
  tt.total_tiles = (int32_t)tiles;
  tt.interleave = 0;
  tt.grid = (int32_t)tiles;
  tt.layout_rows = gt.total_rows;
  if (ga.mode == MGS_GEMM_WGRAD) schedule_k_grouped(tt);
  return tt;
}

// Tiles of a grid sized for the row capacity (device-resident split sizes): M-grouped launches have
// at most ceil(capacity / TM) + E tile rows; K-grouped ones E groups of equal tiles, dealt in steps
// of 8 by the interleaved schedule; 8 more workgroups cover the per-XCD rounding of the contiguous one.
int64_t capacity_grid(const GemmArgs& ga, const GroupTable& gt, int tm, int tn) {
  const int64_t ntn = (ga.n + tn - 1) / tn;
  if (ga.mode == MGS_GEMM_WGRAD) return (int64_t)gt.num_groups * (((ga.m + tm - 1) / tm * ntn + 7) / 8 * 8) + 8;
  return (((int64_t)gt.total_rows + tm - 1) / tm + gt.num_groups) * ntn + 8;
}

// The tile table of one launch built on the device from the device group table `gd` (one
// workgroup): the same tables make_table and schedule_k_grouped build on the host.
__global__ __launch_bounds__(256) void gemm_table_kernel(const GroupTable* __restrict__ gd, int mode,
                                                         int64_t m, int64_t n, int tm, int tn,
                                                         int layout_rows, GemmTable* __restrict__ out) {
  __shared__ int64_t cost[MGS_MAX_GROUPS];
  __shared__ int interleave;
  const int e = gd->num_groups;
  const int64_t ntn = (n + tn - 1) / tn;
  if (threadIdx.x == 0) {
    int64_t tiles = 0;
    for (int g = 0; g < e; ++g) {
      out->tile_off[g] = (int32_t)tiles;
      if (mode == MGS_GEMM_WGRAD) {
        out->tok_off[g] = PANEL_ROWS * gd->panel_off[g];
        tiles += (m + tm - 1) / tm * ntn;
      } else {
        out->tok_off[g] = gd->row_off[g];
        tiles += (gd->row_off[g + 1] - gd->row_off[g] + tm - 1) / tm * ntn;
      }
    }
    out->tok_off[e] = mode == MGS_GEMM_WGRAD ? PANEL_ROWS * gd->panel_off[e] : gd->row_off[e];
    out->tile_off[e] = (int32_t)tiles;
    out->num_groups = e;
    out->total_tiles = (int32_t)tiles;
    out->grid = 0;
    out->stride = 0;
    out->layout_rows = layout_rows;
    out->dev = nullptr;
    interleave = 0;
    if (mode == MGS_GEMM_WGRAD && e > 1) {
      // the host's rule (schedule_k_grouped): deal the groups over the XCDs when the contiguous
      // ranges leave one XCD more than 5 % above the mean cost
      int64_t total = 0, worst = 0;
      for (int g = 0; g < e; ++g) {
        const int64_t steps = (PANEL_ROWS * (int64_t)(gd->panel_off[g + 1] - gd->panel_off[g]) + BK - 1) / BK;
        cost[g] = steps ? steps + 4 : 1;
        total += cost[g] * (out->tile_off[g + 1] - out->tile_off[g]);
      }
      const int64_t q = tiles / 8, r = tiles % 8;
      for (int x = 0; x < 8; ++x) {
        const int64_t a = x * q + (x < r ? x : r), b = (x + 1) * q + (x + 1 < r ? x + 1 : r);
        int64_t c = 0;
        for (int g = 0; g < e; ++g) {
          const int64_t lo = a > out->tile_off[g] ? a : out->tile_off[g];
          const int64_t hi = b < out->tile_off[g + 1] ? b : out->tile_off[g + 1];
          if (hi > lo) c += cost[g] * (hi - lo);
        }
        worst = c > worst ? c : worst;
      }
      interleave = 8 * worst * 100 > total * 105 ? 1 : 0;
    }
    out->interleave = interleave;
    if (interleave) out->stride = (int32_t)(((m + tm - 1) / tm * ntn + 7) / 8 * 8);
  }
  __syncthreads();
  if (!interleave) return;
  // largest cost first, ties in group order (a stable order): group g's rank among the groups
  for (int g = threadIdx.x; g < e; g += blockDim.x) {
    int rank = 0;
    for (int h = 0; h < e; ++h) rank += (cost[h] > cost[g] || (cost[h] == cost[g] && h < g)) ? 1 : 0;
    out->order[rank] = (uint8_t)g;
  }
}

}  // namespace

int64_t gemm_tile_count(const GemmArgs& ga, const GroupTable& gt) {
  if (gt.dev) return capacity_grid(ga, gt, BM2, BN2);
  return make_table(ga, gt, BM2, BN2).total_tiles;
}

hipError_t launch_gemm(const GemmArgs& ga, const GroupTable& gt, hipStream_t st, GemmTable* dev_gemm_table) {
  if (gt.dev) {
    // device-resident split sizes: the launch's table is built on the device first
    hipLaunchKernelGGL(gemm_table_kernel, dim3(1), dim3(256), 0, st, gt.dev, ga.mode, ga.m, ga.n, BM2, BN2,
                       gt.total_rows, dev_gemm_table);
    GemmTable tt{};
    tt.dev = dev_gemm_table;
    const int64_t grid = capacity_grid(ga, gt, BM2, BN2);
    if (ga.fmt == MGS_FMT_MXFP8)
      hipLaunchKernelGGL(gemm_mxfp8_256_kernel, dim3((unsigned)grid), dim3(256), 0, st, ga, tt);
    else
      hipLaunchKernelGGL(gemm_nvfp4_256_kernel, dim3((unsigned)grid), dim3(256), 0, st, ga, tt);
    return hipGetLastError();
  }
  if (ga.fmt == MGS_FMT_MXFP8) {
    const GemmTable tt = make_table(ga, gt, BM2, BN2);
    if (tt.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_mxfp8_256_kernel, dim3((unsigned)tt.grid), dim3(256), 0, st, ga, tt);
  } else {
    const GemmTable tt = make_table(ga, gt, BM2, BN2);
    if (tt.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_nvfp4_256_kernel, dim3((unsigned)tt.grid), dim3(256), 0, st, ga, tt);
  }
  return hipGetLastError();
}

}  // namespace mgs
