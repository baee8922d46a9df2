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
// an E2M1 value and an E4M3 scale needs up to 6 significant bits.  They are dequantized exactly to
// FP16 while staging into LDS (e2m1 * s_b is exact in FP16) and multiplied with the FP16 MFMA; the
// two per-group FP32 factors are applied in the epilogue.
//
// Tile: 128 x 128 per workgroup (4 waves in 2 x 2, each 64 x 64 = 4 x 4 MFMA fragments), K step 128.
// Global -> registers (prefetch of the next K step) -> LDS (rows padded to spread the banks) ->
// fragments.  The MFMA is issued with B as its first operand so each lane's accumulator holds 4
// consecutive output columns of one row (one 16-byte FP32 / 8-byte BF16 store per fragment).
#include "mgs_device.h"

namespace mgs {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_STRIDE8 = BK + 16;     // bytes per LDS row, FP8 tiles
constexpr int LDS_STRIDE16 = BK + 8;     // halfs per LDS row, FP16 tiles

struct TileJob {
  int g;
  const uint8_t* a;   // first row of the A tile (row stride lda bytes)
  const uint8_t* as;  // scales of that row (row stride K / block bytes)
  const uint8_t* b;
  const uint8_t* bs;
  int64_t lda, ldb;   // data bytes per row
  int64_t k;          // reduction length (elements)
  int arows, brows;   // valid rows of the A / B tile
  int64_t crow0, ccol0;
  float* c32;
  uint16_t* c16;
  int64_t ldc;
  float gfactor;
  const uint16_t* bias;  // bias row of the group (length N) or null
};

__device__ __forceinline__ TileJob make_job(const GemmArgs& ga, const GemmTable& tt, int tile) {
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
  const int sblk = nv ? 16 : 32;
  int64_t arows_total, brows_total;
  if (ga.mode == MGS_GEMM_WGRAD) {
    // A = columnwise copy of width m, B = columnwise copy of width n; K = padded tokens of group g
    const int64_t coff = tt.tok_off[g];
    const int64_t mp = tt.tok_off[g + 1] - coff;
    const int ntn = (int)((ga.n + BN - 1) / BN);
    const int tm = lt / ntn, tn = lt - tm * ntn;
    j.k = mp;
    j.lda = nv ? mp / 2 : mp;
    j.ldb = j.lda;
    const int64_t arow0 = (int64_t)tm * BM, brow0 = (int64_t)tn * BN;
    j.a = ga.a_data + (nv ? ga.m * coff / 2 : ga.m * coff) + arow0 * j.lda;
    j.as = ga.a_scales + ga.m * coff / sblk + arow0 * (mp / sblk);
    j.b = ga.b_data + (nv ? ga.n * coff / 2 : ga.n * coff) + brow0 * j.ldb;
    j.bs = ga.b_scales + ga.n * coff / sblk + brow0 * (mp / sblk);
    arows_total = ga.m - arow0;
    brows_total = ga.n - brow0;
    j.crow0 = arow0;
    j.ccol0 = brow0;
    j.ldc = ga.n;
    const int64_t cbase = (int64_t)g * ga.m * ga.n;
    j.c32 = ga.c_f32 ? reinterpret_cast<float*>(ga.c) + cbase : nullptr;
    j.c16 = ga.c_f32 ? nullptr : reinterpret_cast<uint16_t*>(ga.c) + cbase;
    j.bias = nullptr;
  } else {
    const int64_t r0 = tt.tok_off[g];
    const int64_t mg = tt.tok_off[g + 1] - r0;
    const int ntn = (int)((ga.n + BN - 1) / BN);
    const int tm = lt / ntn, tn = lt - tm * ntn;
    j.k = ga.k;
    j.lda = nv ? ga.k / 2 : ga.k;
    j.ldb = j.lda;
    const int64_t arow0 = r0 + (int64_t)tm * BM, brow0 = (int64_t)tn * BN;
    j.a = ga.a_data + arow0 * j.lda;
    j.as = ga.a_scales + arow0 * (ga.k / sblk);
    j.b = ga.b_data + (int64_t)g * ga.n * j.ldb + brow0 * j.ldb;
    j.bs = ga.b_scales + ((int64_t)g * ga.n + brow0) * (ga.k / sblk);
    arows_total = mg - (int64_t)tm * BM;
    brows_total = ga.n - brow0;
    j.crow0 = arow0;
    j.ccol0 = brow0;
    j.ldc = ga.n;
    j.c32 = ga.c_f32 ? reinterpret_cast<float*>(ga.c) : nullptr;
    j.c16 = ga.c_f32 ? nullptr : reinterpret_cast<uint16_t*>(ga.c);
    j.bias = ga.bias ? ga.bias + (int64_t)g * ga.n : nullptr;
  }
  j.arows = (int)min<int64_t>(BM, arows_total);
  j.brows = (int)min<int64_t>(BN, brows_total);
  j.gfactor = nv ? ga.a_gscale[g] * ga.b_gscale[g] : 1.0f;
  return j;
}

// Epilogue for one 16 x 16 fragment held as C[row][col0 .. col0 + 3] in each lane.
__device__ __forceinline__ void store_frag(const TileJob& j, const GemmArgs& ga, int row, int col,
                                           v4f acc) {
  if (row >= j.arows || col >= j.brows) return;  // brows is a multiple of 4 (N % 32 == 0)
  const int64_t gr = j.crow0 + row, gc = j.ccol0 + col;
  float v[4] = {acc[0] * j.gfactor, acc[1] * j.gfactor, acc[2] * j.gfactor, acc[3] * j.gfactor};
  if (j.bias) {
    const uint2 bw = *reinterpret_cast<const uint2*>(j.bias + j.ccol0 + col);
    v[0] += bf16lo(bw.x); v[1] += bf16hi(bw.x); v[2] += bf16lo(bw.y); v[3] += bf16hi(bw.y);
  }
  if (j.c32) {
    float4* p = reinterpret_cast<float4*>(j.c32 + gr * j.ldc + gc);
    if (ga.accumulate) {
      const float4 o = *p;
      v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
    }
    *p = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
    w.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
    *reinterpret_cast<uint2*>(j.c16 + gr * j.ldc + gc) = w;
  }
}

__device__ __forceinline__ void write_zero_tile(const TileJob& j, const GemmArgs& ga) {
  // empty group in WGRAD: dW_g = 0 (unchanged when accumulating)
  if (ga.accumulate) return;
  for (int idx = threadIdx.x; idx < BM * BN; idx += blockDim.x) {
    const int r = idx / BN, c = idx - (idx / BN) * BN;
    if (r >= j.arows || c >= j.brows) continue;
    const int64_t gr = j.crow0 + r, gc = j.ccol0 + c;
    if (j.c32) j.c32[gr * j.ldc + gc] = 0.0f;
    else j.c16[gr * j.ldc + gc] = 0;
  }
}

// ------------------------------------------------------------------------------------ MXFP8 path

__global__ __launch_bounds__(256) void gemm_mxfp8_kernel(GemmArgs ga, GemmTable tt) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * LDS_STRIDE8];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[BN * LDS_STRIDE8];
  const TileJob j = make_job(ga, tt, blockIdx.x);
  if (j.k == 0) {
    write_zero_tile(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t nkb = j.k >> 5;  // 32-blocks along K
  const int nsteps = (int)((j.k + BK - 1) / BK);

  // staging: thread loads rows (tid / 8) + 32 i, 16-byte chunk tid % 8 of the K step
  const int srow = tid >> 3, schunk = tid & 7;
  uint4 ra[4], rb[4];
  auto gload = [&](int step) {
    const int64_t kb = (int64_t)step * BK + schunk * 16;
    const bool kok = kb < j.k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 32 * i;
      ra[i] = (kok && row < j.arows) ? *reinterpret_cast<const uint4*>(j.a + row * j.lda + kb) : make_uint4(0, 0, 0, 0);
      rb[i] = (kok && row < j.brows) ? *reinterpret_cast<const uint4*>(j.b + row * j.ldb + kb) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 32 * i;
      *reinterpret_cast<uint4*>(lds_a + row * LDS_STRIDE8 + schunk * 16) = ra[i];
      *reinterpret_cast<uint4*>(lds_b + row * LDS_STRIDE8 + schunk * 16) = rb[i];
    }
  };
  // per-lane scales of the lane's fragment rows for one K step (K block = step * 4 + q)
  int sa[4], sb[4];
  auto sload = [&](int step) {
    const int64_t kb = (int64_t)step * 4 + q;
    const bool kok = kb < nkb;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int ar = wm * 64 + f * 16 + r16, br = wn * 64 + f * 16 + r16;
      sa[f] = (kok && ar < j.arows) ? j.as[ar * nkb + kb] : 127;
      sb[f] = (kok && br < j.brows) ? j.bs[br * nkb + kb] : 127;
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  gload(0);
  sload(0);
  lstore();
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    int csa[4], csb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) { csa[f] = sa[f]; csb[f] = sb[f]; }
    if (step + 1 < nsteps) {
      gload(step + 1);
      sload(step + 1);
    }
    v8i af[4], bfr[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint8_t* pa = lds_a + (wm * 64 + f * 16 + r16) * LDS_STRIDE8 + q * 16;
      const uint8_t* pb = lds_b + (wn * 64 + f * 16 + r16) * LDS_STRIDE8 + q * 16;
      const uint4 a0 = *reinterpret_cast<const uint4*>(pa), a1 = *reinterpret_cast<const uint4*>(pa + 64);
      const uint4 b0 = *reinterpret_cast<const uint4*>(pb), b1 = *reinterpret_cast<const uint4*>(pb + 64);
      af[f] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      bfr[f] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    }
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bfr[fn], af[fm], acc[fm][fn], 0, 0, 0, csb[fn], 0, csa[fm]);
    __syncthreads();
    if (step + 1 < nsteps) {
      lstore();
      __syncthreads();
    }
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
      store_frag(j, ga, wm * 64 + fm * 16 + r16, wn * 64 + fn * 16 + 4 * q, acc[fm][fn]);
}

// ------------------------------------------------------------------------------------ NVFP4 path

// eight E2M1 codes (a dword, element 2i in the low nibble of byte i) times an exact FP16 block
// scale -> eight FP16 values.  The E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} are FP16 numbers whose
// low byte is zero; their high bytes sit in a two-dword table indexed with V_PERM_B32 (byte selector
// 0..3 -> second operand, 4..7 -> first operand, 12 -> 0x00).  The sign (bit 3 of the nibble) is
// OR-ed into bit 7 of the high byte.  The product with the block scale is exact: at most 6
// significant bits, magnitudes in [2^-10, 2688], all normal FP16 numbers.
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t w, v2h scale) {
  constexpr uint32_t LUT_LO = 0x3E3C3800u;  // codes 0..3: 0, 0.5, 1, 1.5
  constexpr uint32_t LUT_HI = 0x46444240u;  // codes 4..7: 2, 3, 4, 6
  const uint32_t a = __builtin_amdgcn_perm(LUT_HI, LUT_LO, w & 0x07070707u) | ((w << 4) & 0x80808080u);
  const uint32_t b = __builtin_amdgcn_perm(LUT_HI, LUT_LO, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
  // element 2k = byte k of a, element 2k+1 = byte k of b, each as the high byte of an FP16
  uint32_t h[4];
  h[0] = __builtin_amdgcn_perm(b, a, 0x040C000Cu);
  h[1] = __builtin_amdgcn_perm(b, a, 0x050C010Cu);
  h[2] = __builtin_amdgcn_perm(b, a, 0x060C020Cu);
  h[3] = __builtin_amdgcn_perm(b, a, 0x070C030Cu);
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[0]) * scale);
  r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[1]) * scale);
  r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[2]) * scale);
  r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[3]) * scale);
  return r;
}

__global__ __launch_bounds__(256) void gemm_nvfp4_kernel(GemmArgs ga, GemmTable tt) {
  __shared__ __attribute__((aligned(16))) _Float16 lds_a[BM * LDS_STRIDE16];
  __shared__ __attribute__((aligned(16))) _Float16 lds_b[BN * LDS_STRIDE16];
  const TileJob j = make_job(ga, tt, blockIdx.x);
  if (j.k == 0) {
    write_zero_tile(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int64_t nsb = j.k >> 4;  // 16-blocks per row
  const int nsteps = (int)((j.k + BK - 1) / BK);

  // staging: a K step is 64 packed bytes per row; thread handles rows (tid / 8) + 32 i and the
  // 8-byte chunk tid % 8 (16 elements = one scale block)
  const int srow = tid >> 3, schunk = tid & 7;
  uint2 ra[4], rb[4];
  uint32_t sa[4], sb[4];
  auto gload = [&](int step) {
    const int64_t e0 = (int64_t)step * BK + schunk * 16;  // first element of the chunk
    const bool kok = e0 < j.k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 32 * i;
      const bool av = kok && row < j.arows, bv = kok && row < j.brows;
      ra[i] = av ? *reinterpret_cast<const uint2*>(j.a + row * j.lda + e0 / 2) : make_uint2(0, 0);
      rb[i] = bv ? *reinterpret_cast<const uint2*>(j.b + row * j.ldb + e0 / 2) : make_uint2(0, 0);
      sa[i] = av ? j.as[row * nsb + e0 / 16] : 0u;
      sb[i] = bv ? j.bs[row * nsb + e0 / 16] : 0u;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = srow + 32 * i;
      const _Float16 ha = (_Float16)e4m3_value(sa[i] & 0x7f), hb = (_Float16)e4m3_value(sb[i] & 0x7f);
      const v2h fa = v2h{ha, ha}, fb = v2h{hb, hb};
      const uint4 a0 = fp4x8_to_f16(ra[i].x, fa), a1 = fp4x8_to_f16(ra[i].y, fa);
      const uint4 b0 = fp4x8_to_f16(rb[i].x, fb), b1 = fp4x8_to_f16(rb[i].y, fb);
      uint4* pa = reinterpret_cast<uint4*>(lds_a + row * LDS_STRIDE16 + schunk * 16);
      uint4* pb = reinterpret_cast<uint4*>(lds_b + row * LDS_STRIDE16 + schunk * 16);
      pa[0] = a0; pa[1] = a1;
      pb[0] = b0; pb[1] = b1;
    }
  };

  v4f acc[4][4];
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) acc[fm][fn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  gload(0);
  lstore();
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    if (step + 1 < nsteps) gload(step + 1);
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      v8h af[4], bfr[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        af[f] = *reinterpret_cast<const v8h*>(lds_a + (wm * 64 + f * 16 + r16) * LDS_STRIDE16 + s * 32 + q * 8);
        bfr[f] = *reinterpret_cast<const v8h*>(lds_b + (wn * 64 + f * 16 + r16) * LDS_STRIDE16 + s * 32 + q * 8);
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfr[fn], af[fm], acc[fm][fn], 0, 0, 0);
    }
    __syncthreads();
    if (step + 1 < nsteps) {
      lstore();
      __syncthreads();
    }
  }
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
      store_frag(j, ga, wm * 64 + fm * 16 + r16, wn * 64 + fn * 16 + 4 * q, acc[fm][fn]);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& ga, const GemmTable& tt, hipStream_t st) {
  if (tt.total_tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tt.total_tiles);
  if (ga.fmt == MGS_FMT_MXFP8)
    hipLaunchKernelGGL(gemm_mxfp8_kernel, grid, dim3(256), 0, st, ga, tt);
  else
    hipLaunchKernelGGL(gemm_nvfp4_kernel, grid, dim3(256), 0, st, ga, tt);
  return hipGetLastError();
}

}  // namespace mgs
