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
constexpr int LDS_STRIDE16 = BK + 8;     // halfs per LDS row, FP16 tiles

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

// Operand layouts by mode (E groups, elements per byte 1 for MXFP8 and 2 for NVFP4):
//   FPROP / DGRAD A: rowwise qtensor [M x k]                 (scale matrix: all M rows)
//   FPROP B:         rowwise qtensor [E * n x k]             (scale matrix: all E * n rows)
//   DGRAD B:         columnwise qtensor of an [E * k x n] weight: per group [n x kp], kp = roundup(k, 128)
//   WGRAD A / B:     columnwise qtensors of widths m / n: per group [m x mp_g] / [n x mp_g]
template <int TM, int TN>
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
  const int ediv = nv ? 2 : 1;            // elements per byte
  const int sblk = nv ? 16 : 32;          // elements per scale
  const int ntn = (int)((ga.n + TN - 1) / TN);
  const int tm = lt / ntn, tn = lt - tm * ntn;
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
    j.a.srows = tt.tok_off[tt.num_groups];
    j.a.srow0 = arow0;
    j.a.sld = ga.k / sblk;
    if (ga.mode == MGS_GEMM_FPROP) {
      j.b.ld = ga.k / ediv;
      j.b.data = ga.b_data + ((int64_t)g * ga.n + brow0) * j.b.ld;
      j.b.sbase = ga.b_scales;
      j.b.srows = (int64_t)tt.num_groups * ga.n;
      j.b.srow0 = (int64_t)g * ga.n + brow0;
      j.b.sld = ga.k / sblk;
    } else {
      const int64_t kp = (ga.k + COL_ALIGN - 1) / COL_ALIGN * COL_ALIGN;
      j.b.ld = kp / ediv;
      j.b.data = ga.b_data + (int64_t)g * ga.n * j.b.ld + brow0 * j.b.ld;
      j.b.sbase = ga.b_scales + (int64_t)g * ga.n * kp / sblk;
      j.b.srows = ga.n;
      j.b.srow0 = brow0;
      j.b.sld = kp / sblk;
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

// Epilogue for one 16 x 16 fragment held as C[row][col0 .. col0 + 3] in each lane.
__device__ __forceinline__ void store_frag(const TileJob& j, const GemmArgs& ga, int row, int col,
                                           v4f acc) {
  if (row >= j.a.rows || col >= j.b.rows) return;  // b.rows is a multiple of 4 (N % 32 == 0)
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
    w.x = bf16x2(v[0], v[1]);
    w.y = bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(j.c16 + gr * j.ldc + gc) = w;
  }
}

template <int TM, int TN>
__device__ __forceinline__ void write_zero_tile(const TileJob& j, const GemmArgs& ga) {
  // empty group in WGRAD: dW_g = 0 (unchanged when accumulating)
  if (ga.accumulate) return;
  for (int idx = threadIdx.x; idx < TM * TN; idx += blockDim.x) {
    const int r = idx / TN, c = idx - (idx / TN) * TN;
    if (r >= j.a.rows || c >= j.b.rows) continue;
    const int64_t gr = j.crow0 + r, gc = j.ccol0 + c;
    if (j.c32) j.c32[gr * j.ldc + gc] = 0.0f;
    else j.c16[gr * j.ldc + gc] = 0;
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

// a pointer that is the same in every lane, moved to scalar registers
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int xcd_remap_gemm(int b, int n) {
  int q = n >> 3, r = n & 7;
  int x = b & 7, i = b >> 3;
  return x * q + min(x, r) + i;
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mxfp8_256_kernel(GemmArgs ga, GemmTable tt) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE_BYTES];
  const int tile = xcd_remap_gemm(blockIdx.x, gridDim.x);
  const TileJob j = make_job<BM2, BN2>(ga, tt, tile);
  if (j.k == 0) {
    write_zero_tile<BM2, BN2>(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
  const int nsteps = (int)((j.k + BK - 1) / BK);

  // direct-to-LDS loads of step `st` into stage buffer `stg`: wave w fills data rows 64w .. 64w + 63
  // of A and of B (8 instructions of 8 rows each per operand) and their scale bytes (4 instructions
  // of 16 rows x 4 blocks each per operand).  Addresses are a wave-uniform 64-bit base (SGPRs) plus
  // a 32-bit per-lane offset, computed once.
  const uint8_t* abase = uniform_ptr(j.a.data);
  const uint8_t* bbase = uniform_ptr(j.b.data);
  const uint8_t* asbase = uniform_ptr(j.a.sbase);
  const uint8_t* bsbase = uniform_ptr(j.b.sbase);
  const int lrow = lane >> 3, pchunk = lane & 7;
  uint32_t offa[8], offb[8], c16[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = wave * 64 + i * 8 + lrow;
    const int ra = row < j.a.rows ? row : j.a.rows - 1;
    const int rb = row < j.b.rows ? row : j.b.rows - 1;
    c16[i] = (uint32_t)((pchunk ^ (row & 7)) << 4);
    offa[i] = (uint32_t)(ra * j.a.ld);
    offb[i] = (uint32_t)(rb * j.b.ld);
  }
  // scale rows of this lane (one dword = the 4 block scales of a K step per row)
  const int srow = wave * 64 + lane;
  const uint32_t sra = (uint32_t)(j.a.srow0 + (srow < j.a.rows ? srow : j.a.rows - 1));
  const uint32_t srb = (uint32_t)(j.b.srow0 + (srow < j.b.rows ? srow : j.b.rows - 1));
  const uint32_t a_srows = (uint32_t)j.a.srows, b_srows = (uint32_t)j.b.srows;
  auto issue = [&](int st, uint8_t* stg) {
    const uint32_t k0 = (uint32_t)st * BK;
    uint8_t* sa = stg;
    uint8_t* sb = stg + BM2 * BK;
    uint8_t* ssa = stg + DATA_BYTES;
    uint8_t* ssb = ssa + BM2 * 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // tail chunks (at or past K) read chunk 0 of the step instead; they are zeroed in registers
      const uint32_t kk = k0 + ((int64_t)(k0 + c16[i]) < j.k ? c16[i] : 0u);
      __builtin_amdgcn_global_load_lds(abase + (offa[i] + kk), (lds_ptr_t)(sa + (wave * 8 + i) * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(bbase + (offb[i] + kk), (lds_ptr_t)(sb + (wave * 8 + i) * 1024), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(asbase + ((uint32_t)st * a_srows + sra) * 4u, (lds_ptr_t)(ssa + wave * 256), 4, 0, 0);
    __builtin_amdgcn_global_load_lds(bsbase + ((uint32_t)st * b_srows + srb) * 4u, (lds_ptr_t)(ssb + wave * 256), 4, 0, 0);
  };

  v4f acc[8][8];
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
#pragma unroll
    for (int fn = 0; fn < 8; ++fn) acc[fm][fn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // One K step from stage buffer `stg`: every fragment of the step is read from LDS first, then the
  // direct-to-LDS loads of the next step are issued into the other buffer (the compiler makes LDS
  // reads wait for all direct loads in flight, so they must not come after them), then the 64 MFMAs
  // run while those loads are in flight.  With `tail`, K chunks at or past `rem` are zeroed.
  auto step = [&](const uint8_t* stg, bool tail, int64_t rem, int next_st, uint8_t* next_stg) {
    const uint8_t* sa = stg;
    const uint8_t* sb = stg + BM2 * BK;
    const uint8_t* ssa = stg + DATA_BYTES;
    const uint8_t* ssb = ssa + BM2 * 4;
    const bool lo_ok = !tail || 16 * q < rem, hi_ok = !tail || 64 + 16 * q < rem;
    const uint32_t mlo = lo_ok ? 0xffffffffu : 0u, mhi = hi_ok ? 0xffffffffu : 0u;
    v8i bfr[8], afr[8];
    int csb[8], csa[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int row = wn * 128 + f * 16 + r16;
      const uint8_t* pr = sb + row * BK;
      const uint4 b0 = *reinterpret_cast<const uint4*>(pr + ((q ^ (row & 7)) << 4));
      const uint4 b1 = *reinterpret_cast<const uint4*>(pr + (((4 + q) ^ (row & 7)) << 4));
      bfr[f] = v8i{(int)(b0.x & mlo), (int)(b0.y & mlo), (int)(b0.z & mlo), (int)(b0.w & mlo),
                   (int)(b1.x & mhi), (int)(b1.y & mhi), (int)(b1.z & mhi), (int)(b1.w & mhi)};
      csb[f] = ssb[row * 4 + q];
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int row = wm * 128 + f * 16 + r16;
      const uint8_t* pr = sa + row * BK;
      const uint4 a0 = *reinterpret_cast<const uint4*>(pr + ((q ^ (row & 7)) << 4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(pr + (((4 + q) ^ (row & 7)) << 4));
      afr[f] = v8i{(int)(a0.x & mlo), (int)(a0.y & mlo), (int)(a0.z & mlo), (int)(a0.w & mlo),
                   (int)(a1.x & mhi), (int)(a1.y & mhi), (int)(a1.z & mhi), (int)(a1.w & mhi)};
      csa[f] = ssa[row * 4 + q];
    }
    if (next_st >= 0) issue(next_st, next_stg);
#pragma unroll
    for (int fm = 0; fm < 8; ++fm)
#pragma unroll
      for (int fn = 0; fn < 8; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[fn], afr[fm], acc[fm][fn], 0, 0, 0,
                                                                       csb[fn], 0, csa[fm]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int64_t last_rem = j.k - (int64_t)(nsteps - 1) * BK;
  const bool tail_step = last_rem < BK;
  const int full_steps = tail_step ? nsteps - 1 : nsteps;
  for (int st = 0; st < full_steps; ++st) {
    const int nx = st + 1 < nsteps ? st + 1 : -1;
    step(smem + (st & 1) * STAGE_BYTES, false, BK, nx, smem + ((st + 1) & 1) * STAGE_BYTES);
  }
  if (tail_step) step(smem + ((nsteps - 1) & 1) * STAGE_BYTES, true, last_rem, -1, nullptr);
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
#pragma unroll
    for (int fn = 0; fn < 8; ++fn)
      store_frag(j, ga, wm * 128 + fm * 16 + r16, wn * 128 + fn * 16 + 4 * q, acc[fm][fn]);
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
  const TileJob j = make_job<BM, BN>(ga, tt, blockIdx.x);
  if (j.k == 0) {
    write_zero_tile<BM, BN>(j, ga);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;
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
      const bool av = kok && row < j.a.rows, bv = kok && row < j.b.rows;
      ra[i] = av ? *reinterpret_cast<const uint2*>(j.a.data + row * j.a.ld + e0 / 2) : make_uint2(0, 0);
      rb[i] = bv ? *reinterpret_cast<const uint2*>(j.b.data + row * j.b.ld + e0 / 2) : make_uint2(0, 0);
      sa[i] = av ? j.a.sbase[(j.a.srow0 + row) * j.a.sld + e0 / 16] : 0u;
      sb[i] = bv ? j.b.sbase[(j.b.srow0 + row) * j.b.sld + e0 / 16] : 0u;
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

namespace {

// Tile table for one launch: tiles of group g are [tile_off[g], tile_off[g+1]), ordered row-tile
// major (column tiles fastest) so neighbouring tiles share their A rows.
GemmTable make_table(const GemmArgs& ga, const GroupTable& gt, int tm, int tn) {
  GemmTable tt;
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
  return tt;
}

}  // namespace

int64_t gemm_tile_count(const GemmArgs& ga, const GroupTable& gt) {
  const int t = ga.fmt == MGS_FMT_MXFP8 ? BM2 : BM;
  return make_table(ga, gt, t, t).total_tiles;
}

hipError_t launch_gemm(const GemmArgs& ga, const GroupTable& gt, hipStream_t st) {
  if (ga.fmt == MGS_FMT_MXFP8) {
    const GemmTable tt = make_table(ga, gt, BM2, BN2);
    if (tt.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_mxfp8_256_kernel, dim3((unsigned)tt.total_tiles), dim3(256), 0, st, ga, tt);
  } else {
    const GemmTable tt = make_table(ga, gt, BM, BN);
    if (tt.total_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_nvfp4_kernel, dim3((unsigned)tt.total_tiles), dim3(256), 0, st, ga, tt);
  }
  return hipGetLastError();
}

}  // namespace mgs
