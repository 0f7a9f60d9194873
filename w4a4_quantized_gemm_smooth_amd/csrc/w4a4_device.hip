// Device half of libw4a4 for gfx950 (CDNA4): the fused activation quantizer with the low-rank
// down projection, and the 4-bit GEMMs with the low-rank up projection in the epilogue; also the
// first pass of the 8-bit setting's activation side (partial row maxima; the rest of the W8A8 path
// is in w4a4_device_w8a8.hip), the MLP pair's GELU (in the activation kernel, or in fc1's GEMM
// epilogue together with fc2's whole activation side), and the MXFP4 GEMM on 128 x 128 blocks for
// small grids (larger MXFP4 grids run the MXFP4 mode of the INT8 GEMM in w4a4_device_w8a8.hip).
// The device-side C ABI entry points are at the end of this file.
//
// Method: SVDQuant summary page (arXiv 2411.05007v4) §4.2 (smoothing, low-rank branch,
// quantized residual), §4.3 / Fig. 6 (the down projection shares X̂ with the quantizer; the up
// projection is added to the 4-bit GEMM), §3 and App. D (INT4 qmax 7, per-group-64 symmetric
// quantization with 16-bit scales; FP4 E2M1 with qmax 6).
//
// MFMA use on gfx950:
//  * INT4 x INT4 products run on the scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with FP6
//    (E2M3) operands, which issues at twice the fp8 rate. A code q (|q| <= 7) is carried as the
//    E2M3 subnormal sign|00|mag, whose value is q / 8, so every product and every partial sum of
//    one 64-wide group is exact in fp32 (the result is Σ q_x q_w / 64, |Σ| <= 3136). One
//    32x32x64 MFMA is exactly one group. The codes stay 4 bits wide in memory: each 16-code run
//    is stored as its 96-bit FP6 image folded into 64 bits (the zero exponent bits of the outer
//    dwords hold the middle dword), and four AND/AND-OR ops per 16 codes unfold it for the MFMA.
//  * The per-group scale product s_x[m,g] * s_w[n,g] of a 32x32 tile is produced as an exact
//    outer product by one bf16 MFMA (v_mfma_f32_32x32x8_bf16 with one non-zero k), so the
//    group epilogue costs one fp32 FMA per output element.
//  * FP4 (E2M1) codes with E8M0 block scales run on the same scaled MFMA with the block scales
//    applied by the hardware.
//  * The low-rank branch uses the bf16 MFMAs (16x16x32 for the down projection, 32x32x16 for the
//    up projection, accumulating straight into the GEMM accumulators).

#include "w4a4_device_common.h"

using namespace w4a4;
using namespace w4a4::dev;

namespace {

// Folded FP6 layout of INT4 codes. A run of 16 codes c_0..c_15 has the FP6 image
// I = Σ_f (sign_f << 5 | |c_f|) << 6f (96 bits, dwords o0 o1 o2). Bits 3 and 4 of every 6-bit field
// (the exponent) are zero, which frees exactly the bit positions of the middle dword: stored are
// lo = (o0 & C0) | (o1 & C34) and hi = (o1 & C05) | (o2 & C2), with masks over p = bit % 6:
// C0 = {0,1,2,5}, C34 = {3,4}, C05 = {0,5}, C2 = {1,2,3,4}.
constexpr uint32_t FOLD_C0 = 0xE79E79E7u, FOLD_C34 = 0x18618618u, FOLD_C05 = 0x61861861u, FOLD_C2 = 0x9E79E79Eu;

__device__ __forceinline__ uint2 fold_fp6(uint32_t o0, uint32_t o1, uint32_t o2) {
  return make_uint2((o0 & FOLD_C0) | (o1 & FOLD_C34), (o1 & FOLD_C05) | (o2 & FOLD_C2));
}

// 16 B of folded codes (32 codes of one row, one half of a group) -> the 6-dword FP6 operand
__device__ __forceinline__ v8i unfold_fp6(v4i d) {
  return v8i{d[0] & (int)FOLD_C0, (d[0] & (int)FOLD_C34) | (d[1] & (int)FOLD_C05), d[1] & (int)FOLD_C2,
             d[2] & (int)FOLD_C0, (d[2] & (int)FOLD_C34) | (d[3] & (int)FOLD_C05), d[3] & (int)FOLD_C2, 0, 0};
}

// GELU(y) = (y/2)·(1 + erf(y/√2)) in fp32, erf from Abramowitz & Stegun 7.1.28
// (1 − (1 + a1 x + … + a6 x⁶)^−16, |error| ≤ 3e−7), one IEEE operation at a time (this file is built
// with -ffp-contract=off; the division is correctly rounded), so the bf16 rounding of the result
// is reproducible by any host that takes the same steps. Constants are the fp32 roundings of the
// published coefficients and of 1/√2.
__device__ __forceinline__ float gelu32(float y) {
  const float u = y * 0x1.6a09e6p-1f;
  const float ax = fabsf(u);
  float p = 0x1.693ecep-15f;  // a6
  p = p * ax + 0x1.220072p-12f;
  p = p * ax + 0x1.3ecc0ep-13f;
  p = p * ax + 0x1.2fc6d2p-7f;
  p = p * ax + 0x1.5a5fcep-5f;
  p = p * ax + 0x1.20dccep-4f;  // a1
  p = p * ax + 1.0f;
  p = p * p;
  p = p * p;
  p = p * p;
  p = p * p;
  float e = 1.0f - 1.0f / p;
  e = u < 0.f ? -e : e;
  return (0.5f * y) * (1.0f + e);
}

// INT4 codes of one group row held by four lanes (lane bits 4-5 = kc, 16 values each): s =
// bf16(max|X̂| / 7) (0 below 2^-126), q = rint(X̂ · (1/s)) (|q| <= 7 by the symmetric scale). The fp32
// product is formed as in the method, and v_cvt_scalef32_2xpk16_fp6_f32 rounds y / 8 to
// nearest-even on the E2M3 subnormal grid (step 1/8), i.e. emits exactly the carrier field
// sign|00|rint(y). Its two sources interleave (field 2e = src0[e], field 2e+1 = src1[e]); fields
// 16..31 are unused. Returns the lane's 16 codes folded into 8 bytes and the scale's bf16 bits.
__device__ __forceinline__ uint2 quant_int4_lane(const float (&xh)[2][8], uint32_t& s_bits) {
  float amax = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xh[h][e]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  float s = bf16f(bf16_rne(amax / 7.0f));
  if (!(s >= 0x1p-126f)) s = 0.f;
  const float inv = s != 0.f ? 1.0f / s : 0.f;
  v16f ev, od;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ev[e] = xh[e >> 2][2 * (e & 3)] * inv;
    od[e] = xh[e >> 2][2 * (e & 3) + 1] * inv;
    ev[8 + e] = 0.f;
    od[8 + e] = 0.f;
  }
  const v6i img = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
  s_bits = bf16_rne(s);
  return fold_fp6((uint32_t)img[0], (uint32_t)img[1], (uint32_t)img[2]);
}

// ===================================================================================
// Kernel 1: activation side. Per row and group: X̂ = fp32(x * inv_lambda); codes + scales (W8A8:
// the row's running max|X̂| instead, written per slice for the second W8A8 pass);
// t += bf16(X̂) · L1 (MFMA). One block = 128 rows (8 waves of 16) x one slice of at most
// QA_MAX_GS groups: every wave issues the X loads of all its groups at once, and the slice's
// 1/λ and L1 rows are copied into LDS by the LDS DMA path, shared by the 8 row tiles. With
// several slices the partial t of a slice goes to its own scratch plane; t_reduce_kernel sums
// the planes in slice order.
// ===================================================================================
constexpr int QA_WAVES = QA_BLOCK_ROWS / 16;


// LDS bytes of one block: 1/λ (16 B slots), L1 rows of RP rank columns padded by one slot, in
// whole 64-slot DMA instructions
constexpr int qa_lds_slots(int rp, int gs) { return (gs * 16 + rp * (gs * 8 + 1) + 63) / 64 * 64; }

// GELU_IN: the input is a producer's bf16 output Y and the layer's activations are
// X = bf16(GELU(Y)) (the MLP's fc2; INT4 only)
template <int FMT, int NT, bool GELU_IN = false>  // NT = rank_pad / 16 (0 when there is no low-rank branch)
__global__ __launch_bounds__(QA_WAVES * 64, NT <= 2 ? 4 : 2) void quantize_act_kernel(
    // X is not restrict: its loads must stay ahead of the counted wait below
    const uint16_t* X, int M, int K, int ldx, const float* __restrict__ inv_lambda,
    const uint16_t* __restrict__ l1t, int m_pad, int gs, uint8_t* __restrict__ xq, void* __restrict__ xscale,
    float* __restrict__ xl1) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int RP = NT * 16;
  const int G = K / W4A4_GROUP;
  const int nsl = (G + gs - 1) / gs;
  const int rb = blockIdx.x / nsl, sl = blockIdx.x % nsl;
  const int g0 = sl * gs, ng = min(gs, G - g0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // lane (r, kc) owns row r of the wave's tile and the 16 consecutive values 16 kc .. 16 kc + 15
  // of each group
  const int r = lane & 15, kc = lane >> 4;
  const int row = rb * QA_BLOCK_ROWS + wave * 16 + r;
  const bool valid = row < M;

  // ---- 1. 1/λ and L1 rows of the slice -> LDS. Slot s (16 B) of the block's LDS: s < 16 ng are
  // 1/λ; then rank row c uses slots [16 ng + c (8 ng + 1), +8 ng + 1) for k = 64 g0 .. 64 (g0 + ng),
  // the last one padding. Each DMA instruction fills 64 consecutive slots.
  const int n_il = ng * 16, l1_row = ng * 8 + 1, n_all = n_il + RP * l1_row;
  for (int s0 = wave * 64; s0 < n_all; s0 += QA_WAVES * 64) {
    const int s = s0 + lane;
    const void* src = inv_lambda + (size_t)g0 * W4A4_GROUP + 4 * min(s, n_il - 1);
    if (NT > 0 && s >= n_il && s < n_all) {
      const int c = (s - n_il) / l1_row, j = (s - n_il) % l1_row;
      src = l1t + (size_t)c * K + (size_t)g0 * W4A4_GROUP + 8 * (j < ng * 8 ? j : 0);
    }
    __builtin_amdgcn_global_load_lds(src, smem + 16 * s0, 16, 0, 0);
  }

  // ---- 2. X of every group of the slice, straight into registers: exactly 2 * QA_MAX_GS loads
  // per wave after the DMA, unconditional (rows past M read row M-1 and are zeroed at use, groups
  // past the slice reload its last group), so vmcnt(2 QA_MAX_GS) means the DMA has landed while
  // the X loads may still be in flight
  const uint16_t* xrow = X + (size_t)min(row, M - 1) * ldx + (size_t)g0 * W4A4_GROUP + kc * 16;
  uint4 xv[QA_MAX_GS][2];
#pragma unroll
  for (int i = 0; i < QA_MAX_GS; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) xv[i][h] = *reinterpret_cast<const uint4*>(xrow + min(i, ng - 1) * W4A4_GROUP + 8 * h);
  asm volatile("" ::: "memory");  // the loads stay ahead of the wait that counts them
  wait_vmcnt<2 * QA_MAX_GS>();
  __builtin_amdgcn_s_barrier();
  const float* s_il = reinterpret_cast<const float*>(smem);
  const uint8_t* s_l1 = smem + 16 * n_il;
  const int l1_stride = 16 * l1_row;

  constexpr int NTA = NT > 0 ? NT : 1;
  float row_amax = 0.f;  // W8A8: running max|X̂| of the lane's values
  v4f acc[NTA];
#pragma unroll
  for (int c = 0; c < NTA; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int i = 0; i < QA_MAX_GS; ++i) {
    if (i >= ng) break;  // block-uniform
    const int g = g0 + i;
    const float* il = s_il + i * W4A4_GROUP + kc * 16;
    float xh[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float4 i0 = *reinterpret_cast<const float4*>(il + 8 * h);
      const float4 i1 = *reinterpret_cast<const float4*>(il + 8 * h + 4);
      const uint32_t xw[4] = {valid ? xv[i][h].x : 0u, valid ? xv[i][h].y : 0u, valid ? xv[i][h].z : 0u,
                              valid ? xv[i][h].w : 0u};
      const float ilv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t bits = (e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xFFFFu);
        if (GELU_IN) bits = bf16_rne(gelu32(bf16f(bits)));
        xh[h][e] = bf16f(bits) * ilv[e];  // one fp32 multiply (no contraction: nothing to fuse)
      }
    }
    uint2* qdst = reinterpret_cast<uint2*>(xq + ((size_t)g * m_pad + row) * 32 + kc * 8);
    if constexpr (FMT == W4A4_FMT_W8A8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) row_amax = fmaxf(row_amax, fabsf(xh[h][e]));
    } else if constexpr (FMT == W4A4_FMT_INT4_G64) {
      uint32_t sb;
      *qdst = quant_int4_lane(xh, sb);
      if (kc == 0) static_cast<uint16_t*>(xscale)[(size_t)g * m_pad + row] = (uint16_t)sb;
    } else {
      // the lane's 16 values lie in 32-block kc / 2, shared with lane kc ^ 1
      float amax = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(xh[h][e]));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      int e8;
      if (amax == 0.f) {
        e8 = -127;
      } else {
        int ex;
        const float mant = frexpf(amax, &ex);  // amax = mant * 2^ex, mant in [0.5, 1)
        e8 = mant <= 0.75f ? ex - 3 : ex - 2;
        e8 = max(-127, min(127, e8));
      }
      // E2M1 nearest-even of X̂ * 2^-e (exact scaling), sign kept for values that round to
      // zero: v_cvt_scalef32_pk_fp4_f32 with scale 1 puts codes k, k+1 into byte k/2
      uint32_t word[2] = {0u, 0u};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = ldexpf(xh[h][e], -e8);
        word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[0], z[1], 1.0f, 0);
        word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[2], z[3], 1.0f, 1);
        word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[4], z[5], 1.0f, 2);
        word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[6], z[7], 1.0f, 3);
      }
      *qdst = make_uint2(word[0], word[1]);
      if ((kc & 1) == 0)
        static_cast<uint8_t*>(xscale)[(size_t)(2 * g + (kc >> 1)) * m_pad + row] = (uint8_t)(e8 + 127);
    }
    if (NT > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4i a;
#pragma unroll
        for (int d = 0; d < 4; ++d) a[d] = (int)pack_bf16x2(xh[h][2 * d], xh[h][2 * d + 1]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const v4i b = *reinterpret_cast<const v4i*>(s_l1 + (c * 16 + r) * l1_stride + i * 128 + kc * 32 + 16 * h);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc[c], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (FMT == W4A4_FMT_W8A8) {
    // the row's maximum over this slice -> plane sl of the partial maxima behind the scales
    row_amax = fmaxf(row_amax, __shfl_xor(row_amax, 16));
    row_amax = fmaxf(row_amax, __shfl_xor(row_amax, 32));
    if (kc == 0) static_cast<float*>(xscale)[(size_t)m_pad * (1 + sl) + row] = row_amax;
  }
  if (NT > 0) {
    // 16x16 MFMA output: lane holds rank column c*16 + lane%16, rows 4*(lane/16) + v of the tile
    const size_t n = (size_t)m_pad * RP;
    float* dst = xl1 + (nsl > 1 ? n * (1 + sl) : 0) + ((size_t)rb * QA_BLOCK_ROWS + wave * 16) * RP;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * kc + v) * RP + c * 16 + r] = acc[c][v];
  }
}

// t = Σ_slices partial t, summed in slice order (deterministic); n = m_pad * rank_pad floats.
// One float4 per thread; the loads of four planes are issued together.
__global__ __launch_bounds__(256) void t_reduce_kernel(const float* __restrict__ part, int nsl, int n,
                                                       float* __restrict__ t) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= n) return;
  auto ld = [&](int k) { return *reinterpret_cast<const float4*>(part + (size_t)k * n + i); };
  auto add = [](float4& s, const float4& v) {
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  };
  float4 s = ld(0);
  int k = 1;
  for (; k + 3 < nsl; k += 4) {
    const float4 a = ld(k), b = ld(k + 1), c = ld(k + 2), d = ld(k + 3);
    add(s, a);
    add(s, b);
    add(s, c);
    add(s, d);
  }
  for (; k < nsl; ++k) add(s, ld(k));
  *reinterpret_cast<float4*>(t + i) = s;
}

// ===================================================================================
// Kernel 2: the INT4 GEMM + low-rank up projection (+ bias), bf16 out.
//
// Block tile 256 (M) x 256 (N), 8 waves as 2 (M) x 4 (N); each wave owns a 4 x 2 grid of 32x32
// tiles. One K step = one 64-wide group. The codes and scales of each group are copied global ->
// LDS by the LDS DMA path (global_load_lds) into a ring of I4_NS slots, issued four groups before
// their first reader; one barrier per two groups publishes the next slots.
// Per group each wave unfolds its A and B operands to FP6 and runs, per tile, one FP6 MFMA with
// E8M0 scales 2^3 x 2^3 (the exact integer dot product of the group), one bf16 MFMA (the exact
// outer product s_x s_w of the raw bf16 scales) and 16 FMAs into its fp32 accumulators.
// The epilogue adds bf16(t)·L2 and the bias and writes Y through LDS in 16-byte row segments.
// ===================================================================================
constexpr int I4_THREADS = 512;

// One ring slot: the folded codes of 256 A rows and 256 B rows (32 B each, swizzled) and their
// bf16 scales (A rows 0..255, then B rows). Each slot is its own LDS object, so the compiler can
// tell the DMA writes into one slot from the reads of another.
struct I4Slot {
  uint8_t a[256 * 32];
  uint8_t b[256 * 32];
  uint16_t s[512];
  uint16_t z[32];  // zeros (never written by the DMA): k > 0 half of the scale outer-product operand
};

// The next layer's activation side in this GEMM's epilogue (the MLP's fc1 -> GELU -> fc2 join):
// fc2's 1/λ over this layer's N columns, fc2's L1ᵀ [rank2_pad][N], and fc2's outputs in library
// layout: INT4 codes [N/64][m_pad][32 B], bf16 scales [N/64][m_pad], and one partial t plane
// [m_pad][rank2_pad] per 256-column tile of this layer.
struct GeluQuantArgs {
  const float* il2;
  const uint16_t* l1t2;
  uint8_t* xq2;
  uint16_t* xs2;
  float* t2part;
};

// the block's eight ring slots, by value (indexed with constants only, so they stay in registers)
struct SlotSet {
  uint8_t* s[I4_NS];
};

template <int NT2>
__device__ __forceinline__ void gelu_quant_epilogue(v16f (&acc)[I4_MT][2], uint8_t* stage, SlotSet slots,
                                                    const GeluQuantArgs& fa, const uint16_t* bias, int M, int N,
                                                    int m_pad, int m0, int n0, int tn, int wm, int wn, int wave,
                                                    int lane);

// FUSE < 0: the plain GEMM (fa unused). FUSE >= 0 (INT4 only): fc1 of the MLP with fc2's
// activation side in the epilogue, FUSE = fc2's rank_pad / 16; Y may then be NULL.
template <int FMT, int NTR, int FUSE = -1>  // NTR = rank_pad / 16
__global__ __launch_bounds__(I4_THREADS) void gemm_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ xl1,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int ldy, int M, int N, int K,
    int m_pad, int n_pad, GeluQuantArgs fa) {
  static_assert(FMT == W4A4_FMT_INT4_G64, "MXFP4 runs on gemm_mx_small_kernel and gemm_w8a8_kernel<., true>");
  __shared__ __attribute__((aligned(16))) I4Slot sl0, sl1, sl2, sl3, sl4, sl5, sl6, sl7;
  I4Slot* const ring[I4_NS] = {&sl0, &sl1, &sl2, &sl3, &sl4, &sl5, &sl6, &sl7};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived addresses scalar
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, m_pad / I4_BM, n_pad / I4_BN, tm, tn);
  const int m0 = tm * I4_BM, n0 = tn * I4_BN;
  const int G = K / W4A4_GROUP;

  // ---- DMA sources. Instruction w of an operand fills LDS bytes [1024 w, 1024 w + 1024) of the
  // slot, lane i the 16 bytes at 1024 w + 16 i = row 32 w + i / 2, stored half i & 1; the lane
  // loads the global half that the swizzle puts there. Scales: wave w copies 256 bytes, chunk
  // w & 3 of the slot's 1 KB of scales (waves w and w + 4 write the same bytes): the bf16 scales
  // of A rows 0..127, A rows 128..255, B rows 0..127, B rows 128..255.
  const int drow = 32 * wave + (lane >> 1);
  const int dhalf = (lane & 1) ^ ((drow >> 3) & 1);
  const int c_lane = drow * 32 + 16 * dhalf;   // byte offset of the lane's 16 B in a code tile
  const int sblk = wave & 3;
  const int s_lane = 4 * lane;                 // byte offset of the lane's 4 bytes of scales
  // Buffer resources (scalar base + bounds) per operand: the lane offsets stay in one VGPR each and
  // the group offset is a scalar soffset. Loads past a buffer's end would return zeros.
  constexpr int RSRC_W3 = 0x00020000;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xq + (size_t)m0 * 32), 0, (G * m_pad - m0) * 32, RSRC_W3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq + (size_t)n0 * 32), 0, (G * n_pad - n0) * 32, RSRC_W3);
  // scale chunk of this wave: bf16 rows [128 c, 128 c + 128) of A (c = sblk) or B (c = sblk - 2)
  const bool s_is_a = sblk < 2;
  const int s_rows = s_is_a ? m_pad : n_pad, s_row0 = s_is_a ? m0 : n0, sc_ = s_is_a ? sblk : sblk - 2;
  const uint8_t* s_buf = s_is_a ? xs : ws;
  const int s_first = 2 * (s_row0 + 128 * sc_);  // bytes
  const int s_gstride = 2 * s_rows;              // bytes per group: one bf16 per row
  const int s_total = G * s_gstride;
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(s_buf + s_first), 0, s_total - s_first, RSRC_W3);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // 3 vector-memory instructions per wave and group (part 0: A codes, 1: B codes, 2: scales);
  // groups past the end reload the last group
  auto dma_part = [&](int part, int g, I4Slot* sl) {
    g = min(g, G - 1);
    if (part == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sl->a + 1024 * wave), 16, c_lane, g * m_pad * 32, 0, 0);
    else if (part == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sl->b + 1024 * wave), 16, c_lane, g * n_pad * 32, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)(sl->s + 128 * sblk), 4, s_lane, g * s_gstride, 0, 0);
  };
  auto dma = [&](int g, I4Slot* sl) {
    g = min(g, G - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sl->a + 1024 * wave), 16, c_lane, g * m_pad * 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sl->b + 1024 * wave), 16, c_lane, g * n_pad * 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)(sl->s + 128 * sblk), 4, s_lane, g * s_gstride, 0, 0);
  };

  v16f acc[I4_MT][2];
#pragma unroll
  for (int i = 0; i < I4_MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const v16f zero16 = {};
  const int lr = lane & 31, lh = lane >> 5;
  const int arow0 = wm * 128 + lr, bcol0 = wn * 64 + lr;
  // operand byte offsets inside a slot (tile i / j adds 1024 i / 1024 j)
  const int a_off = sw_off32(arow0, lh), b_off = sw_off32(bcol0, lh);

  // low-rank up projection first: acc = bf16(t) · L2 over k = rank index (32x32x16 bf16 MFMA); the
  // 4-bit groups then accumulate on top. Up to rank 32 the block's t tile (256 rows x 32 fp32 =
  // 32 KB, read by four waves each) is copied once into ring slots 6 and 7 by the LDS DMA path
  // before the ring's first groups, and the L2 operands are loaded before them too; all of it
  // lands under the prologue's wait for group 0 and the MFMAs run right after it. Larger ranks
  // load t directly, 32 ranks at a time.
  constexpr int RP = NTR * 16, KS = 2;  // up to two 16-rank MFMA K-steps per batch of loads
  constexpr bool T_LDS = NTR > 0 && NTR <= 2;
  constexpr int TROWB = RP * 4;          // bytes of one t row
  static_assert(256 * 32 * 4 <= 2 * 16384 && 16384 <= (int)sizeof(I4Slot), "t tile fits slots 6 and 7");
  // t row r of the block lives at byte r * TROWB of the tile: the first 16 KB in slot 6, the rest
  // in slot 7
  auto t_row_ptr = [&](int r) -> const uint8_t* {
    const int byte = r * TROWB;
    return byte < 16384 ? reinterpret_cast<const uint8_t*>(ring[6]) + byte
                        : reinterpret_cast<const uint8_t*>(ring[7]) + (byte - 16384);
  };
  v4i LB[KS][2];
  float4 tv[KS][I4_MT][2];
  auto lr_load = [&](int k0) {  // L2 operands, and t when it is not staged in LDS
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kk = k0 + 16 * s;
      if (kk >= RP) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        LB[s][j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + wn * 64 + j * 32 + lr) * RP + kk + 8 * lh);
      if (!T_LDS) {
#pragma unroll
        for (int i = 0; i < I4_MT; ++i) {
          const float* tp = xl1 + (size_t)(m0 + wm * 128 + i * 32 + lr) * RP + kk + 8 * lh;
          tv[s][i][0] = *reinterpret_cast<const float4*>(tp);
          tv[s][i][1] = *reinterpret_cast<const float4*>(tp + 4);
        }
      }
    }
  };
  // t from its LDS tile: one asm block with every read and its own wait (the compiler's LDS-DMA
  // tracking cannot tell slots 6/7 from the ring groups still in flight and would wait for all of
  // them). Lane address of tile row i: the row's byte in the tile plus 32 lh (ranks 8 lh ..).
  auto t_from_lds = [&]() {
    typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
    uint32_t ad[I4_MT];
#pragma unroll
    for (int i = 0; i < I4_MT; ++i)
      ad[i] = (uint32_t)(uintptr_t)(lds_cptr)t_row_ptr(wm * 128 + i * 32 + lr) + 32 * lh;
    if constexpr (NTR == 2) {
      asm volatile(
          "ds_read_b128 %0, %16\n\tds_read_b128 %1, %16 offset:16\n\t"
          "ds_read_b128 %2, %16 offset:64\n\tds_read_b128 %3, %16 offset:80\n\t"
          "ds_read_b128 %4, %17\n\tds_read_b128 %5, %17 offset:16\n\t"
          "ds_read_b128 %6, %17 offset:64\n\tds_read_b128 %7, %17 offset:80\n\t"
          "ds_read_b128 %8, %18\n\tds_read_b128 %9, %18 offset:16\n\t"
          "ds_read_b128 %10, %18 offset:64\n\tds_read_b128 %11, %18 offset:80\n\t"
          "ds_read_b128 %12, %19\n\tds_read_b128 %13, %19 offset:16\n\t"
          "ds_read_b128 %14, %19 offset:64\n\tds_read_b128 %15, %19 offset:80\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[1][0][0]), "=&v"(tv[1][0][1]),
            "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1]), "=&v"(tv[1][1][0]), "=&v"(tv[1][1][1]),
            "=&v"(tv[0][2][0]), "=&v"(tv[0][2][1]), "=&v"(tv[1][2][0]), "=&v"(tv[1][2][1]),
            "=&v"(tv[0][3][0]), "=&v"(tv[0][3][1]), "=&v"(tv[1][3][0]), "=&v"(tv[1][3][1])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
          : "memory");
    } else if constexpr (NTR == 1) {
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\t"
          "ds_read_b128 %2, %9\n\tds_read_b128 %3, %9 offset:16\n\t"
          "ds_read_b128 %4, %10\n\tds_read_b128 %5, %10 offset:16\n\t"
          "ds_read_b128 %6, %11\n\tds_read_b128 %7, %11 offset:16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1]),
            "=&v"(tv[0][2][0]), "=&v"(tv[0][2][1]), "=&v"(tv[0][3][0]), "=&v"(tv[0][3][1])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
          : "memory");
    }
  };
  auto lr_mfma = [&](int k0) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int kk = k0 + 16 * s;
      if (kk >= RP) break;
#pragma unroll
      for (int i = 0; i < I4_MT; ++i) {
        const float4 t0 = tv[s][i][0], t1 = tv[s][i][1];
        const v4i TA = v4i{(int)pack_bf16x2(t0.x, t0.y), (int)pack_bf16x2(t0.z, t0.w), (int)pack_bf16x2(t1.x, t1.y),
                           (int)pack_bf16x2(t1.z, t1.w)};
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(TA), as_bf16x8(LB[s][j]), acc[i][j], 0, 0, 0);
      }
    }
  };
  if (NTR > 0) lr_load(0);
  if (T_LDS) {  // t tile -> slots 6 and 7: TBYTES / 8 bytes per wave, 1 KB per DMA instruction
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(xl1 + (size_t)m0 * RP), 0, (m_pad - m0) * TROWB, RSRC_W3);
    constexpr int TCHUNK = 256 * TROWB / 8;
#pragma unroll
    for (int q = 0; q < TCHUNK / 1024; ++q) {
      const int off = wave * TCHUNK + q * 1024;  // chunks never straddle the 16 KB split
      uint8_t* dst = off < 16384 ? reinterpret_cast<uint8_t*>(ring[6]) + off
                                 : reinterpret_cast<uint8_t*>(ring[7]) + (off - 16384);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t_rsrc, (lds_ptr_t)dst, 16, 16 * lane, off, 0, 0);
    }
  }

  // prologue: zero words of every slot; groups 0 .. NS-3 in flight; group 0 visible
  if (tid < 32) {
#pragma unroll
    for (int s = 0; s < I4_NS; ++s) ring[s]->z[tid] = 0;
  }
#pragma unroll
  for (int s = 0; s < I4_NS - 2; ++s) dma(s, ring[s]);
  wait_vmcnt<3 * (I4_NS - 3)>();
  __builtin_amdgcn_s_barrier();
  if (NTR > 0) {
    if (T_LDS) t_from_lds();
    lr_mfma(0);
#pragma unroll
    for (int k0 = 32; k0 < RP; k0 += 32) {
      lr_load(k0);
      lr_mfma(k0);
    }
  }
  auto a_raw = [&](const I4Slot* sl, int i) { return *reinterpret_cast<const v4i*>(sl->a + a_off + 1024 * i); };
  auto b_raw = [&](const I4Slot* sl, int j) { return *reinterpret_cast<const v4i*>(sl->b + b_off + 1024 * j); };
  // Row rotation against VGPR bank conflicts. The FMA acc[v] += p[v] * sc[v] would read three
  // registers with the same index in three tuples that the allocator places at the same alignment,
  // i.e. three times the same bank. Instead the lane that supplies A row rho of the FP6 MFMA loads
  // row rot(rho, 2), and of the scale MFMA row rot(rho, 1), where rot(rho, k) is the row that the
  // 32x32 output layout (register u = 4 (rho / 8) + rho % 4 of lane half (rho / 4) % 2) puts k
  // registers earlier. Row rho of the tile then sits in register v of acc, v + 2 of p and v + 1 of
  // sc: three different banks, same arithmetic.
  auto rot = [](int rho, int k) {
    const int u = ((((rho >> 3) << 2) | (rho & 3)) - k) & 15;
    return ((u >> 2) << 3) | (rho & 4) | (u & 3);
  };
  const int a_off4 = sw_off32(wm * 128 + rot(lr, 2), lh);
  const int srow0 = wm * 128 + rot(lr, 1);
  auto a_raw4 = [&](const I4Slot* sl, int i) { return *reinterpret_cast<const v4i*>(sl->a + a_off4 + 1024 * i); };
  // operands of the scale outer product: the A side is the bf16 scale of the lane's (rotated) row
  // in every lane; the B side is the scale at k = 0 (lanes 0..31) and zero for k = 4 (lanes
  // 32..63, read from the slot's zero words), and zero for groups past the end, so S = s_x s_w
  // exactly. Kept as one zero-extended register, widened at the MFMA.
  const int sb_lane_off = lh ? (int)offsetof(I4Slot, z) : (int)offsetof(I4Slot, s) + 2 * (256 + bcol0);
  auto sa_val = [&](const I4Slot* sl, int row) -> uint32_t { return sl->s[row]; };
  auto sb_val = [&](const I4Slot* sl, int j, bool live) -> uint32_t {
    const uint32_t s = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sl) + sb_lane_off + (lh ? 0 : 64 * j));
    return live ? s : 0u;
  };
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  auto sc_op = [](uint32_t s) { return __builtin_bit_cast(v4s, v2u{s, 0u}); };

  // its first operands in registers
  v8i Bv[2], Av;
  uint32_t OB[2], OA;
  v4i An_raw, Bn_raw[2];
  uint32_t OAn, OBn[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Bv[j] = unfold_fp6(b_raw(ring[0], j));
    OB[j] = sb_val(ring[0], j, true);
  }
  Av = unfold_fp6(a_raw4(ring[0], 0));
  OA = sa_val(ring[0], srow0);
  An_raw = a_raw4(ring[0], 1);
  OAn = sa_val(ring[0], srow0 + 32);

  constexpr int T = 2 * I4_MT;
  v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Av, Bv[0], zero16, 2, 2, 0, 130, 0, 130);
  v16f sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sc_op(OA), sc_op(OB[0]), zero16, 0, 0, 0);

  for (int g0 = 0; g0 < G; g0 += I4_NS) {
#pragma unroll
    for (int u = 0; u < I4_NS; ++u) {
      const int g = g0 + u;
      const I4Slot* cur = ring[u];
      const I4Slot* nxt = ring[(u + 1) % I4_NS];
      if (u % 2 == 0) {
        // groups g+1 and g+2 have landed in every wave's share of their slots; everyone is done
        // with slots g-2 and g-1, which take groups g+NS-2 (copied during this group) and g+NS-1
        // (during the next)
        wait_vmcnt<3 * (I4_NS - 5)>();
        __builtin_amdgcn_s_barrier();
      }
      const bool live1 = g + 1 < G;
      // ---- the group's 8 tiles, software-pipelined: the FP6 MFMA of tile t+1 is issued before the
      // 16 FMAs of tile t and its outer product right after them; the last tile's successor is
      // tile 0 of group g + 1, whose operands are read from the next slot during this group
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int i = t >> 1, j = t & 1;
        const int t1 = t + 1, i1 = (t1 % T) >> 1, j1 = t1 & 1;
        // consume the operands read two tiles ago first, then issue the next reads, so that the
        // wait for the old reads never has to cover the new ones
        if (t1 == T) {  // switch to group g + 1
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            Bv[jj] = unfold_fp6(Bn_raw[jj]);
            OB[jj] = OBn[jj];
          }
        }
        if (j1 == 0) {  // new tile row: take the prefetched A operand
          Av = unfold_fp6(An_raw);
          OA = OAn;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j1 == 0) {  // prefetch the following row's A operand
          if (t1 < T - 2) {
            An_raw = a_raw4(cur, i1 + 1);
            OAn = sa_val(cur, srow0 + 32 * (i1 + 1));
          } else {  // rows 0 and 1 of the next group follow rows 3 and 0
            const int r1 = t1 == T - 2 ? 0 : 1;
            An_raw = a_raw4(nxt, r1);
            OAn = sa_val(nxt, srow0 + 32 * r1);
          }
        }
        if (t1 == T - 2) {  // next group's B operands and scales
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            Bn_raw[jj] = b_raw(nxt, jj);
            OBn[jj] = sb_val(nxt, jj, live1);
          }
        }
        // this group's copy of group g + NS - 2 into the slot freed at the last barrier, one
        // instruction every other tile (issued together right after the barrier, the copies of all
        // eight waves queue up at once and stall their issue: measured 5-7% slower)
        if (t == 1 || t == 3 || t == 5) dma_part(t >> 1, g + I4_NS - 2, ring[(u + I4_NS - 2) % I4_NS]);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch reads here, two tiles ahead of their use
        // raised wave priority around each MFMA issue keeps the matrix pipe fed while the other
        // wave of the SIMD is in its FMAs
        __builtin_amdgcn_s_setprio(1);
        const v16f pn = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Av, Bv[j1], zero16, 2, 2, 0, 130, 0, 130);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_fmaf(p[(v + 2) & 15], sc[(v + 1) & 15], acc[i][j][v]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sc_op(OA), sc_op(OB[j1]), zero16, 0, 0, 0);
        __builtin_amdgcn_s_setprio(0);
        p = pn;
      }
    }
  }
  wait_vmcnt<0>();  // no LDS DMA may outlive the block
  __builtin_amdgcn_s_barrier();  // every wave is done with the ring (and its DMA has landed)
  uint8_t* stage = reinterpret_cast<uint8_t*>(ring[0]);
#pragma unroll
  for (int w = 1; w < I4_NS; ++w)
    if (wave == w) stage = reinterpret_cast<uint8_t*>(ring[w]);  // wave-uniform select
  static_assert(64 * Y_ES <= (int)sizeof(I4Slot), "staging fits a ring slot");
  if constexpr (FUSE < 0) {
    store_y(acc, stage, bias, Y, ldy, M, N, m0 + wm * 128, n0 + wn * 64, lane);
  } else {
    if (Y) store_y(acc, stage, bias, Y, ldy, M, N, m0 + wm * 128, n0 + wn * 64, lane);  // for checking
    const SlotSet slots{{reinterpret_cast<uint8_t*>(&sl0), reinterpret_cast<uint8_t*>(&sl1),
                         reinterpret_cast<uint8_t*>(&sl2), reinterpret_cast<uint8_t*>(&sl3),
                         reinterpret_cast<uint8_t*>(&sl4), reinterpret_cast<uint8_t*>(&sl5),
                         reinterpret_cast<uint8_t*>(&sl6), reinterpret_cast<uint8_t*>(&sl7)}};
    gelu_quant_epilogue<FUSE>(acc, stage, slots, fa, bias, M, N, m_pad, m0, n0, tn, wm, wn, wave, lane);
  }
}


// fc2's activation side from this wave's 128 x 64 block of fc1 results: X₂ = bf16(GELU(bf16(acc +
// bias))) (padding rows: 0), staged in the wave's ring slot 64 rows at a time (row stride Y_ES),
// read back with the activation kernel's lane layout (16 rows x 4 lanes of 16 values per pass),
// smoothed, quantized to INT4 codes of fc2's group n0/64 + wn, and multiplied into partial
// t₂ = bf16(X̂₂)·L1₂ (16x16x32 bf16 MFMAs, L1₂ operands loaded once). The four waves that share
// block rows then sum their partials through LDS in a fixed order into this tile's plane.
template <int NT2>
__device__ __forceinline__ void gelu_quant_epilogue(v16f (&acc)[I4_MT][2], uint8_t* stage, SlotSet slots,
                                                    const GeluQuantArgs& fa, const uint16_t* bias, int M, int N,
                                                    int m_pad, int m0, int n0, int tn, int wm, int wn, int wave,
                                                    int lane) {
  constexpr int RP2 = NT2 * 16, NT2A = NT2 > 0 ? NT2 : 1;
  const int lr = lane & 31, lh = lane >> 5;  // 32x32 MFMA output layout
  const int r = lane & 15, kc = lane >> 4;   // activation-kernel layout
  const int gcol0 = n0 + wn * 64;
  const bool gvalid = gcol0 < N;  // N is a multiple of 64: the wave's columns are one whole group
  const int g2 = gcol0 >> 6;
  float bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = gcol0 + j * 32 + lr;
    bcol[j] = (bias && col < N) ? bf16f(bias[col]) : 0.f;
  }
  float il[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v = gvalid ? *reinterpret_cast<const float4*>(fa.il2 + gcol0 + kc * 16 + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
    il[4 * q] = v.x;
    il[4 * q + 1] = v.y;
    il[4 * q + 2] = v.z;
    il[4 * q + 3] = v.w;
  }
  v4i B2[NT2A][2];
  v4f tacc[8][NT2A];
#pragma unroll
  for (int c = 0; c < NT2A; ++c) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      B2[c][h] = (NT2 > 0 && gvalid)
                     ? *reinterpret_cast<const v4i*>(fa.l1t2 + (size_t)(c * 16 + r) * N + gcol0 + kc * 16 + 8 * h)
                     : v4i{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < 8; ++p) tacc[p][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int rl = ii * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          const int grow = m0 + wm * 128 + half * 64 + rl;  // rows grow, grow + 1
          const uint32_t y = pack_bf16x2(acc[2 * half + ii][j][v] + bcol[j], acc[2 * half + ii][j][v + 1] + bcol[j]);
          const uint32_t x0 = grow < M ? bf16_rne(gelu32(bf16f(y & 0xFFFFu))) : 0u;
          const uint32_t x1 = grow + 1 < M ? bf16_rne(gelu32(bf16f(y >> 16))) : 0u;
          uint16_t* d = reinterpret_cast<uint16_t*>(stage + rl * Y_ES + (j * 32 + lr) * 2);
          d[0] = (uint16_t)x0;
          d[Y_ES / 2] = (uint16_t)x1;
        }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int rr = pass * 16 + r;
      const int row = m0 + wm * 128 + half * 64 + rr;
      const uint4 lo = *reinterpret_cast<const uint4*>(stage + rr * Y_ES + kc * 32);
      const uint4 hi = *reinterpret_cast<const uint4*>(stage + rr * Y_ES + kc * 32 + 16);
      const uint32_t xw[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      float xh[2][8];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t bits = (e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xFFFFu);
        xh[e >> 3][e & 7] = bf16f(bits) * il[e];  // X̂₂, one fp32 multiply
      }
      uint32_t sb;
      const uint2 q = quant_int4_lane(xh, sb);
      if (gvalid) {
        *reinterpret_cast<uint2*>(fa.xq2 + ((size_t)g2 * m_pad + row) * 32 + kc * 8) = q;
        if (kc == 0) fa.xs2[(size_t)g2 * m_pad + row] = (uint16_t)sb;
      }
      if constexpr (NT2 > 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v4i a;
#pragma unroll
          for (int d = 0; d < 4; ++d) a[d] = (int)pack_bf16x2(xh[h][2 * d], xh[h][2 * d + 1]);
#pragma unroll
          for (int c = 0; c < NT2; ++c)
            tacc[half * 4 + pass][c] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(B2[c][h]), tacc[half * 4 + pass][c], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (NT2 > 0) {
    // 16x16 MFMA output: lane holds rank column c*16 + lane%16, rows 4*(lane/16) + v of its pass
    __builtin_amdgcn_s_barrier();  // every wave is done with its staging slot
    float* mine = reinterpret_cast<float*>(stage);  // the wave's own slot
    static_assert(128 * RP2 * 4 <= (int)sizeof(I4Slot), "a wave's partial t fits its ring slot");
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
      for (int c = 0; c < NT2; ++c)
#pragma unroll
        for (int v = 0; v < 4; ++v) mine[(p * 16 + 4 * kc + v) * RP2 + c * 16 + r] = tacc[p][c][v];
    __builtin_amdgcn_s_barrier();
    const int tid = wave * 64 + lane;
    constexpr int Q = RP2 / 4;  // float4 per row
#pragma unroll
    for (int idx0 = 0; idx0 < 256 * Q; idx0 += I4_THREADS) {
      const int idx = idx0 + tid, row = idx / Q, q = idx % Q;
      const int wr = row >> 7, lrow = row & 127;
      float4 sum = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // the four column waves of these rows, in order
        const float* src = reinterpret_cast<const float*>(wr ? slots.s[4 + w] : slots.s[w]);
        const float4 v = *reinterpret_cast<const float4*>(src + lrow * RP2 + 4 * q);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
      }
      *reinterpret_cast<float4*>(fa.t2part + ((size_t)tn * m_pad + m0 + row) * RP2 + 4 * q) = sum;
    }
  }
}

// ===================================================================================
// Kernel 2b: the MXFP4 GEMM on 128 x 128 blocks, for grids with fewer 256 x 256 tiles than the
// GPU has compute units (small M: K = N = 3072 at M = 1024 is 48 large tiles for 256 CUs). Four
// waves as 2 x 2, each 64 x 64 (2 x 2 tiles of 32x32); a ring of 8 slots of 9 KB, so two blocks
// share a CU (the kernel runs when one round of blocks covers the grid; a 16-slot ring, one block per
// CU, measured no faster at M = 1024; larger grids run the MXFP4 mode of the INT8 GEMM). Codes and
// E8M0 block scales are copied by the LDS DMA path six groups ahead, one barrier per two groups,
// the scaled MFMA applies the block scales, the low-rank up projection comes first (t and L2
// straight from global memory), Y goes out through LDS.
// Groups past the end of K are zero-filled by pointing the copy's lane offset past the buffer's
// range (a raw buffer load outside num_records returns zeros): zero codes add exactly 0.
// ===================================================================================
constexpr int MX_BM = 128, MX_THREADS = 256, MX_MT = 2;
constexpr int MX_NS = 8;            // ring slots (groups); even
constexpr int MX_SMALL_GRID = 512;  // the 128 x 128 kernel runs when its grid is at most this

struct MxSlot {
  uint8_t a[128 * 32];
  uint8_t b[128 * 32];
  uint8_t s[512];    // E8M0: A block 2g (128 rows), A block 2g+1, B block 2g, B block 2g+1
  uint8_t pad[512];  // 9 KB: room for a wave's 64 x 144-byte Y staging
};

template <int NTR>  // NTR = rank_pad / 16
__global__ __launch_bounds__(MX_THREADS, 2) void gemm_mx_small_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ xl1,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int ldy, int M, int N, int K,
    int m_pad, int n_pad) {
  __shared__ __attribute__((aligned(16))) MxSlot sl0, sl1, sl2, sl3, sl4, sl5, sl6, sl7;
  MxSlot* const ring[MX_NS] = {&sl0, &sl1, &sl2, &sl3, &sl4, &sl5, &sl6, &sl7};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, m_pad / MX_BM, n_pad / MX_BM, tm, tn);
  const int m0 = tm * MX_BM, n0 = tn * MX_BM;
  const int G = K / W4A4_GROUP;

  // code DMA: wave w fills bytes [1024 w, 1024 w + 1024) of an operand's 4 KB, lane i the 16 B of
  // row 32 w + i / 2 that the swizzle puts there
  const int drow = 32 * wave + (lane >> 1);
  const int c_lane = drow * 32 + 16 * ((lane & 1) ^ ((drow >> 3) & 1));
  constexpr int RSRC_W3 = 0x00020000;
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(xq + (size_t)m0 * 32), 0, (G * m_pad - m0) * 32, RSRC_W3);
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq + (size_t)n0 * 32), 0, (G * n_pad - n0) * 32, RSRC_W3);
  // scale DMA: the 256 B of A (even waves) or B (odd waves; waves 2 and 3 repeat 0 and 1): lanes
  // 0..31 the 128 rows of block 2g, lanes 32..63 those of block 2g + 1 (planes [K/32][rows])
  const bool s_is_a = (wave & 1) == 0;
  const int s_rows = s_is_a ? m_pad : n_pad, s_row0 = s_is_a ? m0 : n0;
  const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>((s_is_a ? xs : ws) + s_row0), 0, (K / W4A4_MX_BLOCK) * s_rows - s_row0, RSRC_W3);
  const int s_lane = (lane >> 5) * s_rows + 4 * (lane & 31);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](int g, MxSlot* sl) {  // 3 vector-memory instructions per wave and group
    const int oob = g < G ? 0 : (int)0x80000000;
    g = min(g, G - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sl->a + 1024 * wave), 16, c_lane | oob, g * m_pad * 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sl->b + 1024 * wave), 16, c_lane | oob, g * n_pad * 32, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)(sl->s + 256 * (wave & 1)), 4, s_lane, g * 2 * s_rows, 0, 0);
  };

  v16f acc[MX_MT][2];
#pragma unroll
  for (int i = 0; i < MX_MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};
  const int lr = lane & 31, lh = lane >> 5;
  const int arow0 = wm * 64 + lr, bcol0 = wn * 64 + lr;

  // low-rank up projection first: acc = bf16(t)·L2 (32x32x16 bf16 MFMAs), 32 ranks per batch of
  // register loads; the first batch is issued before the ring's copies and lands under the
  // prologue's wait
  constexpr int RP = NTR * 16;
  v4i LB[2][2];
  float4 tv[2][MX_MT][2];
  auto lr_load = [&](int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = k0 + 16 * s;
      if (kk >= RP) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        LB[s][j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + bcol0 + j * 32) * RP + kk + 8 * lh);
#pragma unroll
      for (int i = 0; i < MX_MT; ++i) {
        const float* tp = xl1 + (size_t)(m0 + arow0 + i * 32) * RP + kk + 8 * lh;
        tv[s][i][0] = *reinterpret_cast<const float4*>(tp);
        tv[s][i][1] = *reinterpret_cast<const float4*>(tp + 4);
      }
    }
  };
  auto lr_mfma = [&](int k0) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (k0 + 16 * s >= RP) break;
#pragma unroll
      for (int i = 0; i < MX_MT; ++i) {
        const float4 t0 = tv[s][i][0], t1 = tv[s][i][1];
        const v4i TA = v4i{(int)pack_bf16x2(t0.x, t0.y), (int)pack_bf16x2(t0.z, t0.w), (int)pack_bf16x2(t1.x, t1.y),
                           (int)pack_bf16x2(t1.z, t1.w)};
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(TA), as_bf16x8(LB[s][j]), acc[i][j], 0, 0, 0);
      }
    }
  };
  if (NTR > 0) lr_load(0);
#pragma unroll
  for (int s = 0; s < MX_NS - 2; ++s) dma(s, ring[s]);
  wait_vmcnt<3 * (MX_NS - 3)>();  // the low-rank operands and group 0 have landed
  __builtin_amdgcn_s_barrier();
  if (NTR > 0) {
    lr_mfma(0);
#pragma unroll
    for (int k0 = 32; k0 < RP; k0 += 32) {  // larger ranks: later batches wait for their loads
      lr_load(k0);
      wait_vmcnt<0>();
      lr_mfma(k0);
    }
  }

  const int a_off = sw_off32(arow0, lh), b_off = sw_off32(bcol0, lh);
  // operands of group g + 1 are read at the start of group g (double-buffered registers)
  auto rd = [&](const MxSlot* sl, v4i (&A)[MX_MT], v4i (&B)[2], int (&sA)[MX_MT], int (&sB)[2]) {
#pragma unroll
    for (int i = 0; i < MX_MT; ++i) {
      A[i] = *reinterpret_cast<const v4i*>(sl->a + a_off + 1024 * i);
      sA[i] = sl->s[128 * lh + arow0 + 32 * i];
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      B[j] = *reinterpret_cast<const v4i*>(sl->b + b_off + 1024 * j);
      sB[j] = sl->s[256 + 128 * lh + bcol0 + 32 * j];
    }
  };
  auto op8 = [](v4i v) { return v8i{v[0], v[1], v[2], v[3], 0, 0, 0, 0}; };
  v4i A[2][MX_MT], B[2][2];
  int sA[2][MX_MT], sB[2][2];
  rd(ring[0], A[0], B[0], sA[0], sB[0]);
  for (int g0 = 0; g0 < G; g0 += MX_NS) {
#pragma unroll
    for (int u = 0; u < MX_NS; ++u) {
      const int g = g0 + u, c = u & 1;
      if (u % 2 == 0) {
        // groups g+1 and g+2 have landed; everyone is done with slots g-2 and g-1, which take
        // groups g+NS-2 (copied during this group) and g+NS-1 (during the next)
        wait_vmcnt<3 * (MX_NS - 5)>();
        __builtin_amdgcn_s_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      rd(ring[(u + 1) % MX_NS], A[c ^ 1], B[c ^ 1], sA[c ^ 1], sB[c ^ 1]);
      dma(g + MX_NS - 2, ring[(u + MX_NS - 2) % MX_NS]);
#pragma unroll
      for (int t = 0; t < 2 * MX_MT; ++t) {
        const int i = t >> 1, j = t & 1;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op8(A[c][i]), op8(B[c][j]), acc[i][j], 4, 4, 0,
                                                                  sA[c][i], 0, sB[c][j]);
      }
      // the next group's LDS reads and this group's copies issue between this group's MFMAs
#pragma unroll
      for (int q = 0; q < 2 * MX_MT; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        if (q < 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one copy
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);    // the rest of the reads
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  wait_vmcnt<0>();  // no LDS DMA may outlive the block
  __builtin_amdgcn_s_barrier();
  uint8_t* stage = reinterpret_cast<uint8_t*>(ring[0]);
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (wave == w) stage = reinterpret_cast<uint8_t*>(ring[w]);  // wave-uniform select
  static_assert(64 * Y_ES <= (int)sizeof(MxSlot), "staging fits a ring slot");
  store_y(acc, stage, bias, Y, ldy, M, N, m0 + wm * 64, n0 + wn * 64, lane);
}

// ----------------------------------------------------------------------------- launch helpers
template <int FMT, int NT, bool GELU_IN = false>
hipError_t launch_qa(const uint16_t* X, int M, int K, int ldx, const float* il, const uint16_t* l1t, int m_pad,
                     uint8_t* xq, void* xs, float* xl1, hipStream_t st) {
  const int gs = qa_group_slice(M, K), nsl = qa_slices(M, K);
  const size_t lds = 16 * (size_t)qa_lds_slots(NT * 16, gs);
  if (lds > 65536) {  // large ranks: allow the block more than 64 KB of dynamic LDS
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&quantize_act_kernel<FMT, NT, GELU_IN>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
  }
  hipLaunchKernelGGL((quantize_act_kernel<FMT, NT, GELU_IN>), dim3(m_pad / QA_BLOCK_ROWS * nsl), dim3(QA_WAVES * 64), lds, st,
                     X, M, K, ldx, il, l1t, m_pad, gs, xq, xs, xl1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (FMT == W4A4_FMT_W8A8)  // per-token scales from the slices' partial maxima, the codes, and t
    return launch_quantize_w8(X, M, K, ldx, il, m_pad, nsl, xq, static_cast<float*>(xs), xl1, NT * 16, st);
  if (NT == 0 || nsl == 1) return hipSuccess;
  const int n = m_pad * NT * 16;
  hipLaunchKernelGGL(t_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, xl1 + n, nsl, n, xl1);
  return hipGetLastError();
}

template <int FMT, bool GELU_IN = false>
hipError_t dispatch_qa(int nt, const uint16_t* X, int M, int K, int ldx, const float* il, const uint16_t* l1t,
                       int m_pad, uint8_t* xq, void* xs, float* xl1, hipStream_t st) {
  switch (nt) {
#define W4A4_QA_CASE(n) \
  case n: return launch_qa<FMT, n, GELU_IN>(X, M, K, ldx, il, l1t, m_pad, xq, xs, xl1, st);
    W4A4_QA_CASE(0) W4A4_QA_CASE(1) W4A4_QA_CASE(2) W4A4_QA_CASE(3) W4A4_QA_CASE(4)
    W4A4_QA_CASE(5) W4A4_QA_CASE(6) W4A4_QA_CASE(7) W4A4_QA_CASE(8)
#undef W4A4_QA_CASE
  }
  return hipErrorInvalidValue;
}

template <int NTR>
hipError_t launch_gemm(int fmt, const uint8_t* xq, const void* xs, const float* xl1, const uint8_t* wq,
                       const void* ws, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy, int M,
                       int N, int K, int m_pad, int n_pad, hipStream_t st) {
  const dim3 grid((m_pad / I4_BM) * (n_pad / I4_BN)), block(I4_THREADS);
  const uint8_t* xsb = static_cast<const uint8_t*>(xs);
  const uint8_t* wsb = static_cast<const uint8_t*>(ws);
  if (fmt == W4A4_FMT_INT4_G64)
    hipLaunchKernelGGL((gemm_kernel<W4A4_FMT_INT4_G64, NTR>), grid, block, 0, st, xq, xsb, xl1, wq, wsb, l2t, bias, Y,
                       ldy, M, N, K, m_pad, n_pad, GeluQuantArgs{});
  else if ((m_pad / MX_BM) * (n_pad / MX_BM) <= MX_SMALL_GRID)  // one round of small blocks (2 per CU) covers it
    hipLaunchKernelGGL((gemm_mx_small_kernel<NTR>), dim3((m_pad / MX_BM) * (n_pad / MX_BM)), dim3(MX_THREADS), 0, st,
                       xq, xsb, xl1, wq, wsb, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad);
  else  // larger grids: the INT8 kernel's structure (copies from one wave per SIMD) on FP4 operands
    return dispatch_gemm_mx(NTR, xq, xsb, xl1, wq, wsb, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad, st);
  return hipGetLastError();
}

template <int NTR, int NT2>
hipError_t launch_gemm_gelu_quant(const uint8_t* xq, const void* xs, const float* xl1, const uint8_t* wq,
                                  const void* ws, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy,
                                  int M, int N, int K, int m_pad, int n_pad, const GeluQuantArgs& fa, float* t2,
                                  hipStream_t st) {
  const int tiles_n = n_pad / I4_BN;
  hipLaunchKernelGGL((gemm_kernel<W4A4_FMT_INT4_G64, NTR, NT2>), dim3((m_pad / I4_BM) * tiles_n), dim3(I4_THREADS), 0, st, xq,
                     static_cast<const uint8_t*>(xs), xl1, wq, static_cast<const uint8_t*>(ws), l2t, bias, Y, ldy, M, N,
                     K, m_pad, n_pad, fa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || NT2 == 0 || tiles_n == 1) return e;
  const int n = m_pad * NT2 * 16;
  hipLaunchKernelGGL(t_reduce_kernel, dim3((n / 4 + 255) / 256), dim3(256), 0, st, fa.t2part, tiles_n, n, t2);
  return hipGetLastError();
}

hipError_t dispatch_gemm_gelu_quant(int ntr, int nt2, const uint8_t* xq, const void* xs, const float* xl1,
                                    const uint8_t* wq, const void* ws, const uint16_t* l2t, const uint16_t* bias,
                                    uint16_t* Y, int ldy, int M, int N, int K, int m_pad, int n_pad,
                                    const GeluQuantArgs& fa, float* t2, hipStream_t st) {
#define W4A4_GQ_CASE(a, b)                                                                                      \
  if (ntr == a && nt2 == b)                                                                                      \
    return launch_gemm_gelu_quant<a, b>(xq, xs, xl1, wq, ws, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad, fa, t2, st);
  W4A4_GQ_CASE(0, 0) W4A4_GQ_CASE(0, 1) W4A4_GQ_CASE(0, 2)
  W4A4_GQ_CASE(1, 0) W4A4_GQ_CASE(1, 1) W4A4_GQ_CASE(1, 2)
  W4A4_GQ_CASE(2, 0) W4A4_GQ_CASE(2, 1) W4A4_GQ_CASE(2, 2)
#undef W4A4_GQ_CASE
  return hipErrorInvalidValue;
}

hipError_t dispatch_gemm(int ntr, int fmt, const uint8_t* xq, const void* xs, const float* xl1, const uint8_t* wq,
                         const void* ws, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy, int M,
                         int N, int K, int m_pad, int n_pad, hipStream_t st) {
  switch (ntr) {
#define W4A4_G_CASE(n) \
  case n: return launch_gemm<n>(fmt, xq, xs, xl1, wq, ws, l2t, bias, Y, ldy, M, N, K, m_pad, n_pad, st);
    W4A4_G_CASE(0) W4A4_G_CASE(1) W4A4_G_CASE(2) W4A4_G_CASE(3) W4A4_G_CASE(4)
    W4A4_G_CASE(5) W4A4_G_CASE(6) W4A4_G_CASE(7) W4A4_G_CASE(8)
#undef W4A4_G_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace

// ================================================================================ C ABI (device)
extern "C" {

w4a4_status_t w4a4_quantize_act(const uint16_t* X, int M, int K, int ldx, const float* inv_lambda,
                                const uint16_t* l1t, int rank, int fmt, uint8_t* xq, void* xscale, float* xl1,
                                w4a4_stream_t stream) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  // N is not involved on this side; rank <= K is the relevant bound
  w4a4_status_t st = check_shape(M, rank > 0 ? rank : 1, K, rank, fmt);
  if (st != W4A4_OK) return st;
  if (!X || !inv_lambda || !xq || !xscale) return W4A4_ERR_INVALID_ARG;
  if (ldx < K || ldx % 8 != 0) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(inv_lambda) || !aligned16(xq) || !aligned16(xscale)) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!l1t || !xl1 || !aligned16(l1t) || !aligned16(xl1))) return W4A4_ERR_INVALID_ARG;
  const int m_pad = rows_pad_of(M), nt = rank_pad_of(rank) / 16;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (fmt == W4A4_FMT_INT4_G64)
    e = dispatch_qa<W4A4_FMT_INT4_G64>(nt, X, M, K, ldx, inv_lambda, l1t, m_pad, xq, xscale, xl1, hs);
  else if (fmt == W4A4_FMT_MXFP4_B32)
    e = dispatch_qa<W4A4_FMT_MXFP4_B32>(nt, X, M, K, ldx, inv_lambda, l1t, m_pad, xq, xscale, xl1, hs);
  else
    e = dispatch_qa<W4A4_FMT_W8A8>(nt, X, M, K, ldx, inv_lambda, l1t, m_pad, xq, xscale, xl1, hs);
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

w4a4_status_t w4a4_lowrank_linear(const uint8_t* xq, const void* xscale, const float* xl1, const uint8_t* wq,
                                  const void* wscale, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y,
                                  int ldy, int M, int N, int K, int rank, int fmt, w4a4_stream_t stream) {
  w4a4_status_t st = check_shape(M, N, K, rank, fmt);
  if (st != W4A4_OK) return st;
  if (!xq || !xscale || !wq || !wscale || !Y || ldy < N) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xscale) || !aligned16(wq) || !aligned16(wscale)) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!xl1 || !l2t || !aligned16(xl1) || !aligned16(l2t))) return W4A4_ERR_INVALID_ARG;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return W4A4_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(Y) & 1u) return W4A4_ERR_INVALID_ARG;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = fmt == W4A4_FMT_W8A8
                     ? dispatch_gemm_w8a8(rank_pad_of(rank) / 16, xq, static_cast<const float*>(xscale), xl1, wq,
                                          static_cast<const float*>(wscale), l2t, bias, Y, ldy, M, N, K,
                                          rows_pad_of(M), rows_pad_of(N), hs)
                     : dispatch_gemm(rank_pad_of(rank) / 16, fmt, xq, xscale, xl1, wq, wscale, l2t, bias, Y, ldy, M,
                                     N, K, rows_pad_of(M), rows_pad_of(N), hs);
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

w4a4_status_t w4a4_gelu_quantize_act(const uint16_t* Y, int M, int K, int ldy, const float* inv_lambda,
                                     const uint16_t* l1t, int rank, int fmt, uint8_t* xq, void* xscale, float* xl1,
                                     w4a4_stream_t stream) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  if (fmt != W4A4_FMT_INT4_G64) return W4A4_ERR_UNSUPPORTED;
  w4a4_status_t st = check_shape(M, rank > 0 ? rank : 1, K, rank, fmt);
  if (st != W4A4_OK) return st;
  if (!Y || !inv_lambda || !xq || !xscale) return W4A4_ERR_INVALID_ARG;
  if (ldy < K || ldy % 8 != 0) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(Y) || !aligned16(inv_lambda) || !aligned16(xq) || !aligned16(xscale)) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!l1t || !xl1 || !aligned16(l1t) || !aligned16(xl1))) return W4A4_ERR_INVALID_ARG;
  const hipError_t e = dispatch_qa<W4A4_FMT_INT4_G64, true>(rank_pad_of(rank) / 16, Y, M, K, ldy, inv_lambda, l1t,
                                                            rows_pad_of(M), xq, xscale, xl1,
                                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

w4a4_status_t w4a4_lowrank_linear_gelu_quant(const uint8_t* xq, const void* xscale, const float* xl1,
                                             const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                             const uint16_t* bias, int M, int N, int K, int rank, int fmt,
                                             const float* inv_lambda2, const uint16_t* l1t2, int rank2,
                                             uint8_t* xq2, void* xscale2, float* xl1_2, uint16_t* Y, int ldy,
                                             w4a4_stream_t stream) {
  w4a4_status_t st = check_shape(M, N, K, rank, fmt);
  if (st != W4A4_OK) return st;
  if (fmt != W4A4_FMT_INT4_G64 || rank > 32 || rank2 > 32) return W4A4_ERR_UNSUPPORTED;
  // the next layer's K is this layer's N: whole groups of 64
  st = check_shape(M, rank2 > 0 ? rank2 : 1, N, rank2, fmt);
  if (st != W4A4_OK) return st;
  if (!xq || !xscale || !wq || !wscale || !inv_lambda2 || !xq2 || !xscale2) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(xq) || !aligned16(xscale) || !aligned16(wq) || !aligned16(wscale)) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(inv_lambda2) || !aligned16(xq2) || !aligned16(xscale2)) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!xl1 || !l2t || !aligned16(xl1) || !aligned16(l2t))) return W4A4_ERR_INVALID_ARG;
  if (rank2 > 0 && (!l1t2 || !xl1_2 || !aligned16(l1t2) || !aligned16(xl1_2))) return W4A4_ERR_INVALID_ARG;
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 1u)) return W4A4_ERR_INVALID_ARG;
  if (Y && ((reinterpret_cast<uintptr_t>(Y) & 1u) || ldy < N)) return W4A4_ERR_INVALID_ARG;
  const int m_pad = rows_pad_of(M), n_pad = rows_pad_of(N), rp2 = rank_pad_of(rank2);
  const int tiles_n = n_pad / 256;
  GeluQuantArgs fa{inv_lambda2, l1t2, xq2, static_cast<uint16_t*>(xscale2),
                   rank2 > 0 ? (tiles_n > 1 ? xl1_2 + (size_t)m_pad * rp2 : xl1_2) : nullptr};
  const hipError_t e = dispatch_gemm_gelu_quant(rank_pad_of(rank) / 16, rp2 / 16, xq, xscale, xl1, wq, wscale, l2t,
                                                bias, Y, ldy, M, N, K, m_pad, n_pad, fa, xl1_2,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

size_t w4a4_gelu_quant_xl1_bytes(int M, int N, int rank2) {
  if (M < 1 || N < 1 || rank2 < 1) return 0;
  const size_t t = size_t(rows_pad_of(M)) * size_t(rank_pad_of(rank2)) * 4;
  const size_t tiles_n = size_t(rows_pad_of(N) / 256);
  return tiles_n > 1 ? t * (1 + tiles_n) : t;
}

}  // extern "C"
