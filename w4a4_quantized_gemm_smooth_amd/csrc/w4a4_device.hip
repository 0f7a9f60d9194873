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
//    32x32x64 MFMA is exactly one group. The codes are stored as these FP6 images (6 bits per
//    code: a 16-byte main part and an 8-byte extra part per half row-group), so the GEMM reads its
//    MFMA operands from LDS as they are.
//  * The per-group scale product s_x[m,g] * s_w[n,g] of a 32x32 tile is produced as an exact
//    outer product by one bf16 MFMA (v_mfma_f32_32x32x8_bf16 with one non-zero k), so the
//    group epilogue costs one fp32 FMA per output element.
//  * FP4 (E2M1) codes with E8M0 block scales run on the same scaled MFMA with the block scales
//    applied by the hardware.
//  * The low-rank branch uses the bf16 MFMAs (16x16x32 for the down projection, 32x32x16 for the
//    up projection, accumulating straight into the GEMM accumulators).

#include <atomic>
#include <mutex>

#include "w4a4_device_common.h"

using namespace w4a4;
using namespace w4a4::dev;

namespace {

// INT4 code layout (shared with the host preparation): per row and group the FP6 images of the four
// 16-code runs (run j = codes 16j .. 16j+15, image dwords d0 d1 d2, field f = sign<<5 | |q| at bit
// 6f). Half h (runs 2h, 2h+1) is one lane's 6-dword MFMA operand, split into a 16-byte main part
// [d0 d1 d2 of run 2h, d0 of run 2h+1] at byte (g·rows_pad + row)·32 + 16h and an 8-byte extra part
// [d1 d2 of run 2h+1] at byte rows_pad·K/2 + ((2g + h)·rows_pad + row)·8 of the code buffer.
// Byte offset of the part that run kc (kc = 0..3) of a row of group g stores whole: run 2h the 16-byte
// main part of half h (its own three dwords and run 2h+1's first, taken from that run's lane), run
// 2h+1 the 8-byte extra part (its other two dwords).
__device__ __forceinline__ int int4_part_offset(int g, int row, int rows_pad, int K, int kc) {
  const int h = kc >> 1;
  return (kc & 1) == 0 ? (g * rows_pad + row) * 32 + 16 * h
                       : rows_pad * (K / 2) + ((2 * g + h) * rows_pad + row) * 8;
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

// The GELU of a bf16 input rounded to bf16 is a function of the input's 16 bits. The kernels
// take it from a table of bf16(gelu32(x)) over the inputs with 2^-20 <= |x| < 256 (biased exponent
// 107..134, both signs: 2 x 28 x 128 entries, 14 KB) that they keep in LDS, and evaluate gelu32
// itself for every other input (zeros, tiny and huge magnitudes, Inf and NaN: rare in a layer's
// output); either way the value is exactly what evaluating gelu32 gives. The table, laid out
// [sign][exponent - 107][mantissa], is filled once per device by gelu_table_kernel with the
// function above and copied into each block's LDS.
constexpr int GELU_E0 = 107, GELU_NE = 28;                 // exponents 107 .. 134
constexpr int GELU_SIGN = GELU_NE * 128;                   // entries per sign
constexpr int GELU_TAB = 2 * GELU_SIGN;                    // 7168 entries
constexpr int GELU_SLOTS = GELU_TAB * 2 / 16;              // 896 16-byte LDS slots
static __device__ __attribute__((aligned(16))) uint16_t gelu_tab[GELU_TAB];
__global__ void gelu_table_kernel() {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= GELU_TAB) return;
  const uint32_t x = (uint32_t)(i / GELU_SIGN) << 15 | (uint32_t)(GELU_E0 + (i % GELU_SIGN) / 128) << 7 | (uint32_t)(i % 128);
  gelu_tab[i] = (uint16_t)bf16_rne(gelu32(bf16f(x)));
}
// offset of bf16 input `b` in the table's magnitude range, or >= GELU_SIGN outside it
__device__ __forceinline__ uint32_t gelu_off(uint32_t b) { return (b & 0x7FFFu) - (uint32_t)(GELU_E0 << 7); }
// bf16(GELU(b)) from the LDS table `tab` for an input in its range (gelu_off(b) < GELU_SIGN)
__device__ __forceinline__ uint32_t gelu_tab_lookup(uint32_t b, const uint16_t* tab) {
  return tab[gelu_off(b) + (b >> 15) * (uint32_t)GELU_SIGN];
}
// bf16(GELU(b)) for any input
__device__ __forceinline__ uint32_t gelu_any(uint32_t b, const uint16_t* tab) {
  return gelu_off(b) < (uint32_t)GELU_SIGN ? gelu_tab_lookup(b, tab) : bf16_rne(gelu32(bf16f(b)));
}
// 2 NW inputs packed two to a word (input 2e in the low half of w[e]) -> b[2e], b[2e + 1], the
// same values as gelu_any of each: the plain lookups when every input of the lane is in the
// table's range. The offsets, their range check and the table byte offsets (below 14 KB) are
// formed two inputs at a time with packed 16-bit integer operations; the table's LDS address is
// added per input.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int NW>
__device__ __forceinline__ void gelu_pk(const uint32_t (&w)[NW], uint32_t (&b)[2 * NW], const uint16_t* tab) {
  typedef __attribute__((address_space(3))) const uint16_t* lds_u16;
  constexpr unsigned short E0 = GELU_E0 << 7, SIGN_BYTES = 2 * GELU_SIGN;
  u16x2 off[NW], mx = {0, 0};
#pragma unroll
  for (int e = 0; e < NW; ++e) {
    off[e] = __builtin_bit_cast(u16x2, w[e] & 0x7FFF7FFFu) - u16x2{E0, E0};  // gelu_off of both halves
    mx = __builtin_elementwise_max(mx, off[e]);
  }
  if (mx.x < GELU_SIGN && mx.y < GELU_SIGN) {
    const uint32_t base = (uint32_t)(uintptr_t)(lds_u16)tab;
#pragma unroll
    for (int e = 0; e < NW; ++e) {
      const u16x2 sgn = __builtin_bit_cast(u16x2, w[e]) >> (unsigned short)15;
      const u16x2 byte = (off[e] << (unsigned short)1) + sgn * u16x2{SIGN_BYTES, SIGN_BYTES};
      b[2 * e] = *(lds_u16)(uintptr_t)(base + byte.x);
      b[2 * e + 1] = *(lds_u16)(uintptr_t)(base + byte.y);
    }
  } else {
#pragma unroll
    for (int e = 0; e < NW; ++e) {
      b[2 * e] = gelu_any(w[e] & 0xFFFFu, tab);
      b[2 * e + 1] = gelu_any(w[e] >> 16, tab);
    }
  }
}

// INT4 codes of one group row held by four lanes (lane bits 4-5 = kc, 16 values each): s =
// bf16(max|X̂| / 7) (0 below 2^-126), q = rint(X̂ · (1/s)) (|q| <= 7 by the symmetric scale). The fp32
// product is formed as in the method, and v_cvt_scalef32_2xpk16_fp6_f32 rounds y / 8 to
// nearest-even on the E2M3 subnormal grid (step 1/8), i.e. emits exactly the carrier field
// sign|00|rint(y). Its two sources interleave (field 2e = src0[e], field 2e+1 = src1[e]); fields
// 16..31 are unused. Returns the 96-bit image of the lane's 16 codes and the scale's bf16 bits.
__device__ __forceinline__ uint3 quant_int4_lane(const float (&xh)[2][8], uint32_t& s_bits) {
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
  return make_uint3((uint32_t)img[0], (uint32_t)img[1], (uint32_t)img[2]);
}

// ===================================================================================
// Kernel 1: activation side. Per row and group: X̂ = fp32(x · (1/λ)); codes + scales (W8A8: the
// row's running max|X̂| instead, written per slice for the second W8A8 pass); t += bf16(X̂)·L1
// (MFMA). One block = 64 rows (4 waves of 16) x one slice of at most QA_MAX_GS groups, so the
// slice's L1 rows are fetched once per 64 rows: they and the slice's 1/λ are copied into LDS by the
// LDS DMA path, and every wave issues the X loads of all its groups at once (buffer loads over the
// wave's rows: rows past M and groups past the slice read as zeros, so padding rows come out as zero
// codes, scales and t without any per-row select). With several slices the partial t of a slice
// goes to its own plane and t_reduce_kernel sums the planes in slice order (deterministic; a
// reduction inside one kernel would need device-scope release fences, which write back the per-XCD
// L2s). Lane (r, kc) = (lane & 15, lane >> 4) owns row r of its wave's rows and the values
// 16 kc .. 16 kc + 15 of each group; each lane reads one 1/λ value per group and the DPP row
// broadcast hands value e of its 16-lane row straight to the multiply of element e. INT4: the
// row's group maximum over its four lanes by two lane swaps, s = bf16(max/7), y = fp32(X̂ · (1/s)),
// and one FP6 conversion emits the codes of two groups (32 values) at once; MXFP4: E8M0 exponent
// and E2M1 codes. The down projection runs on 16x16x32 bf16 MFMAs with L1 from LDS.
// ===================================================================================
constexpr int QA_WAVES = QA_BLOCK_ROWS / 16;

// Exact shortcuts for the two divisions of the INT4 group quantizer. Both were checked
// exhaustively on the host against IEEE division (this file is built with fp32 denormals preserved,
// which the first one needs for tiny maxima):
//  * s = bf16(amax / 7), flushed to 0 below 2^-126: the product amax · fp32(1/7) corrected once by
//    its exact fma residual rounds to the same s as the IEEE quotient, for every finite amax >= 0;
//  * 1/s for a bf16 scale s >= 2^-126: one Newton step y0 + y0 · fma(−s, y0, 1) from any y0 within
//    one ulp of 1/s (v_rcp_f32 is) is the correctly rounded reciprocal.
__device__ __forceinline__ float int4_scale(float amax) {
  constexpr float c = 1.0f / 7.0f;
  const float q0 = amax * c;
  const float q = __builtin_fmaf(__builtin_fmaf(-7.0f, q0, amax), c, q0);
  const float s = bf16f(bf16_rne(q));
  return s >= 0x1p-126f ? s : 0.f;
}
__device__ __forceinline__ float int4_recip(float s) {  // 0 for s == 0
  const float y0 = __builtin_amdgcn_rcpf(s);
  const float y = __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
  return s != 0.f ? y : 0.f;
}

// max over the four lanes r, r+16, r+32, r+48 (one group row): two gfx950 lane swaps
__device__ __forceinline__ float max_over_kc(float m) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// max over lanes r + 16 kc and r + 16 (kc ^ 1) (the two lanes of one MX 32-block)
__device__ __forceinline__ float max_over_kc_pair(float m) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// X̂ of two groups for this lane: 2 x 16 bf16 values (two 16-byte loads each) times 1/λ, value e's
// factor taken from lane e of the lane's 16-lane row by a DPP row broadcast folded into the
// multiply. Every value is unpacked before the first multiply: a DPP instruction may not read a
// register that the previous two VALU instructions wrote.
template <int E = 0>
__device__ __forceinline__ void scale_pair(const float (&ua)[16], const float (&ub)[16], uint32_t ila, uint32_t ilb,
                                           float (&xa)[16], float (&xb)[16]) {
  if constexpr (E < 16) {
    xa[E] = ua[E] * __int_as_float(__builtin_amdgcn_mov_dpp((int)ila, 0x150 + E, 0xF, 0xF, true));
    xb[E] = ub[E] * __int_as_float(__builtin_amdgcn_mov_dpp((int)ilb, 0x150 + E, 0xF, 0xF, true));
    scale_pair<E + 1>(ua, ub, ila, ilb, xa, xb);
  }
}

template <bool GELU_IN>
__device__ __forceinline__ void unpack16(const v4i (&xv)[2], float (&u)[16], const uint16_t* gtab) {
  uint32_t bits[16];
  if constexpr (GELU_IN) {
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = (uint32_t)xv[q >> 2][q & 3];
    gelu_pk(w, bits, gtab);  // the 16 table reads go out together
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t w = (uint32_t)xv[e >> 3][(e >> 1) & 3];
      bits[e] = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) u[e] = bf16f(bits[e]);
}

// X̂ = fp32(x · (1/λ)), one fp32 multiply per value (no contraction: nothing to fuse)
template <bool GELU_IN>
__device__ __forceinline__ void smooth_pair(const v4i (&xva)[2], const v4i (&xvb)[2], uint32_t ila, uint32_t ilb,
                                            float (&xa)[16], float (&xb)[16], const uint16_t* gtab) {
  float ua[16], ub[16];
  unpack16<GELU_IN>(xva, ua, gtab);
  unpack16<GELU_IN>(xvb, ub, gtab);
  scale_pair(ua, ub, ila, ilb, xa, xb);
}

// LDS of one block in 16-byte slots: 1/λ, L1 rows of RP rank columns padded by one slot, and with
// the GELU on load its table, in whole 64-slot DMA instructions
constexpr int qa_lds_slots(int rp, int gs, bool gelu = false) {
  return (gs * 16 + rp * (gs * 8 + 1) + (gelu ? GELU_SLOTS : 0) + 63) / 64 * 64;
}

template <int FMT, int NT, bool GELU_IN = false>  // NT = rank_pad / 16 (0 when there is no low-rank branch)
__global__ __launch_bounds__(QA_WAVES * 64) void quantize_act_kernel(
    const uint16_t* X, int M, int K, int ldx, const float* __restrict__ inv_lambda,
    const uint16_t* __restrict__ l1t, int m_pad, int gs, uint8_t* __restrict__ xq, void* __restrict__ xscale,
    float* __restrict__ xl1) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int RP = NT * 16, NTA = NT > 0 ? NT : 1;
  const int G = K / W4A4_GROUP;
  const int nsl = (G + gs - 1) / gs;
  const int rb = blockIdx.x / nsl, sl = blockIdx.x % nsl;
  const int g0 = sl * gs, ng = min(gs, G - g0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kc = lane >> 4;
  const int row0 = rb * QA_BLOCK_ROWS + wave * 16, row = row0 + r;

  // ---- 1. 1/λ and L1 rows of the slice -> LDS. Slot s (16 B) of the block's LDS: s < 16 ng are
  // 1/λ; then rank row c uses slots [16 ng + c (8 ng + 1), +8 ng + 1) for k = 64 g0 .. 64 (g0 + ng),
  // the last one padding. Each DMA instruction fills 64 consecutive slots.
  // With the GELU on load its table follows: slots [n_l1, n_l1 + GELU_SLOTS).
  const int n_il = ng * 16, l1_row = ng * 8 + 1, n_l1 = n_il + RP * l1_row;
  const int n_all = n_l1 + (GELU_IN ? GELU_SLOTS : 0);
  for (int s0 = wave * 64; s0 < n_all; s0 += QA_WAVES * 64) {
    const int s = s0 + lane;
    const void* src = inv_lambda + (size_t)g0 * W4A4_GROUP + 4 * min(s, n_il - 1);
    if (NT > 0 && s >= n_il && s < n_l1) {
      const int c = (s - n_il) / l1_row, j = (s - n_il) % l1_row;
      src = l1t + (size_t)c * K + (size_t)g0 * W4A4_GROUP + 8 * (j < ng * 8 ? j : 0);
    }
    if (GELU_IN && s >= n_l1) src = gelu_tab + 8 * min(s - n_l1, GELU_SLOTS - 1);
    __builtin_amdgcn_global_load_lds(src, smem + 16 * s0, 16, 0, 0);
  }

  // ---- 2. X of every group of the slice, straight into registers: exactly 2 * QA_MAX_GS buffer
  // loads per wave after the DMA (rows past M and groups past the slice read as zeros), so
  // vmcnt(2 QA_MAX_GS) means the DMA has landed while the X loads may still be in flight. Every part
  // of the resource is wave-uniform; readfirstlane keeps it in scalar registers.
  const int valid = __builtin_amdgcn_readfirstlane(max(0, min(16, M - row0)));
  const uint64_t xbase = reinterpret_cast<uint64_t>(valid > 0 ? X + (size_t)row0 * ldx : X);
  const uint64_t xb_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xbase);
  const uint64_t xb_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(xbase >> 32));
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(xb_lo | (xb_hi << 32)), 0, __builtin_amdgcn_readfirstlane(valid * ldx * 2), 0x00020000);
  constexpr int OOB = 0x7FFFFF00;  // an offset past every buffer: loads read zeros, stores are dropped
  v4i xv[QA_MAX_GS][2];
#pragma unroll
  for (int i = 0; i < QA_MAX_GS; ++i) {
    const int off = i < ng ? (r * ldx + (g0 + i) * W4A4_GROUP + kc * 16) * 2 : OOB;
    xv[i][0] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    xv[i][1] = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 16, 0, 0);
  }
  asm volatile("" ::: "memory");  // the loads stay ahead of the wait that counts them
  wait_vmcnt<2 * QA_MAX_GS>();
  __builtin_amdgcn_s_barrier();
  const uint32_t* s_il = reinterpret_cast<const uint32_t*>(smem);
  const uint8_t* s_l1 = smem + 16 * n_il;
  const int l1_stride = 16 * l1_row;
  const uint16_t* s_gelu = reinterpret_cast<const uint16_t*>(smem + 16 * n_l1);

  // the outputs as buffers: a store whose offset lies past the buffer is dropped, so a pair without
  // its second group needs no branch
  const int G2 = FMT == W4A4_FMT_MXFP4_B32 ? 2 * G : G;  // scale planes
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc(xq, 0, G * m_pad * (FMT == W4A4_FMT_INT4_G64 ? 48 : 32), 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      xscale, 0, FMT == W4A4_FMT_W8A8 ? 0 : G2 * m_pad * (FMT == W4A4_FMT_INT4_G64 ? 2 : 1), 0x00020000);

  v4f acc[NTA];
#pragma unroll
  for (int c = 0; c < NTA; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
  float row_amax = 0.f;  // W8A8: running max|X̂| of the lane's values
  // t += bf16(X̂)·L1 for group i of the slice: the lane's 8 values of half h are the A operand's k
  // slots 8 (lane / 16) .., paired with the same k of L1 (from LDS) in the B operand
  auto down = [&](const float (&xh)[16], int i) {
    if constexpr (NT > 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4i a;
#pragma unroll
        for (int d = 0; d < 4; ++d) a[d] = (int)pack_bf16x2(xh[8 * h + 2 * d], xh[8 * h + 2 * d + 1]);
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          const v4i b = *reinterpret_cast<const v4i*>(s_l1 + (c * 16 + r) * l1_stride + i * 128 + kc * 32 + 16 * h);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), acc[c], 0, 0, 0);
        }
      }
    }
  };

#pragma unroll
  for (int i = 0; i < QA_MAX_GS; i += 2) {
    if (i >= ng) break;  // block-uniform
    const bool two = i + 1 < ng;
    const int ga = g0 + i, gb = ga + 1;
    // this lane's 1/λ of both groups (a missing second group reads the first's: its X is zero)
    const uint32_t ila = s_il[i * W4A4_GROUP + kc * 16 + r];
    const uint32_t ilb = s_il[min(i + 1, ng - 1) * W4A4_GROUP + kc * 16 + r];
    float xa[16], xb[16];  // group gb is all zeros when the slice has no such group
    smooth_pair<GELU_IN>(xv[i], xv[i + 1], ila, ilb, xa, xb, s_gelu);
    if constexpr (FMT == W4A4_FMT_INT4_G64) {
      float ma = 0.f, mb = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ma = fmaxf(ma, fabsf(xa[e]));
        mb = fmaxf(mb, fabsf(xb[e]));
      }
      const float sa = int4_scale(max_over_kc(ma)), sb = int4_scale(max_over_kc(mb));
      const float ia = int4_recip(sa), ib = int4_recip(sb);
      // y = X̂ · (1/s); v_cvt_scalef32_2xpk16_fp6_f32 rounds y / 8 to nearest-even on the E2M3
      // subnormal grid (step 1/8), i.e. emits the carrier field sign|00|rint(y) (|y| < 7.5 by the
      // symmetric scale). Sources interleave: field 2e = src0[e], field 2e+1 = src1[e]; fields
      // 0..15 are group a's values, 16..31 group b's.
      v16f ev, od;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ev[e] = xa[2 * e] * ia;
        od[e] = xa[2 * e + 1] * ia;
        ev[8 + e] = xb[2 * e] * ib;
        od[8 + e] = xb[2 * e + 1] * ib;
      }
      const v6i img = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, 8.0f);
      // the even-kc lane of each pair (lanes r + 16 kc, r + 16 (kc + 1)) stores the main part, the
      // odd one the extra part: one lane swap brings the odd run's first dword to its partner
      // (the swap's second result holds, in the even rows of 16 lanes, the odd rows' values)
      const bool main_lane = (kc & 1) == 0;
      const auto pa = __builtin_amdgcn_permlane16_swap(img[0], img[0], false, false);
      const auto pb = __builtin_amdgcn_permlane16_swap(img[3], img[3], false, false);
      const int oa = int4_part_offset(ga, row, m_pad, K, kc), ob = two ? int4_part_offset(gb, row, m_pad, K, kc) : OOB;
      __builtin_amdgcn_raw_buffer_store_b128(v4i{img[0], img[1], img[2], (int)pa[1]}, qr, main_lane ? oa : OOB, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(v2i{img[1], img[2]}, qr, main_lane ? OOB : oa, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{img[3], img[4], img[5], (int)pb[1]}, qr, main_lane ? ob : OOB, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(v2i{img[4], img[5]}, qr, main_lane ? OOB : ob, 0, 0);
      // the four lanes of a row store the same scale
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_rne(sa), sr, (ga * m_pad + row) * 2, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_rne(sb), sr, two ? (gb * m_pad + row) * 2 : OOB, 0, 0);
    } else if constexpr (FMT == W4A4_FMT_MXFP4_B32) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // both groups computed (b is zeros when missing), stores dropped then
        const float (&xh)[16] = j ? xb : xa;
        const int g = ga + j;
        // the lane's 16 values lie in 32-block kc / 2, shared with lane kc ^ 1
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(xh[e]));
        amax = max_over_kc_pair(amax);
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
          for (int e = 0; e < 8; ++e) z[e] = ldexpf(xh[8 * h + e], -e8);
          word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[0], z[1], 1.0f, 0);
          word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[2], z[3], 1.0f, 1);
          word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[4], z[5], 1.0f, 2);
          word[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[h], z[6], z[7], 1.0f, 3);
        }
        const bool live = j == 0 || two;
        __builtin_amdgcn_raw_buffer_store_b64(v2i{(int)word[0], (int)word[1]}, qr,
                                              live ? (g * m_pad + row) * 32 + kc * 8 : OOB, 0, 0);
        // lanes kc and kc ^ 1 store the same exponent byte of their block
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(e8 + 127), sr,
                                             live ? (2 * g + (kc >> 1)) * m_pad + row : OOB, 0, 0);
      }
    } else {  // W8A8: only the row maximum here; the codes need all of K
#pragma unroll
      for (int e = 0; e < 16; ++e) row_amax = fmaxf(row_amax, fmaxf(fabsf(xa[e]), fabsf(xb[e])));
    }
    down(xa, i);
    if (two) down(xb, i + 1);
  }
  if constexpr (FMT == W4A4_FMT_W8A8) {
    // the row's maximum over this slice -> plane sl of the partial maxima behind the scales
    row_amax = max_over_kc(row_amax);
    if (kc == 0) static_cast<float*>(xscale)[(size_t)m_pad * (1 + sl) + row] = row_amax;
  }
  if (NT > 0) {
    // 16x16 MFMA output: lane holds rank column c*16 + lane%16, rows 4*(lane/16) + v of the tile
    const size_t n = (size_t)m_pad * RP;
    float* dst = xl1 + (nsl > 1 ? n * (1 + sl) : 0) + (size_t)row0 * RP;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[(4 * kc + v) * RP + c * 16 + r] = acc[c][v];
  }
}

// t = Σ_slices partial t, summed in slice order (deterministic); n = m_pad * rank_pad floats.
// One float4 per thread; the loads of up to TR_PLANES planes are issued together (one memory round
// trip for the usual slice counts).
constexpr int TR_PLANES = 8;
__global__ __launch_bounds__(256) void t_reduce_kernel(const float* __restrict__ part, int nsl, int n,
                                                       float* __restrict__ t) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= n) return;
  auto ld = [&](int k) { return *reinterpret_cast<const float4*>(part + (size_t)k * n + i); };
  float4 s = ld(0);
  for (int k0 = 1; k0 < nsl; k0 += TR_PLANES) {
    float4 v[TR_PLANES];
#pragma unroll
    for (int k = 0; k < TR_PLANES; ++k)
      if (k0 + k < nsl) v[k] = ld(k0 + k);
#pragma unroll
    for (int k = 0; k < TR_PLANES; ++k)
      if (k0 + k < nsl) {
        s.x += v[k].x;
        s.y += v[k].y;
        s.z += v[k].z;
        s.w += v[k].w;
      }
  }
  *reinterpret_cast<float4*>(t + i) = s;
}

// ===================================================================================
// Kernel 2: the INT4 GEMM + low-rank up projection (+ bias), bf16 out.
//
// Block tile 256 (M) x 256 (N), 8 waves as 2 (M) x 4 (N); each wave owns a 4 x 2 grid of 32x32
// tiles. One K step = one 64-wide group. The codes (FP6 images: a 16-byte main and an 8-byte
// extra part per row and half) and scales of each group are copied global -> LDS by the LDS DMA
// path (buffer_load ... lds) into a ring of I4_RING slots, issued four groups before their first
// reader; one barrier per two groups publishes the next slots. Per group each wave reads its A and
// B operands as they are (one 16-byte and one 8-byte LDS read each, no unpacking) and runs, per
// tile, one FP6 MFMA with E8M0 scales 2^3 x 2^3 (the exact integer dot product of the group), one
// bf16 MFMA (the exact outer product s_x s_w of the raw bf16 scales) and 16 FMAs into its fp32
// accumulators.
// The epilogue adds bf16(t)·L2 and the bias and writes Y through LDS in 16-byte row segments.
// ===================================================================================
constexpr int I4_THREADS = 512;

// One ring slot: the codes of 256 A rows and 256 B rows of one group, main parts (32 B per row,
// halves swizzled) and extra parts ([half][row][8 B]), and their bf16 scales (A rows 0..255, then
// B rows). Each slot is its own LDS object, so the compiler can tell the DMA writes into one slot
// from the reads of another. Six slots (150 KB) fill the CU's LDS.
constexpr int I4_RING = 6;  // even: one barrier per two groups
struct I4Slot {
  uint8_t a[256 * 32];
  uint8_t b[256 * 32];
  uint8_t ax[2 * 256 * 8];
  uint8_t bx[2 * 256 * 8];
  uint16_t s[512];
  uint16_t z[32];  // zeros (never written by the DMA): k > 0 half of the scale outer-product operand
};
// After the main loop every wave stages its output through half a slot (wave w: slot w / 2)
constexpr int I4_STAGE = 12800;
static_assert(2 * I4_STAGE <= (int)sizeof(I4Slot) && I4_THREADS / 64 <= 2 * I4_RING, "staging areas");

// The next layer's activation side in this GEMM's epilogue (the MLP's fc1 -> GELU -> fc2 join):
// fc2's 1/λ over this layer's N columns, fc2's L1ᵀ [rank2_pad][N], and fc2's outputs in library
// layout: INT4 codes (FP6 images of K = N), bf16 scales [N/64][m_pad], and one partial t plane
// [m_pad][rank2_pad] per 256-column tile of this layer.
struct GeluQuantArgs {
  const float* il2;
  const uint16_t* l1t2;
  uint8_t* xq2;
  uint16_t* xs2;
  float* t2part;
};

// the eight waves' staging areas, by value (indexed with constants only, so they stay in registers)
struct SlotSet {
  uint8_t* s[8];
};

template <int NT2>
__device__ __forceinline__ void gelu_quant_epilogue(v16f (&acc)[I4_MT][2], uint8_t* stage, SlotSet slots,
                                                    const uint16_t* gtab, const GeluQuantArgs& fa,
                                                    const uint16_t* bias, int M, int N, int m_pad, int m0, int n0,
                                                    int tn, int wm, int wn, int wave, int lane);

// FUSE < 0: the plain GEMM (fa unused). FUSE >= 0 (INT4 only): fc1 of the MLP with fc2's
// activation side in the epilogue, FUSE = fc2's rank_pad / 16; Y may then be NULL.
template <int FMT, int NTR, int FUSE = -1>  // NTR = rank_pad / 16
__global__ __launch_bounds__(I4_THREADS) void gemm_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, const float* __restrict__ xl1,
    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ ws, const uint16_t* __restrict__ l2t,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int ldy, int M, int N, int K,
    int m_pad, int n_pad, GeluQuantArgs fa) {
  static_assert(FMT == W4A4_FMT_INT4_G64, "MXFP4 runs on gemm_mx_small_kernel and gemm_w8a8_kernel<., true>");
  static_assert(I4_RING == 6, "six ring objects");
  __shared__ __attribute__((aligned(16))) I4Slot sl0, sl1, sl2, sl3, sl4, sl5;
  I4Slot* const ring[I4_RING] = {&sl0, &sl1, &sl2, &sl3, &sl4, &sl5};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps derived addresses scalar
  const int wm = wave >> 2, wn = wave & 3;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, m_pad / I4_BM, n_pad / I4_BN, tm, tn);
  const int m0 = tm * I4_BM, n0 = tn * I4_BN;
  const int G = K / W4A4_GROUP;

  // ---- DMA sources. Instruction w of an operand's main parts fills LDS bytes [1024 w, +1024) of the
  // slot, lane i the 16 bytes at 1024 w + 16 i = row 32 w + i / 2, stored half i & 1; the lane
  // loads the global half that the swizzle puts there. Extra parts: wave w < 4 copies quarter w of
  // A's 4 KB ([half][row][8 B]: half w / 2, rows 128 (w & 1) ..), wave w >= 4 quarter w - 4 of B's.
  // Scales: wave w copies 256 bytes, chunk w & 3 of the slot's 1 KB of scales (waves w and w + 4
  // write the same bytes): the bf16 scales of A rows 0..127, A rows 128..255, B rows 0..127,
  // B rows 128..255.
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
  // extra parts: planes [2 G][rows_pad][8 B] behind the main planes
  const bool x_is_a = wave < 4;
  const int x_rows = x_is_a ? m_pad : n_pad, x_row0 = x_is_a ? m0 : n0, xq4 = wave & 3;
  const uint8_t* x_buf = (x_is_a ? xq : wq) + (size_t)x_rows * (K / 2);
  const __amdgpu_buffer_rsrc_t x_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(x_buf + (size_t)x_row0 * 8), 0, (2 * G * x_rows - x_row0) * 8, RSRC_W3);
  const int x_lane = (xq4 >> 1) * x_rows * 8 + (xq4 & 1) * 1024 + 16 * lane;  // half, row block, lane
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
  // 4 vector-memory instructions per wave and group (part 0: A main parts, 1: B main parts,
  // 2: scales, 3: extra parts); groups past the end reload the last group
  constexpr int DMA_PER_GROUP = 4;
  auto dma_part = [&](int part, int g, I4Slot* sl) {
    g = min(g, G - 1);
    if (part == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sl->a + 1024 * wave), 16, c_lane, g * m_pad * 32, 0, 0);
    else if (part == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sl->b + 1024 * wave), 16, c_lane, g * n_pad * 32, 0, 0);
    else if (part == 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(s_rsrc, (lds_ptr)(sl->s + 128 * sblk), 4, s_lane, g * s_gstride, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rsrc, (lds_ptr)((x_is_a ? sl->ax : sl->bx) + 1024 * xq4), 16, x_lane,
                                               g * 2 * x_rows * 8, 0, 0);
  };
  auto dma = [&](int g, I4Slot* sl) {
#pragma unroll
    for (int part = 0; part < DMA_PER_GROUP; ++part) dma_part(part, g, sl);
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
  // 4-bit groups then accumulate on top. Up to rank 48 the block's t tile (256 rows x rank_pad
  // fp32, at most 48 KB, read by four waves each) is copied once into the last two ring slots by
  // the LDS DMA path before the ring's first groups, and the L2 operands are loaded before them
  // too; all of it lands under the prologue's wait for group 0 and the MFMAs run right after it.
  // Larger ranks load t directly, 32 ranks at a time.
  constexpr int RP = NTR * 16, KS = 2;  // up to two 16-rank MFMA K-steps per batch of loads
  constexpr bool T_LDS = NTR > 0 && NTR <= 3;
  constexpr int TROWB = RP * 4;          // bytes of one t row
  constexpr int TSPLIT = 128 * TROWB;    // rows 0..127 of the tile in slot 4, rows 128..255 in slot 5
  static_assert(!T_LDS || TSPLIT <= (int)offsetof(I4Slot, z), "half the t tile fits a slot below its zero words");
  auto t_row_ptr = [&](int r) -> const uint8_t* {
    const int byte = r * TROWB;
    return byte < TSPLIT ? reinterpret_cast<const uint8_t*>(ring[I4_RING - 2]) + byte
                         : reinterpret_cast<const uint8_t*>(ring[I4_RING - 1]) + (byte - TSPLIT);
  };
  // Within a staged t row, 16-byte chunk c sits at chunk position c ^ t_chunk_sw(r) (LDS banks)
  constexpr int TCH = T_LDS ? TROWB / 16 : 1;  // chunks per t row
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
  // t from its LDS tile, ranks k0 .. k0 + 31 (one or two 16-rank K-steps): one asm block with
  // every read and its own wait (the compiler's LDS-DMA tracking cannot tell slots 4/5 from the
  // ring groups still in flight and would wait for all of them). The lane's rows i = 0..3 (32
  // apart, one slot) share the chunk swizzle t_chunk_sw(lr): one address per chunk, the rows as
  // immediate offsets RS·i. Chunk of (K-step s, half h): k0 / 4 + 4 s + 2 lh + h.
  auto t_from_lds = [&](int k0) {
    typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
    constexpr int RS = 32 * TROWB;  // bytes from row i to row i + 1 of the lane
    const uint32_t row0 = (uint32_t)(uintptr_t)(lds_cptr)t_row_ptr(wm * 128 + lr);
    const int x = t_chunk_sw<RP>(lr), cb = k0 / 4 + 2 * lh;
    uint32_t ad[4];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) ad[ci] = row0 + 16 * ((cb + (ci & 1) + 4 * (ci >> 1)) ^ x);
    if (RP - k0 >= 32) {
      asm volatile(
          "ds_read_b128 %0, %16\n\tds_read_b128 %4, %16 offset:%c20\n\t"
          "ds_read_b128 %8, %16 offset:%c21\n\tds_read_b128 %12, %16 offset:%c22\n\t"
          "ds_read_b128 %1, %17\n\tds_read_b128 %5, %17 offset:%c20\n\t"
          "ds_read_b128 %9, %17 offset:%c21\n\tds_read_b128 %13, %17 offset:%c22\n\t"
          "ds_read_b128 %2, %18\n\tds_read_b128 %6, %18 offset:%c20\n\t"
          "ds_read_b128 %10, %18 offset:%c21\n\tds_read_b128 %14, %18 offset:%c22\n\t"
          "ds_read_b128 %3, %19\n\tds_read_b128 %7, %19 offset:%c20\n\t"
          "ds_read_b128 %11, %19 offset:%c21\n\tds_read_b128 %15, %19 offset:%c22\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[1][0][0]), "=&v"(tv[1][0][1]),
            "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1]), "=&v"(tv[1][1][0]), "=&v"(tv[1][1][1]),
            "=&v"(tv[0][2][0]), "=&v"(tv[0][2][1]), "=&v"(tv[1][2][0]), "=&v"(tv[1][2][1]),
            "=&v"(tv[0][3][0]), "=&v"(tv[0][3][1]), "=&v"(tv[1][3][0]), "=&v"(tv[1][3][1])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(RS), "i"(2 * RS), "i"(3 * RS)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %2, %8 offset:%c10\n\t"
          "ds_read_b128 %4, %8 offset:%c11\n\tds_read_b128 %6, %8 offset:%c12\n\t"
          "ds_read_b128 %1, %9\n\tds_read_b128 %3, %9 offset:%c10\n\t"
          "ds_read_b128 %5, %9 offset:%c11\n\tds_read_b128 %7, %9 offset:%c12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1]),
            "=&v"(tv[0][2][0]), "=&v"(tv[0][2][1]), "=&v"(tv[0][3][0]), "=&v"(tv[0][3][1])
          : "v"(ad[0]), "v"(ad[1]), "i"(RS), "i"(2 * RS), "i"(3 * RS)
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
  v4i LBn[2] = {};  // staged t above rank 32: the L2 operands of ranks 32 .. 47, loaded up front too
  if constexpr (T_LDS && NTR > 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      LBn[j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + wn * 64 + j * 32 + lr) * RP + 32 + 8 * lh);
  }
  if constexpr (T_LDS) {  // t tile -> the last two slots: TBYTES / 8 bytes per wave, 1 KB per DMA instruction
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(xl1 + (size_t)m0 * RP), 0, (m_pad - m0) * TROWB, RSRC_W3);
    constexpr int TCHUNK = 256 * TROWB / 8;
    static_assert(TCHUNK % 1024 == 0 && TSPLIT % 1024 == 0, "whole DMA instructions, none across the split");
#pragma unroll
    for (int q = 0; q < TCHUNK / 1024; ++q) {
      const int off = wave * TCHUNK + q * 1024;
      uint8_t* dst = off < TSPLIT ? reinterpret_cast<uint8_t*>(ring[I4_RING - 2]) + off
                                  : reinterpret_cast<uint8_t*>(ring[I4_RING - 1]) + (off - TSPLIT);
      // lane: LDS chunk position p of tile row r gets the row's chunk p ^ t_chunk_sw(r)
      const int slot = off / 16 + lane, r = slot / TCH, pc = slot % TCH;
      const int src = r * TROWB + 16 * (pc ^ t_chunk_sw<RP>(r));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t_rsrc, (lds_ptr_t)dst, 16, src, 0, 0, 0);
    }
  }

  // prologue: zero words of every slot; groups 0 .. NS-3 in flight; group 0 visible
  if (tid < 32) {
#pragma unroll
    for (int s = 0; s < I4_RING; ++s) ring[s]->z[tid] = 0;
  }
#pragma unroll
  for (int s = 0; s < I4_RING - 2; ++s) dma(s, ring[s]);
  wait_vmcnt<DMA_PER_GROUP * (I4_RING - 3)>();
  __builtin_amdgcn_s_barrier();
  if (NTR > 0) {
    if constexpr (T_LDS) t_from_lds(0);
    lr_mfma(0);
#pragma unroll
    for (int k0 = 32; k0 < RP; k0 += 32) {
      if constexpr (T_LDS) {
        LB[0][0] = LBn[0];
        LB[0][1] = LBn[1];
        t_from_lds(k0);
      } else {
        lr_load(k0);
      }
      lr_mfma(k0);
    }
  }
  // an operand as it sits in LDS: the 16-byte main part and the 8-byte extra part of the lane's half
  struct Raw {
    v4i m;
    v2i x;
  };
  auto op6 = [](const Raw& r) { return v8i{r.m[0], r.m[1], r.m[2], r.m[3], r.x[0], r.x[1], 0, 0}; };
  const int bx_off = lh * 2048 + bcol0 * 8;
  auto b_raw = [&](const I4Slot* sl, int j) {
    return Raw{*reinterpret_cast<const v4i*>(sl->b + b_off + 1024 * j), *reinterpret_cast<const v2i*>(sl->bx + bx_off + 256 * j)};
  };
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
  const int ax_off4 = lh * 2048 + (wm * 128 + rot(lr, 2)) * 8;
  const int srow0 = wm * 128 + rot(lr, 1);
  auto a_raw4 = [&](const I4Slot* sl, int i) {
    return Raw{*reinterpret_cast<const v4i*>(sl->a + a_off4 + 1024 * i), *reinterpret_cast<const v2i*>(sl->ax + ax_off4 + 256 * i)};
  };
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
  Raw An_raw, Bn_raw[2];
  uint32_t OAn, OBn[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    Bv[j] = op6(b_raw(ring[0], j));
    OB[j] = sb_val(ring[0], j, true);
  }
  Av = op6(a_raw4(ring[0], 0));
  OA = sa_val(ring[0], srow0);
  An_raw = a_raw4(ring[0], 1);
  OAn = sa_val(ring[0], srow0 + 32);

  constexpr int T = 2 * I4_MT;
  v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Av, Bv[0], zero16, 2, 2, 0, 130, 0, 130);
  v16f sc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(sc_op(OA), sc_op(OB[0]), zero16, 0, 0, 0);

  for (int g0 = 0; g0 < G; g0 += I4_RING) {
#pragma unroll
    for (int u = 0; u < I4_RING; ++u) {
      const int g = g0 + u;
      const I4Slot* cur = ring[u];
      const I4Slot* nxt = ring[(u + 1) % I4_RING];
      if (u % 2 == 0) {
        // groups g+1 and g+2 have landed in every wave's share of their slots; everyone is done
        // with slots g-2 and g-1, which take groups g+NS-2 (copied during this group) and g+NS-1
        // (during the next)
        wait_vmcnt<DMA_PER_GROUP * (I4_RING - 5)>();
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
            Bv[jj] = op6(Bn_raw[jj]);
            OB[jj] = OBn[jj];
          }
        }
        if (j1 == 0) {  // new tile row: take the prefetched A operand
          Av = op6(An_raw);
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
        // this group's copy of group g + I4_RING - 2 into the slot freed at the last barrier, one
        // instruction every other tile (issued together right after the barrier, the copies of all
        // eight waves queue up at once and stall their issue: measured 5-7% slower)
        if (t & 1) dma_part(t >> 1, g + I4_RING - 2, ring[(u + I4_RING - 2) % I4_RING]);
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
  const uint16_t* gtab = reinterpret_cast<const uint16_t*>(ring[4]);
  if constexpr (FUSE >= 0) {  // the GELU table into slot 4, idle from here on (1 KB per instruction)
    static_assert(GELU_SLOTS * 16 <= (int)sizeof(I4Slot) && GELU_SLOTS <= 16 * 64, "GELU table fits slot 4");
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = wave + 8 * q;
      if (c * 64 < GELU_SLOTS)
        __builtin_amdgcn_global_load_lds(gelu_tab + 8 * min(c * 64 + lane, GELU_SLOTS - 1),
                                         reinterpret_cast<uint8_t*>(ring[4]) + 1024 * c, 16, 0, 0);
    }
  }
  // the eight waves' staging areas: wave w uses half (w & 1) of slot w / 2
  SlotSet slots;
#pragma unroll
  for (int w = 0; w < 8; ++w) slots.s[w] = reinterpret_cast<uint8_t*>(ring[w >> 1]) + (w & 1) * I4_STAGE;
  uint8_t* stage = slots.s[0];
#pragma unroll
  for (int w = 1; w < 8; ++w)
    if (wave == w) stage = slots.s[w];  // wave-uniform select
  static_assert(64 * Y_ES <= I4_STAGE, "staging fits half a ring slot");
  if constexpr (FUSE < 0) {
    store_y(acc, stage, bias, Y, ldy, M, N, m0 + wm * 128, n0 + wn * 64, lane);
  } else {
    if (Y) store_y(acc, stage, bias, Y, ldy, M, N, m0 + wm * 128, n0 + wn * 64, lane);  // for checking
    gelu_quant_epilogue<FUSE>(acc, stage, slots, gtab, fa, bias, M, N, m_pad, m0, n0, tn, wm, wn, wave, lane);
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
                                                    const uint16_t* gtab, const GeluQuantArgs& fa,
                                                    const uint16_t* bias, int M, int N, int m_pad, int m0, int n0,
                                                    int tn, int wm, int wn, int wave, int lane) {
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
  wait_vmcnt<0>();               // this wave's copies of the GELU table have landed
  __builtin_amdgcn_s_barrier();  // and every other wave's
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // the half's 64 GELU values per lane: every table read issued before the first is used (the
    // reads are unconditional; rows past M are zeroed afterwards)
    uint32_t gx[2][2][16];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // one 32 x 32 tile (16 values of the lane) at a time
        uint32_t yw[8];
#pragma unroll
        for (int v = 0; v < 16; v += 2)
          yw[v / 2] = pack_bf16x2(acc[2 * half + ii][j][v] + bcol[j], acc[2 * half + ii][j][v + 1] + bcol[j]);
        gelu_pk(yw, gx[ii][j], gtab);
      }
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int rl = ii * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          const int grow = m0 + wm * 128 + half * 64 + rl;  // rows grow, grow + 1
          uint16_t* d = reinterpret_cast<uint16_t*>(stage + rl * Y_ES + (j * 32 + lr) * 2);
          d[0] = (uint16_t)(grow < M ? gx[ii][j][v] : 0u);
          d[Y_ES / 2] = (uint16_t)(grow + 1 < M ? gx[ii][j][v + 1] : 0u);
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
      const uint3 q = quant_int4_lane(xh, sb);
      if (gvalid) {  // wave-uniform: every lane takes part in the lane swap
        // even-kc lanes store the 16-byte main part (with the odd partner's first dword), odd-kc
        // lanes the 8-byte extra part
        const auto pq = __builtin_amdgcn_permlane16_swap(q.x, q.x, false, false);
        uint8_t* const dst = fa.xq2 + int4_part_offset(g2, row, m_pad, N, kc);
        if ((kc & 1) == 0)
          *reinterpret_cast<uint4*>(dst) = make_uint4(q.x, q.y, q.z, pq[1]);
        else
          *reinterpret_cast<uint2*>(dst) = make_uint2(q.y, q.z);
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
    // 16x16 MFMA output: lane holds rank column c*16 + lane%16, rows 4*(lane/16) + v of its pass.
    // The partials go through the waves' staging areas 64 rows (of each wave's 128) at a time.
    float* mine = reinterpret_cast<float*>(stage);
    static_assert(64 * RP2 * 4 <= I4_STAGE, "64 rows of a wave's partial t fit its staging area");
    const int tid = wave * 64 + lane;
    constexpr int Q = RP2 / 4;  // float4 per row
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      __builtin_amdgcn_s_barrier();  // every wave is done with the staging areas
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int c = 0; c < NT2; ++c)
#pragma unroll
          for (int v = 0; v < 4; ++v) mine[(p * 16 + 4 * kc + v) * RP2 + c * 16 + r] = tacc[4 * hp + p][c][v];
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int idx0 = 0; idx0 < 128 * Q; idx0 += I4_THREADS) {
        const int idx = idx0 + tid, row = idx / Q, q = idx % Q;
        const int wr = row >> 6, lrow = row & 63;
        float4 sum = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // the four column waves of these rows, in order
          // (a select between constant indices: a run-time index would put the array in scratch)
          const float* src = reinterpret_cast<const float*>(wr ? slots.s[4 + w] : slots.s[w]);
          const float4 v = *reinterpret_cast<const float4*>(src + lrow * RP2 + 4 * q);
          sum.x += v.x;
          sum.y += v.y;
          sum.z += v.z;
          sum.w += v.w;
        }
        const int brow = wr * 128 + hp * 64 + lrow;  // row within the block
        *reinterpret_cast<float4*>(fa.t2part + ((size_t)tn * m_pad + m0 + brow) * RP2 + 4 * q) = sum;
      }
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
  // Up to rank 32 the block's t tile (128 rows x rank_pad fp32, at most 16 KB) is copied by the
  // LDS DMA path into slots 6 and 7 (rows 0..63 and 64..127), idle until the main loop's first
  // copies; larger ranks load t directly.
  constexpr bool T_LDS = NTR > 0 && NTR <= 2;
  constexpr int TROWB = RP * 4;
  constexpr int TCH = T_LDS ? TROWB / 16 : 1;  // 16-byte chunks per t row
  static_assert(!T_LDS || 64 * TROWB <= (int)sizeof(MxSlot), "half the t tile fits a slot");
  auto lr_load = [&](int k0) {  // L2 operands, and t when it is not staged in LDS
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = k0 + 16 * s;
      if (kk >= RP) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        LB[s][j] = *reinterpret_cast<const v4i*>(l2t + (size_t)(n0 + bcol0 + j * 32) * RP + kk + 8 * lh);
      if (!T_LDS) {
#pragma unroll
        for (int i = 0; i < MX_MT; ++i) {
          const float* tp = xl1 + (size_t)(m0 + arow0 + i * 32) * RP + kk + 8 * lh;
          tv[s][i][0] = *reinterpret_cast<const float4*>(tp);
          tv[s][i][1] = *reinterpret_cast<const float4*>(tp + 4);
        }
      }
    }
  };
  // t from its LDS tile: one asm block with every read and its own wait (the compiler's LDS-DMA
  // tracking cannot tell slots 6/7 from the ring groups still in flight and would wait for all of
  // them). The lane's rows wm * 64 + lr + 32 i (i = 0, 1: one slot, 32 rows apart) share the chunk
  // swizzle t_chunk_sw(lr): one address per chunk, the second row as an immediate offset. Chunk
  // of (K-step s, half h): 4 s + 2 lh + h.
  auto t_from_lds = [&]() {
    typedef __attribute__((address_space(3))) const uint8_t* lds_cptr;
    constexpr int RS = 32 * TROWB;  // bytes from row i = 0 to row i = 1 of the lane
    const uint8_t* slot = reinterpret_cast<const uint8_t*>(wm ? ring[7] : ring[6]);
    const uint32_t row0 = (uint32_t)(uintptr_t)(lds_cptr)(slot + lr * TROWB);
    const int x = t_chunk_sw<RP>(lr);
    uint32_t ad[4];
#pragma unroll
    for (int ci = 0; ci < 4; ++ci) ad[ci] = row0 + 16 * ((2 * lh + (ci & 1) + 4 * (ci >> 1)) ^ x);
    if constexpr (NTR == 2) {
      asm volatile(
          "ds_read_b128 %0, %8\n\tds_read_b128 %4, %8 offset:%c12\n\t"
          "ds_read_b128 %1, %9\n\tds_read_b128 %5, %9 offset:%c12\n\t"
          "ds_read_b128 %2, %10\n\tds_read_b128 %6, %10 offset:%c12\n\t"
          "ds_read_b128 %3, %11\n\tds_read_b128 %7, %11 offset:%c12\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[1][0][0]), "=&v"(tv[1][0][1]),
            "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1]), "=&v"(tv[1][1][0]), "=&v"(tv[1][1][1])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(RS)
          : "memory");
    } else if constexpr (NTR == 1) {
      asm volatile(
          "ds_read_b128 %0, %4\n\tds_read_b128 %2, %4 offset:%c6\n\t"
          "ds_read_b128 %1, %5\n\tds_read_b128 %3, %5 offset:%c6\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(tv[0][0][0]), "=&v"(tv[0][0][1]), "=&v"(tv[0][1][0]), "=&v"(tv[0][1][1])
          : "v"(ad[0]), "v"(ad[1]), "i"(RS)
          : "memory");
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
  if constexpr (T_LDS) {  // t tile -> slots 6 and 7: 16 * TROWB bytes per wave, 1 KB per DMA instruction
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const __amdgpu_buffer_rsrc_t t_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(xl1 + (size_t)m0 * RP), 0, (m_pad - m0) * TROWB, RSRC_W3);
    constexpr int TCHUNK = 128 * TROWB / 4;  // wave w: rows 32 w .. 32 w + 31
    static_assert(TCHUNK % 1024 == 0, "whole DMA instructions");
#pragma unroll
    for (int q = 0; q < TCHUNK / 1024; ++q) {
      const int off = wave * TCHUNK + q * 1024;  // byte of the tile; rows 0..63 in slot 6
      uint8_t* dst = reinterpret_cast<uint8_t*>(off >= 64 * TROWB ? ring[7] : ring[6]) + (off % (64 * TROWB));
      // lane: LDS chunk position p of tile row r gets the row's chunk p ^ t_chunk_sw(r)
      const int slot = off / 16 + lane, r = slot / TCH, pc = slot % TCH;
      const int src = r * TROWB + 16 * (pc ^ t_chunk_sw<RP>(r));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(t_rsrc, (lds_ptr_t)dst, 16, src, 0, 0, 0);
    }
  }
#pragma unroll
  for (int s = 0; s < MX_NS - 2; ++s) dma(s, ring[s]);
  wait_vmcnt<3 * (MX_NS - 3)>();  // the low-rank operands and group 0 have landed
  __builtin_amdgcn_s_barrier();
  if (NTR > 0) {
    if constexpr (T_LDS) t_from_lds();
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
// The GELU table of the current device, filled on first use: on `st`, then waited for, so that calls
// on any stream find it complete. A failed fill (e.g. a first call during stream capture, where
// waiting is not allowed) is retried by the next call.
hipError_t ensure_gelu_table(hipStream_t st) {
  constexpr int MAXD = 64;
  static std::atomic<bool> ready[MAXD];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAXD) return hipErrorInvalidDevice;
  if (ready[dev].load(std::memory_order_acquire)) return hipSuccess;
  try {
    std::lock_guard<std::mutex> lock(mu);
    if (ready[dev].load(std::memory_order_relaxed)) return hipSuccess;
    hipLaunchKernelGGL(gelu_table_kernel, dim3((GELU_TAB + 255) / 256), dim3(256), 0, st);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess) ready[dev].store(true, std::memory_order_release);
    return e;
  } catch (...) {  // std::mutex::lock reports failure by throwing
    return hipErrorUnknown;
  }
}

template <int FMT, int NT, bool GELU_IN = false>
hipError_t launch_qa(const uint16_t* X, int M, int K, int ldx, const float* il, const uint16_t* l1t, int m_pad,
                     uint8_t* xq, void* xs, float* xl1, hipStream_t st) {
  const int gs = qa_group_slice(M, K), nsl = qa_slices(M, K);
  const size_t lds = 16 * (size_t)qa_lds_slots(NT * 16, gs, GELU_IN);
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
  if (ldx < K || ldx % 8 != 0 || ldx > QA_MAX_LDX) return W4A4_ERR_INVALID_ARG;
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
  if (ldy < K || ldy % 8 != 0 || ldy > QA_MAX_LDX) return W4A4_ERR_INVALID_ARG;
  if (!aligned16(Y) || !aligned16(inv_lambda) || !aligned16(xq) || !aligned16(xscale)) return W4A4_ERR_INVALID_ARG;
  if (rank > 0 && (!l1t || !xl1 || !aligned16(l1t) || !aligned16(xl1))) return W4A4_ERR_INVALID_ARG;
  if (ensure_gelu_table(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return W4A4_ERR_HIP;
  const hipError_t e = dispatch_qa<W4A4_FMT_INT4_G64, true>(rank_pad_of(rank) / 16, Y, M, K, ldy, inv_lambda, l1t,
                                                            rows_pad_of(M), xq, xscale, xl1,
                                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

}  // extern "C"

namespace {

// Argument checks shared by the two entry points of the producer-side MLP GEMM.
w4a4_status_t check_gelu_quant_args(const uint8_t* xq, const void* xscale, const float* xl1, const uint8_t* wq,
                                    const void* wscale, const uint16_t* l2t, const uint16_t* bias, int M, int N,
                                    int K, int rank, int fmt, const float* inv_lambda2, const uint16_t* l1t2,
                                    int rank2, uint8_t* xq2, void* xscale2, float* xl1_2, uint16_t* Y, int ldy) {
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
  return W4A4_OK;
}

// The no-allocation entry point's scratch: fc2's per-256-column-tile partial t planes live in this
// fixed array (one copy per GPU, from the loading of this code object until the process ends).
// In host code `scratch` names a host-side stand-in, not device memory: kernels and copies use the
// per-device address taken with hipGetSymbolAddress below, never the name.
constexpr size_t NOALLOC_SCRATCH_FLOATS = size_t(W4A4_NOALLOC_SCRATCH_BYTES) / sizeof(float);
static __device__ __attribute__((aligned(256))) float scratch[NOALLOC_SCRATCH_FLOATS];

constexpr int SCRATCH_MAX_DEVICES = 64;
std::once_flag scratch_once[SCRATCH_MAX_DEVICES];
float* scratch_addr[SCRATCH_MAX_DEVICES];
hipError_t scratch_status[SCRATCH_MAX_DEVICES];

// The current device's address of `scratch`, looked up once per device with that device current.
hipError_t scratch_of_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  try {
    std::call_once(scratch_once[dev], [dev] {
      void* p = nullptr;
      scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      scratch_addr[dev] = static_cast<float*>(p);
    });
  } catch (...) {  // std::call_once reports a failed synchronization by throwing
    return hipErrorUnknown;
  }
  if (scratch_status[dev] != hipSuccess) return scratch_status[dev];
  if (!scratch_addr[dev]) return hipErrorInvalidSymbol;
  *out = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

w4a4_status_t w4a4_lowrank_linear_gelu_quant(const uint8_t* xq, const void* xscale, const float* xl1,
                                             const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                             const uint16_t* bias, int M, int N, int K, int rank, int fmt,
                                             const float* inv_lambda2, const uint16_t* l1t2, int rank2,
                                             uint8_t* xq2, void* xscale2, float* xl1_2, uint16_t* Y, int ldy,
                                             w4a4_stream_t stream) {
  const w4a4_status_t st = check_gelu_quant_args(xq, xscale, xl1, wq, wscale, l2t, bias, M, N, K, rank, fmt,
                                                 inv_lambda2, l1t2, rank2, xq2, xscale2, xl1_2, Y, ldy);
  if (st != W4A4_OK) return st;
  const int m_pad = rows_pad_of(M), n_pad = rows_pad_of(N), rp2 = rank_pad_of(rank2);
  const int tiles_n = n_pad / 256;
  GeluQuantArgs fa{inv_lambda2, l1t2, xq2, static_cast<uint16_t*>(xscale2),
                   rank2 > 0 ? (tiles_n > 1 ? xl1_2 + (size_t)m_pad * rp2 : xl1_2) : nullptr};
  if (ensure_gelu_table(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return W4A4_ERR_HIP;
  const hipError_t e = dispatch_gemm_gelu_quant(rank_pad_of(rank) / 16, rp2 / 16, xq, xscale, xl1, wq, wscale, l2t,
                                                bias, Y, ldy, M, N, K, m_pad, n_pad, fa, xl1_2,
                                                reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4A4_OK : W4A4_ERR_HIP;
}

w4a4_status_t w4a4_lowrank_linear_gelu_quant_noalloc(const uint8_t* xq, const void* xscale, const float* xl1,
                                                     const uint8_t* wq, const void* wscale, const uint16_t* l2t,
                                                     const uint16_t* bias, int M, int N, int K, int rank, int fmt,
                                                     const float* inv_lambda2, const uint16_t* l1t2, int rank2,
                                                     uint8_t* xq2, void* xscale2, float* t2, uint16_t* Y, int ldy,
                                                     w4a4_stream_t stream) {
  const w4a4_status_t st = check_gelu_quant_args(xq, xscale, xl1, wq, wscale, l2t, bias, M, N, K, rank, fmt,
                                                 inv_lambda2, l1t2, rank2, xq2, xscale2, t2, Y, ldy);
  if (st != W4A4_OK) return st;
  const int m_pad = rows_pad_of(M), n_pad = rows_pad_of(N), rp2 = rank_pad_of(rank2);
  const int tiles_n = n_pad / 256;
  const bool planes = rank2 > 0 && tiles_n > 1;  // one tile writes t2 itself, no plane needed
  if (planes && size_t(tiles_n) * size_t(m_pad) * size_t(rp2) > NOALLOC_SCRATCH_FLOATS) return W4A4_ERR_TOO_LARGE;
  float* part = nullptr;
  if (planes && scratch_of_current_device(&part) != hipSuccess) return W4A4_ERR_HIP;
  GeluQuantArgs fa{inv_lambda2, l1t2, xq2, static_cast<uint16_t*>(xscale2),
                   rank2 > 0 ? (planes ? part : t2) : nullptr};
  if (ensure_gelu_table(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return W4A4_ERR_HIP;
  const hipError_t e = dispatch_gemm_gelu_quant(rank_pad_of(rank) / 16, rp2 / 16, xq, xscale, xl1, wq, wscale, l2t,
                                                bias, Y, ldy, M, N, K, m_pad, n_pad, fa, t2,
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
