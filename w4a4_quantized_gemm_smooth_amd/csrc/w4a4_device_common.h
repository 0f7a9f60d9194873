// Device-side helpers shared by the two kernel translation units of libw4a4:
//   w4a4_device.hip       the activation kernels and the 4-bit GEMMs (INT4, MXFP4), and the C ABI
//   w4a4_device_w8a8.hip  the W8A8 kernels (8-bit setting, App. D of the SVDQuant page)
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "w4a4_internal.h"

namespace w4a4 {
namespace dev {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef int v6i __attribute__((ext_vector_type(6)));

__device__ __forceinline__ float bf16f(uint32_t h16) { return __uint_as_float(h16 << 16); }

// float -> bf16 bits, nearest-even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ v8bf as_bf16x8(v4i v) { return __builtin_bit_cast(v8bf, v); }

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left alone), visible to the compiler's wait tracking
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}


__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {  // v_cvt_pk_bf16_f32, nearest-even
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), bf2));
}

// Block tiling shared by the GEMMs: 256 x 256 output tiles; a ring of I4_NS K-step slots in LDS;
// each wave owns I4_MT 32-row tiles of its block rows.
constexpr int I4_BM = 256, I4_BN = 256;
constexpr int I4_MT = 4;            // 32-row tiles per wave (M)
constexpr int I4_GROUP_M = 4;
constexpr int I4_NS = 8;            // ring slots (K steps); even

// LDS swizzle of 32-byte code rows: row r, 16-byte half h (rows 8..15 of every 16 swap halves, so
// the 16-byte reads of 8 consecutive lanes cover all 64 banks)
__device__ __forceinline__ int sw_off32(int r, int h) { return r * 32 + 16 * (h ^ ((r >> 3) & 1)); }

// Chunk swizzle of a t row staged in LDS (rows of RP fp32, 16-byte chunks): row r keeps its chunk c
// at position c ^ t_chunk_sw(r), so that 16-byte reads of one chunk of 32 consecutive rows hit
// distinct banks (2 ways, the minimum for 64 lanes) where rows two (RP 32) or four (RP 16, 48) apart
// would otherwise share them. The XOR stays inside the row (8 chunks, or an aligned group of 4).
// Compute it into a local before passing it to a builtin: as a call inside the argument list of
// the LDS-DMA builtin in a kernel template, the host pass drops the kernel's launch stubs.
template <int RP>
__device__ __forceinline__ int t_chunk_sw(int r) { return RP == 32 ? (r >> 1) & 7 : (r >> 2) & 3; }

// Tile order. Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8),
// so consecutive logical tiles are handed to the same XCD; logical tiles then sweep N in groups of
// I4_GROUP_M M-tiles, so the blocks an XCD runs together share A and B slices in its L2.
__device__ __forceinline__ void tile_of(int b, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = b & 7, idx = b >> 3, q = nblocks >> 3, rem = nblocks & 7;
  const int logical = xcd * q + min(xcd, rem) + idx;
  const int per_group = I4_GROUP_M * tiles_n;
  const int first_m = (logical / per_group) * I4_GROUP_M;
  const int gsize = min(tiles_m - first_m, I4_GROUP_M);
  const int in_group = logical % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Y store shared by the GEMMs: the wave's (32 MT) x 64 block of fp32 results (+ bias) -> bf16 Y
// through LDS, so that every lane writes whole 16-byte row segments. The block goes out in pieces
// of 64 rows, staged in `stage` (an idle ring slot of the wave, 9 KB) with a 144-byte row stride
// (conflict-free 2-byte writes and 16-byte reads). The 32x32 MFMA output layout: lane holds column
// lane%32 and rows 8*(v/4) + 4*(lane/32) + v%4. r0, c0: first row and column of the wave's block.
constexpr int Y_ES = 144;
template <int MT>
__device__ __forceinline__ void store_y(v16f (&acc)[MT][2], uint8_t* stage, const uint16_t* bias, uint16_t* Y,
                                        int ldy, int M, int N, int r0, int c0, int lane) {
  static_assert(MT % 2 == 0, "pieces of 64 rows");
  const int lr = lane & 31, lh = lane >> 5;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(Y) & 15u) == 0) && (ldy % 8 == 0);
  float bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = c0 + j * 32 + lr;
    bcol[j] = (bias && col < N) ? bf16f(bias[col]) : 0.f;
  }
#pragma unroll
  for (int half = 0; half < MT / 2; ++half) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const int rl = ii * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
          const uint32_t pr = pack_bf16x2(acc[2 * half + ii][j][v] + bcol[j], acc[2 * half + ii][j][v + 1] + bcol[j]);
          uint16_t* d = reinterpret_cast<uint16_t*>(stage + rl * Y_ES + (j * 32 + lr) * 2);
          d[0] = (uint16_t)pr;
          d[Y_ES / 2] = (uint16_t)(pr >> 16);
        }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int idx = q * 64 + lane, rr = idx >> 3, c = idx & 7;
      const uint4 val = *reinterpret_cast<const uint4*>(stage + rr * Y_ES + c * 16);
      const int row = r0 + half * 64 + rr, col = c0 + c * 8;
      if (row >= M) continue;
      uint16_t* dst = Y + (size_t)row * ldy + col;
      if (vec_ok && col + 8 <= N) {
        *reinterpret_cast<uint4*>(dst) = val;
      } else {
        const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (col + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

}  // namespace dev

// Launchers of the W8A8 translation unit (asynchronous on `st`; they return the launch status).
// Per-token INT8 codes and scales from the partial row maxima the activation kernel left behind
// the scales (nsl planes); with rank_pad > 0 and nsl > 1 it also sums the partial t planes.
hipError_t launch_quantize_w8(const uint16_t* X, int M, int K, int ldx, const float* inv_lambda, int m_pad, int nsl,
                              uint8_t* xq, float* xscale, float* xl1, int rank_pad, hipStream_t st);
// The W8A8 GEMM with the low-rank up projection and bias in its epilogue; ntr = rank_pad / 16.
hipError_t dispatch_gemm_w8a8(int ntr, const uint8_t* xq, const float* xscale, const float* xl1, const uint8_t* wq,
                              const float* wscale, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy,
                              int M, int N, int K, int m_pad, int n_pad, hipStream_t st);
// The MXFP4 GEMM on the INT8 kernel's structure (E8M0 block scales applied by the scaled MFMA)
hipError_t dispatch_gemm_mx(int ntr, const uint8_t* xq, const uint8_t* xscale, const float* xl1, const uint8_t* wq,
                            const uint8_t* wscale, const uint16_t* l2t, const uint16_t* bias, uint16_t* Y, int ldy,
                            int M, int N, int K, int m_pad, int n_pad, hipStream_t st);

}  // namespace w4a4
