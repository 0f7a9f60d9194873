// Internal helpers shared by the host (w4a4_host.cpp) and device (w4a4_device.hip) halves of
// libw4a4. Not part of the public ABI.
#pragma once

#include <climits>
#include <cstddef>
#include <cstdint>

#include "w4a4.h"

namespace w4a4 {

inline int round_up(int x, int a) { return (x + a - 1) / a * a; }
inline int rank_pad_of(int rank) { return round_up(rank, W4A4_RANK_ALIGN); }
inline int rows_pad_of(int rows) { return round_up(rows, W4A4_ROW_ALIGN); }

inline bool fmt_known(int fmt) {
  return fmt == W4A4_FMT_INT4_G64 || fmt == W4A4_FMT_MXFP4_B32 || fmt == W4A4_FMT_W8A8;
}

// Shared shape checks: M, N >= 1; K a positive multiple of 64; 0 <= rank <= min(N, K, MAX).
inline w4a4_status_t check_shape(int M, int N, int K, int rank, int fmt) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < W4A4_GROUP || K % W4A4_GROUP != 0) return W4A4_ERR_INVALID_ARG;
  // rows are padded to a multiple of W4A4_ROW_ALIGN in int arithmetic: keep that from overflowing
  if (M > INT_MAX - W4A4_ROW_ALIGN || N > INT_MAX - W4A4_ROW_ALIGN) return W4A4_ERR_INVALID_ARG;
  if (rank < 0 || rank > W4A4_MAX_RANK || rank > N || rank > K) return W4A4_ERR_INVALID_ARG;
  // W8A8: the int32 dot product of 127-bounded codes must not overflow, and the one-byte codes
  // (rows_pad * K bytes per operand) must stay below 2^31 bytes
  if (fmt == W4A4_FMT_W8A8 && (K > W4A4_W8A8_MAX_K || (long long)rows_pad_of(M) * K >= (1LL << 31) ||
                               (long long)rows_pad_of(N) * K >= (1LL << 31)))
    return W4A4_ERR_INVALID_ARG;
  // sizes must stay addressable with 32-bit element offsets inside the kernels
  if ((long long)rows_pad_of(M) * K > (1LL << 31) || (long long)rows_pad_of(N) * K > (1LL << 31))
    return W4A4_ERR_INVALID_ARG;
  // t (fp32) and L2^T (bf16) are addressed with 32-bit byte offsets too
  if ((long long)rows_pad_of(M) * rank_pad_of(rank) * 4 >= (1LL << 31)) return W4A4_ERR_INVALID_ARG;
  return W4A4_OK;
}

// Activation kernel blocking: 64 rows x a slice of at most QA_MAX_GS groups per block, so the
// slice's L1 rows are fetched once per 64 rows. With several slices each block writes the partial t
// of its slice to a scratch plane behind t, and a second kernel sums the planes in slice order
// (deterministic). A reduction inside the kernel (the last block of a row block to finish sums the
// planes) needs every block to wait for its partial to be written through to the device-coherent
// level before it counts itself, which costs more than the second launch.
#ifndef W4A4_QA_BLOCK_ROWS  // build-time tuning knobs (rows per block: a multiple of 16, at most 256)
#define W4A4_QA_BLOCK_ROWS 64
#endif
#ifndef W4A4_QA_MAX_GS
#define W4A4_QA_MAX_GS 8
#endif
#ifndef W4A4_QA_TARGET_BLOCKS
#define W4A4_QA_TARGET_BLOCKS 256
#endif
constexpr int QA_BLOCK_ROWS = W4A4_QA_BLOCK_ROWS, QA_MAX_GS = W4A4_QA_MAX_GS;
constexpr int QA_TARGET_BLOCKS = W4A4_QA_TARGET_BLOCKS;  // slices are added until the grid has this many blocks
static_assert(QA_BLOCK_ROWS % 16 == 0 && QA_BLOCK_ROWS <= 256 && QA_MAX_GS % 2 == 0, "activation blocking");
inline int qa_group_slice(int M, int K) {  // groups per slice
  const int rb = rows_pad_of(M) / QA_BLOCK_ROWS, G = K / W4A4_GROUP;
  int ks = (QA_TARGET_BLOCKS + rb - 1) / rb;
  if (ks < (G + QA_MAX_GS - 1) / QA_MAX_GS) ks = (G + QA_MAX_GS - 1) / QA_MAX_GS;
  if (ks > G) ks = G;
  return (G + ks - 1) / ks;
}
inline int qa_slices(int M, int K) {
  const int gs = qa_group_slice(M, K), G = K / W4A4_GROUP;
  return (G + gs - 1) / gs;
}
// floats of the xl1 buffer: t [m_pad][rank_pad], then [slices][m_pad][rank_pad] partial planes
// when there is more than one slice
inline size_t xl1_floats(int M, int K, int rank) {
  const size_t t = size_t(rows_pad_of(M)) * size_t(rank_pad_of(rank));
  const int ks = qa_slices(M, K);
  return rank == 0 ? 0 : (ks > 1 ? t * size_t(1 + ks) : t);
}

// floats of a W8A8 xscale buffer: the [m_pad] per-token scales, then one [m_pad] plane of partial
// row maxima per slice (written by the first activation kernel, reduced by the second)
inline size_t w8_xscale_floats(int M, int K) { return size_t(rows_pad_of(M)) * size_t(1 + qa_slices(M, K)); }

// Largest activation row stride (elements) the activation kernel addresses: 16 rows of it must
// stay below 2^31 bytes (32-bit buffer offsets).
constexpr int QA_MAX_LDX = 1 << 26;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace w4a4
