// Internal helpers shared by the host (w4a4_host.cpp) and device (w4a4_device.hip) halves of
// libw4a4. Not part of the public ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include "w4a4.h"

namespace w4a4 {

inline int round_up(int x, int a) { return (x + a - 1) / a * a; }
inline int rank_pad_of(int rank) { return round_up(rank, W4A4_RANK_ALIGN); }
inline int rows_pad_of(int rows) { return round_up(rows, W4A4_ROW_ALIGN); }

inline bool fmt_known(int fmt) { return fmt == W4A4_FMT_INT4_G64 || fmt == W4A4_FMT_MXFP4_B32; }

// Shared shape checks: M, N >= 1; K a positive multiple of 64; 0 <= rank <= min(N, K, MAX).
inline w4a4_status_t check_shape(int M, int N, int K, int rank, int fmt) {
  if (!fmt_known(fmt)) return W4A4_ERR_UNSUPPORTED;
  if (M < 1 || N < 1 || K < W4A4_GROUP || K % W4A4_GROUP != 0) return W4A4_ERR_INVALID_ARG;
  if (rank < 0 || rank > W4A4_MAX_RANK || rank > N || rank > K) return W4A4_ERR_INVALID_ARG;
  // sizes must stay addressable with 32-bit element offsets inside the kernels
  if ((long long)rows_pad_of(M) * K > (1LL << 31) || (long long)rows_pad_of(N) * K > (1LL << 31))
    return W4A4_ERR_INVALID_ARG;
  return W4A4_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace w4a4
