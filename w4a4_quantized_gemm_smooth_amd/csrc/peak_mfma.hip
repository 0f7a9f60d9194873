// Measured MFMA peak of gfx950 for the roofline (a measurement helper for the benchmark, not part
// of the layer's ABI): every wave runs independent chains of one MFMA instruction back to back on
// register operands, with no memory traffic, so the time per instruction is the matrix pipe's own.
// Built into libw4a4_peak.so.
//
//   kind 0: v_mfma_i32_32x32x32_i8                     (int8,  32768 MACs)
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4, FP6 E2M3 (65536 MACs; the INT4 carrier of the GEMM)
//   kind 2: v_mfma_scale_f32_32x32x64_f8f6f4, FP4 E2M1 (65536 MACs)
//   kind 3: v_mfma_f32_32x32x16_bf16                   (bf16,  16384 MACs)

#include <hip/hip_runtime.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int CHAINS = 8;

template <int KIND>
__global__ __launch_bounds__(256) void peak_kernel(int iters, float* __restrict__ out) {
  const int t = threadIdx.x;
  // operands derived from the thread index, so nothing folds at compile time; small values keep
  // every sum finite
  const v4i a4 = v4i{t & 3, (t >> 2) & 3, 1, 2};
  const v8i a8 = v8i{t & 7, 1, 2, 3, 4, 5, 0, 0};
  v16i iacc[CHAINS];
  v16f facc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) {
    iacc[c] = v16i{};
    facc[c] = v16f{};
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) {
      if constexpr (KIND == 0)
        iacc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a4, a4, iacc[c], 0, 0, 0);
      else if constexpr (KIND == 1)
        facc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, facc[c], 2, 2, 0, 127, 0, 127);
      else if constexpr (KIND == 2)
        facc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, a8, facc[c], 4, 4, 0, 127, 0, 127);
      else
        facc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a4), __builtin_bit_cast(v8bf, a4),
                                                          facc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if constexpr (KIND == 0)
        s += (float)iacc[c][v];
      else
        s += facc[c][v];
    }
  out[blockIdx.x * 256 + t] = s;
}

}  // namespace

extern "C" {

// MACs of one instruction of `kind`, or 0 for an unknown kind
long long w4a4_peak_mfma_macs(int kind) {
  return kind == 0 ? 32768 : kind == 1 || kind == 2 ? 65536 : kind == 3 ? 16384 : 0;
}

// Launches `blocks` blocks of 256 threads, each wave running iters x 8 instructions of `kind`;
// out holds blocks * 256 floats. Returns 0, or -1 for a bad argument, or the HIP error code.
int w4a4_peak_mfma_launch(int kind, int blocks, int iters, float* out, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1 || w4a4_peak_mfma_macs(kind) == 0) return -1;
  switch (kind) {
    case 0: hipLaunchKernelGGL(peak_kernel<0>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
    case 1: hipLaunchKernelGGL(peak_kernel<1>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
    case 2: hipLaunchKernelGGL(peak_kernel<2>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
    default: hipLaunchKernelGGL(peak_kernel<3>, dim3(blocks), dim3(256), 0, stream, iters, out); break;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
